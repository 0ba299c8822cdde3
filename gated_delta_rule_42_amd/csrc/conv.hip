// conv.hip -- causal depthwise conv1d over a varlen batch with a rolling
// per-slot conv state.
//
// Page "[Feature][KDA] Add Kimi K3 KDA execution", KDA execution step 2 (run
// the causal convolution and update its cache) and What this PR does
// (causal-convolution state packing).
//
//     y_t[c] = act( bias[c] + sum_{j<W} w[c, j] * x_{t-W+1+j}[c] )
//
// with inputs before a sequence's first token taken from its conv state
// (row W-2 = most recent), zeros without an initial state.
//
// Two kernels, both HBM-bound:
//   conv_kernel   each thread owns 8 channels (one 16 B bf16 vector) of a
//                 tile of TB consecutive tokens and slides the W-tap window
//                 along it in registers; x is read once (plus W-1 halo rows
//                 per tile), y written once.
//   state_kernel  writes each sequence's new state (its last W-1 inputs).  It
//                 runs after conv_kernel on the same stream because
//                 conv_kernel reads the old state; each thread reads all the
//                 old rows it needs before writing, so no thread overwrites a
//                 row another still reads.

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kConvBlock = 256;   // channel groups per block
constexpr int kConvTile = 16;     // tokens per thread
constexpr int kMaxWidth = 8;

__device__ __forceinline__ void ld8(const float* p, float (&x)[8])
{
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
__device__ __forceinline__ void ld8(const bf16* p, float (&x)[8])
{
    const bf16x8 t = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = static_cast<float>(t[i]);
}
__device__ __forceinline__ void st8(float* p, const float (&x)[8])
{
    *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(x[4], x[5], x[6], x[7]);
}
__device__ __forceinline__ void st8(bf16* p, const float (&x)[8])
{
    bf16x8 t;
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = static_cast<bf16>(x[i]);
    *reinterpret_cast<bf16x8*>(p) = t;
}

// Sequence containing token t: largest i with cu[i] <= t (binary search).
__device__ __forceinline__ int find_seq(const int32_t* cu, int n, int64_t t)
{
    int lo = 0, hi = n;            // invariant: cu[lo] <= t < cu[hi] when t < cu[n]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if ((int64_t)cu[mid] <= t) lo = mid; else hi = mid;
    }
    return lo;
}

template <int W, typename T>
__global__ __launch_bounds__(kConvBlock)
void conv_kernel(const T* __restrict__ x, int64_t xs, const T* __restrict__ w,
                 const T* __restrict__ bias, const T* __restrict__ state, int64_t num_slots,
                 const int32_t* __restrict__ cu, const int32_t* __restrict__ slots,
                 const uint8_t* __restrict__ has_init, int n_seqs, int channels, bool silu,
                 T* __restrict__ y, int64_t ys)
{
    const int cg = blockIdx.y * kConvBlock + threadIdx.x;
    const int c0 = cg * 8;
    if (c0 >= channels) return;
    const int64_t end = cu[n_seqs];
    const int64_t t_begin = (int64_t)blockIdx.x * kConvTile;
    if (t_begin >= end) return;
    const int64_t t_end = t_begin + kConvTile < end ? t_begin + kConvTile : end;

    float wt[W][8], bs[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int j = 0; j < W; ++j) wt[j][i] = to_f32(w[(int64_t)(c0 + i) * W + j]);
        bs[i] = bias ? to_f32(bias[c0 + i]) : 0.0f;
    }

    int seq = find_seq(cu, n_seqs, t_begin);
    float hist[W - 1][8];          // hist[W-2] = most recent input
    int64_t t = t_begin;
    while (t < t_end) {
        while (seq < n_seqs - 1 && (int64_t)cu[seq + 1] <= t) ++seq;   // skip empty sequences
        const int64_t s0 = cu[seq], s1 = cu[seq + 1];
        const int64_t stop = s1 < t_end ? s1 : t_end;
        const int slot = slots[seq];
        if (slot < 0 || slot >= num_slots) {          // padding (or bad slot): zero rows
            float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            if (slot < 0)
                for (; t < stop; ++t) st8(y + t * ys + c0, z);
            t = stop;
            continue;
        }
        const bool init = has_init ? has_init[seq] != 0 : true;
        const T* st = state + (int64_t)slot * (W - 1) * channels + c0;
        // Window before token t: positions t-W+1 .. t-1.
#pragma unroll
        for (int j = 0; j < W - 1; ++j) {
            const int64_t p = t - (W - 1) + j;
            if (p >= s0) {
                ld8(x + p * xs + c0, hist[j]);
            } else if (init) {
                ld8(st + (int64_t)((W - 1) - (s0 - p)) * channels, hist[j]);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) hist[j][i] = 0.0f;
            }
        }
        for (; t < stop; ++t) {
            float cur[8], out[8];
            ld8(x + t * xs + c0, cur);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float acc = bs[i];
#pragma unroll
                for (int j = 0; j < W - 1; ++j) acc += wt[j][i] * hist[j][i];
                acc += wt[W - 1][i] * cur[i];
                out[i] = silu ? silu_f32(acc) : acc;
            }
            st8(y + t * ys + c0, out);
#pragma unroll
            for (int j = 0; j < W - 2; ++j) {
#pragma unroll
                for (int i = 0; i < 8; ++i) hist[j][i] = hist[j + 1][i];
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) hist[W - 2][i] = cur[i];
        }
    }
}

template <int W, typename T>
__global__ __launch_bounds__(kConvBlock)
void state_kernel(const T* __restrict__ x, int64_t xs, T* __restrict__ state, int64_t num_slots,
                  const int32_t* __restrict__ cu, const int32_t* __restrict__ slots,
                  const uint8_t* __restrict__ has_init, int channels)
{
    const int seq = blockIdx.x;
    const int c0 = (blockIdx.y * kConvBlock + threadIdx.x) * 8;
    if (c0 >= channels) return;
    const int slot = slots[seq];
    const int64_t s0 = cu[seq], s1 = cu[seq + 1];
    if (slot < 0 || slot >= num_slots || s1 <= s0) return;
    const bool init = has_init ? has_init[seq] != 0 : true;
    T* st = state + (int64_t)slot * (W - 1) * channels + c0;
    float nw[W - 1][8];
#pragma unroll
    for (int j = 0; j < W - 1; ++j) {
        const int64_t p = s1 - (W - 1) + j;
        if (p >= s0) {
            ld8(x + p * xs + c0, nw[j]);
        } else if (init) {
            ld8(st + (int64_t)((W - 1) - (s0 - p)) * channels, nw[j]);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) nw[j][i] = 0.0f;
        }
    }
#pragma unroll
    for (int j = 0; j < W - 1; ++j) st8(st + (int64_t)j * channels, nw[j]);
}

template <int W, typename T>
hipError_t launch_typed(const ConvArgs& a, hipStream_t stream)
{
    const int groups = a.channels / 8;
    const unsigned gc = (unsigned)((groups + kConvBlock - 1) / kConvBlock);
    const int64_t tiles = (a.total_tokens + kConvTile - 1) / kConvTile;
    if (tiles > 0) {
        if (tiles > INT32_MAX) return hipErrorInvalidValue;
        hipLaunchKernelGGL((conv_kernel<W, T>), dim3((unsigned)tiles, gc), dim3(kConvBlock), 0,
                           stream, static_cast<const T*>(a.x), a.x_stride,
                           static_cast<const T*>(a.weight), static_cast<const T*>(a.bias),
                           static_cast<const T*>(a.state), a.num_slots, a.cu_seqlens, a.slots,
                           a.has_init, a.num_seqs, a.channels, (a.flags & KDA_CONV_SILU) != 0,
                           static_cast<T*>(a.y), a.y_stride);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((state_kernel<W, T>), dim3((unsigned)a.num_seqs, gc), dim3(kConvBlock), 0,
                       stream, static_cast<const T*>(a.x), a.x_stride, static_cast<T*>(a.state),
                       a.num_slots, a.cu_seqlens, a.slots, a.has_init, a.channels);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_width(const ConvArgs& a, hipStream_t stream)
{
    switch (a.width) {
        case 2: return launch_typed<2, T>(a, stream);
        case 3: return launch_typed<3, T>(a, stream);
        case 4: return launch_typed<4, T>(a, stream);
        case 5: return launch_typed<5, T>(a, stream);
        case 6: return launch_typed<6, T>(a, stream);
        case 7: return launch_typed<7, T>(a, stream);
        case 8: return launch_typed<8, T>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_causal_conv1d(const ConvArgs& a, hipStream_t stream)
{
    static_assert(kMaxWidth == 8, "width dispatch");
    return a.dtype == KDA_BF16 ? launch_width<bf16>(a, stream) : launch_width<float>(a, stream);
}

}  // namespace kda
