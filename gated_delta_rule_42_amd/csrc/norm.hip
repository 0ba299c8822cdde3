// norm.hip -- gated RMSNorm on [tokens, heads, dim] rows, norm before gate.
//
// Page "[Feature][KDA] Add Kimi K3 KDA execution", What this PR does: the KDA
// output goes through a fused normalisation-and-gating step whose result is
// allocated separately so the input is preserved; How was this patch tested:
// the norm-gate variants are fp16 and bf16 data, sigmoid and SiLU gates,
// packed (strided) gates, the affine path, and the residual / prenorm path.
//
//     h = x + residual                        (residual optional, fp32 sum)
//     residual_out = h                        (optional: the prenorm output)
//     y = (h * rsqrt(mean(h^2) + eps) * w + b) * act(gate)
//     act(z) = z * sigmoid(z)  (SiLU)  or  sigmoid(z)
//
// HBM-bound (reads x, residual and gate once, writes y and residual_out
// once).  LPR lanes share one row: each lane owns dim/LPR elements in
// 8-element vectors, the sum of squares is reduced across the LPR lanes with
// shuffles in a fixed order, so results are deterministic.  When a lane
// owns one vector, everything is loaded once before the reduction; otherwise
// x (and the residual) are read a second time after it, from the cache.

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ void load8(const float* p, float (&x)[8])
{
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
__device__ __forceinline__ void load8(const bf16* p, float (&x)[8])
{
    const bf16x8 t = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = static_cast<float>(t[i]);
}
__device__ __forceinline__ void load8(const f16* p, float (&x)[8])
{
    const f16x8 t = *reinterpret_cast<const f16x8*>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = static_cast<float>(t[i]);
}
// The outputs (y and the prenorm sum) are written once and not read again
// here: nontemporal stores, which also leave less to write back behind the
// kernel (the next prefill call of a pipeline runs faster after it).
__device__ __forceinline__ void store8(float* p, const float (&x)[8])
{
    __builtin_nontemporal_store(f32x4{x[0], x[1], x[2], x[3]}, reinterpret_cast<f32x4*>(p));
    __builtin_nontemporal_store(f32x4{x[4], x[5], x[6], x[7]}, reinterpret_cast<f32x4*>(p + 4));
}
__device__ __forceinline__ void store8(bf16* p, const float (&x)[8])
{
    bf16x8 t;
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = static_cast<bf16>(x[i]);
    __builtin_nontemporal_store(__builtin_bit_cast(f32x4, t), reinterpret_cast<f32x4*>(p));
}
__device__ __forceinline__ void store8(f16* p, const float (&x)[8])
{
    f16x8 t;
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = static_cast<f16>(x[i]);
    __builtin_nontemporal_store(__builtin_bit_cast(f32x4, t), reinterpret_cast<f32x4*>(p));
}

constexpr int kNormBlock = 256;

// T: x, gate, weight, bias and y; R: residual and residual_out (T or fp32).
// PLAIN: no residual, no residual_out, no bias and the SiLU gate, known at
// compile time (the kernel is bound by its vector instructions about as much
// as by HBM, so the plain norm of the KDA output gets its own copy).
template <int LPR, bool PLAIN, typename T, typename R>
__global__ __launch_bounds__(kNormBlock)
void gated_rmsnorm_kernel(const T* __restrict__ x, int64_t xs, const T* __restrict__ gate,
                          int64_t gs, const R* __restrict__ res, int64_t rs,
                          const T* __restrict__ w, const T* __restrict__ bias,
                          T* __restrict__ y, int64_t ys, R* __restrict__ res_out, int64_t ros,
                          int64_t rows, int heads, int dim, float eps, bool sigmoid)
{
    constexpr int kRowsPerBlock = kNormBlock / LPR;
    const int lane_in_row = threadIdx.x % LPR;
    const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / LPR;
    const bool live = row < rows;
    const int64_t t = live ? row / heads : 0;
    const int64_t off = live ? (int64_t)(row % heads) * dim : 0;
    const T* xr = x + t * xs + off;
    const T* gr = gate + t * gs + off;
    const R* rr = !PLAIN && res ? res + t * rs + off : nullptr;
    R* ror = !PLAIN && res_out ? res_out + t * ros + off : nullptr;
    const T* bb = PLAIN ? nullptr : bias;
    const bool sig = !PLAIN && sigmoid;
    T* yr = y + t * ys + off;

    // h = x (+ residual) for one of this lane's vectors.
    auto row_vec = [&](int c, float (&hv)[8]) {
        load8(xr + c, hv);
        if (rr) {
            float rv[8];
            load8(rr + c, rv);
#pragma unroll
            for (int i = 0; i < 8; ++i) hv[i] += rv[i];
        }
    };

    if (dim == LPR * 8) {
        // One 8-element vector per lane (dim 128 with 16 lanes per row, and
        // every dim whose vector count is a power of two up to 64): the gate,
        // weight and bias loads go out with x, before the reduction, and x is
        // not read twice.  The arithmetic is that of the loop below.
        const int c = lane_in_row * 8;
        float hv[8], gv[8], wv[8], bv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) { hv[i] = 0.0f; gv[i] = 0.0f; wv[i] = 1.0f; bv[i] = 0.0f; }
        float ss = 0.0f;
        if (live) {
            row_vec(c, hv);
            load8(gr + c, gv);
            if (w) load8(w + c, wv);
            if (bb) load8(bb + c, bv);
            if (ror) store8(ror + c, hv);
#pragma unroll
            for (int i = 0; i < 8; ++i) ss = __builtin_fmaf(hv[i], hv[i], ss);
        }
#pragma unroll
        for (int o = LPR / 2; o > 0; o >>= 1) ss += __shfl_xor(ss, o, LPR);
        if (!live) return;
        const float inv = rms_inv(ss, dim, eps);
        float out[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) out[i] = gated_norm_out(hv[i], inv, wv[i], bv[i], gv[i], sig);
        store8(yr + c, out);
        return;
    }

    // Sum of squares of h; the prenorm output is written here.
    float ss = 0.0f;
    if (live) {
        for (int c = lane_in_row * 8; c < dim; c += LPR * 8) {
            float hv[8];
            row_vec(c, hv);
            if (ror) store8(ror + c, hv);
#pragma unroll
            for (int i = 0; i < 8; ++i) ss = __builtin_fmaf(hv[i], hv[i], ss);
        }
    }
#pragma unroll
    for (int o = LPR / 2; o > 0; o >>= 1) ss += __shfl_xor(ss, o, LPR);
    if (!live) return;
    const float inv = rms_inv(ss, dim, eps);

    for (int c = lane_in_row * 8; c < dim; c += LPR * 8) {
        float hv[8], gv[8], wv[8], bv[8], out[8];
        row_vec(c, hv);
        load8(gr + c, gv);
        if (w) {
            load8(w + c, wv);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) wv[i] = 1.0f;
        }
        if (bb) {
            load8(bb + c, bv);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) bv[i] = 0.0f;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) out[i] = gated_norm_out(hv[i], inv, wv[i], bv[i], gv[i], sig);
        store8(yr + c, out);
    }
}

template <int LPR, bool PLAIN, typename T, typename R>
hipError_t launch_lpr(const RmsNormArgs& a, hipStream_t stream)
{
    const int64_t rows = a.tokens * a.heads;
    constexpr int kRowsPerBlock = kNormBlock / LPR;
    const int64_t blocks = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
    if (blocks > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gated_rmsnorm_kernel<LPR, PLAIN, T, R>), dim3((unsigned)blocks),
                       dim3(kNormBlock), 0, stream, static_cast<const T*>(a.x), a.x_stride,
                       static_cast<const T*>(a.gate), a.gate_stride,
                       static_cast<const R*>(a.residual), a.residual_stride,
                       static_cast<const T*>(a.weight), static_cast<const T*>(a.bias),
                       static_cast<T*>(a.y), a.y_stride, static_cast<R*>(a.residual_out),
                       a.residual_out_stride, rows, a.heads, a.dim, a.eps, a.sigmoid);
    return hipGetLastError();
}

template <bool PLAIN, typename T, typename R>
hipError_t launch_typed(const RmsNormArgs& a, hipStream_t stream)
{
    // Largest power-of-two lane count (<= 64) that splits the row into whole
    // 8-element vectors per lane.
    const int vecs = a.dim / 8;
    int lpr = 64;
    while (lpr > 1 && vecs % lpr != 0) lpr >>= 1;
    switch (lpr) {
        case 64: return launch_lpr<64, PLAIN, T, R>(a, stream);
        case 32: return launch_lpr<32, PLAIN, T, R>(a, stream);
        case 16: return launch_lpr<16, PLAIN, T, R>(a, stream);
        case 8: return launch_lpr<8, PLAIN, T, R>(a, stream);
        case 4: return launch_lpr<4, PLAIN, T, R>(a, stream);
        case 2: return launch_lpr<2, PLAIN, T, R>(a, stream);
        default: return launch_lpr<1, PLAIN, T, R>(a, stream);
    }
}

template <typename T>
hipError_t launch_variant(const RmsNormArgs& a, hipStream_t stream)
{
    if (!a.residual && !a.residual_out && !a.bias && !a.sigmoid)
        return launch_typed<true, T, T>(a, stream);
    if (a.residual_f32) return launch_typed<false, T, float>(a, stream);
    return launch_typed<false, T, T>(a, stream);
}

}  // namespace

hipError_t launch_gated_rmsnorm(const RmsNormArgs& a, hipStream_t stream)
{
    switch (a.dtype) {
        case KDA_BF16: return launch_variant<bf16>(a, stream);
        case KDA_F16: return launch_variant<f16>(a, stream);
        default: return launch_variant<float>(a, stream);
    }
}

}  // namespace kda
