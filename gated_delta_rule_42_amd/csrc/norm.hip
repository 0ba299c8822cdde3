// norm.hip -- gated RMSNorm on [tokens, heads, dim] rows, norm before gate.
//
// Page "[Feature][KDA] Add Kimi K3 KDA execution", What this PR does: the KDA
// output goes through a fused normalisation-and-gating step whose result is
// allocated separately so the input is preserved; the gate may be a packed
// (strided) tensor.
//
//     y = x * rsqrt(mean(x^2) + eps) * w * silu(gate)
//
// HBM-bound (reads x and gate once, writes y once).  LPR lanes share one row:
// each lane owns dim/LPR elements in 8-element vectors (16 B for bf16), the
// sum of squares is reduced across the LPR lanes with shuffles in a fixed
// order, so results are deterministic.

#include "kda_device.cuh"
#include "kda_internal.h"

namespace kda {
namespace {

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
__device__ __forceinline__ void store8(float* p, const float (&x)[8])
{
    *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(x[4], x[5], x[6], x[7]);
}
__device__ __forceinline__ void store8(bf16* p, const float (&x)[8])
{
    bf16x8 t;
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = static_cast<bf16>(x[i]);
    *reinterpret_cast<bf16x8*>(p) = t;
}

constexpr int kNormBlock = 256;

template <int LPR, typename T>
__global__ __launch_bounds__(kNormBlock)
void gated_rmsnorm_kernel(const T* __restrict__ x, int64_t xs, const T* __restrict__ gate,
                          int64_t gs, const T* __restrict__ w, T* __restrict__ y, int64_t ys,
                          int64_t rows, int heads, int dim, float eps)
{
    constexpr int kRowsPerBlock = kNormBlock / LPR;
    const int lane_in_row = threadIdx.x % LPR;
    const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / LPR;
    const bool live = row < rows;
    const int64_t t = live ? row / heads : 0;
    const int h = live ? (int)(row % heads) : 0;
    const T* xr = x + t * xs + (int64_t)h * dim;
    const T* gr = gate + t * gs + (int64_t)h * dim;
    T* yr = y + t * ys + (int64_t)h * dim;

    // Sum of squares over the row (each lane: its 8-element vectors).
    float ss = 0.0f;
    if (live) {
        for (int c = lane_in_row * 8; c < dim; c += LPR * 8) {
            float xv[8];
            load8(xr + c, xv);
#pragma unroll
            for (int i = 0; i < 8; ++i) ss += xv[i] * xv[i];
        }
    }
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) ss += __shfl_xor(ss, off, LPR);
    if (!live) return;
    const float inv = 1.0f / sqrtf(ss / (float)dim + eps);

    for (int c = lane_in_row * 8; c < dim; c += LPR * 8) {
        float xv[8], gv[8], wv[8], out[8];
        load8(xr + c, xv);
        load8(gr + c, gv);
        if (w) {
            load8(w + c, wv);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) wv[i] = 1.0f;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float z = gv[i];
            const float silu = z / (1.0f + __expf(-z));
            out[i] = xv[i] * inv * wv[i] * silu;
        }
        store8(yr + c, out);
    }
}

template <int LPR, typename T>
hipError_t launch_lpr(const RmsNormArgs& a, hipStream_t stream)
{
    const int64_t rows = a.tokens * a.heads;
    constexpr int kRowsPerBlock = kNormBlock / LPR;
    const int64_t blocks = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
    if (blocks > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gated_rmsnorm_kernel<LPR, T>), dim3((unsigned)blocks), dim3(kNormBlock),
                       0, stream, static_cast<const T*>(a.x), a.x_stride,
                       static_cast<const T*>(a.gate), a.gate_stride,
                       static_cast<const T*>(a.weight), static_cast<T*>(a.y), a.y_stride, rows,
                       a.heads, a.dim, a.eps);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_typed(const RmsNormArgs& a, hipStream_t stream)
{
    // Largest power-of-two lane count (<= 64) that splits the row into whole
    // 8-element vectors per lane.
    const int vecs = a.dim / 8;
    int lpr = 64;
    while (lpr > 1 && vecs % lpr != 0) lpr >>= 1;
    switch (lpr) {
        case 64: return launch_lpr<64, T>(a, stream);
        case 32: return launch_lpr<32, T>(a, stream);
        case 16: return launch_lpr<16, T>(a, stream);
        case 8: return launch_lpr<8, T>(a, stream);
        case 4: return launch_lpr<4, T>(a, stream);
        case 2: return launch_lpr<2, T>(a, stream);
        default: return launch_lpr<1, T>(a, stream);
    }
}

}  // namespace

hipError_t launch_gated_rmsnorm(const RmsNormArgs& a, hipStream_t stream)
{
    return a.dtype == KDA_BF16 ? launch_typed<bf16>(a, stream) : launch_typed<float>(a, stream);
}

}  // namespace kda
