// kda_device.h -- device helpers shared by the KDA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Scalar conversions.  bf16 -> fp32 is exact; fp32 -> bf16 rounds to nearest
// even (the language's conversion; gfx950 has a native instruction for it).
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return static_cast<float>(x); }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return static_cast<bf16>(x); }

// ---------------------------------------------------------------------------
// Vector I/O of 4 consecutive elements (16 B for fp32, 8 B for bf16).  The
// address must be aligned to the vector size.
__device__ __forceinline__ void load4(const float* p, float (&x)[4])
{
    const float4 t = *reinterpret_cast<const float4*>(p);
    x[0] = t.x; x[1] = t.y; x[2] = t.z; x[3] = t.w;
}
__device__ __forceinline__ void load4(const bf16* p, float (&x)[4])
{
    const bf16x4 t = *reinterpret_cast<const bf16x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = static_cast<float>(t[i]);
}
__device__ __forceinline__ void store4(float* p, const float (&x)[4])
{
    *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ void store4(bf16* p, const float (&x)[4])
{
    bf16x4 t;
#pragma unroll
    for (int i = 0; i < 4; ++i) t[i] = static_cast<bf16>(x[i]);
    *reinterpret_cast<bf16x4*>(p) = t;
}

// Streaming variants for data read once and written once (the recurrent
// states of decode): nontemporal accesses keep the stream from being retained
// in the caches, which raises the achieved HBM bandwidth of a read-modify-write
// pass (measured on MI355X: 6.1 vs 5.4 TB/s for a 1 GiB in-place update).
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void load4_stream(const float* p, float (&x)[4])
{
    const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    x[0] = t[0]; x[1] = t[1]; x[2] = t[2]; x[3] = t[3];
}
__device__ __forceinline__ void load4_stream(const bf16* p, float (&x)[4])
{
    const u32x2 t = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    const bf16x4 b = __builtin_bit_cast(bf16x4, t);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = static_cast<float>(b[i]);
}
__device__ __forceinline__ void store4_stream(float* p, const float (&x)[4])
{
    const f32x4 t = {x[0], x[1], x[2], x[3]};
    __builtin_nontemporal_store(t, reinterpret_cast<f32x4*>(p));
}
__device__ __forceinline__ void store4_stream(bf16* p, const float (&x)[4])
{
    bf16x4 b;
#pragma unroll
    for (int i = 0; i < 4; ++i) b[i] = static_cast<bf16>(x[i]);
    __builtin_nontemporal_store(__builtin_bit_cast(u32x2, b), reinterpret_cast<u32x2*>(p));
}

// ---------------------------------------------------------------------------
// Wave reductions (64 lanes).
__device__ __forceinline__ float wave_sum(float x)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, kWave);
    return x;
}

__device__ __forceinline__ int wave_inclusive_scan(int x, int lane)
{
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        int y = __shfl_up(x, off, kWave);
        if (lane >= off) x += y;
    }
    return x;
}

// ---------------------------------------------------------------------------
// Workgroup barrier that orders LDS traffic only: waits for this wave's LDS
// operations, then synchronises the waves.  Unlike __syncthreads() it does not
// wait for outstanding global loads (including asynchronous loads into LDS
// buffers that the barrier does not protect), so prefetches stay in flight.
// The memory clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wait until at most N vector-memory operations issued by this wave are
// outstanding (they complete in issue order).  gfx9 encoding of s_waitcnt:
// vmcnt in bits [3:0] and [15:14]; expcnt [6:4] and lgkmcnt [11:8] left at
// their maxima (no wait).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// ---------------------------------------------------------------------------
// MFMA wrappers.
//
// v_mfma_f32_16x16x32_bf16: D[16x16] += A[16x32] * B[32x16].
//   A: lane l supplies row (l % 16), 8 K-elements of lane group (l / 16).
//   B: lane l supplies column (l % 16), the same 8 K-elements.
//   C/D: lane l holds column (l % 16), rows 4*(l/16) .. 4*(l/16)+3.
// A and B name their K-elements the same way, so any consistent relabelling
// of K (used to feed accumulators straight back in as B operands) leaves the
// product unchanged.
__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// v_mfma_f32_16x16x4_f32: D[16x16] += A[16x4] * B[4x16] in fp32.
//   A: lane l supplies A[l % 16][l / 16]; B: lane l supplies B[l / 16][l % 16].
__device__ __forceinline__ f32x4 mfma16x16x4f32(float a, float b, const f32x4& c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// SiLU(a) = a / (1 + e^{-a}), with the hardware reciprocal (within 1 ulp)
// in place of a correctly rounded division.  The conv kernel and the conv
// front end of the prefill both use this one definition, so their outputs
// agree bit for bit.
__device__ __forceinline__ float silu_f32(float a)
{
    return a * __builtin_amdgcn_rcpf(1.0f + __expf(-a));
}

// Gated RMSNorm arithmetic: 1 / rms from a row's sum of squares, and one
// output element (h * inv * w + b) * act(z) with act(z) = z * sigmoid(z), or
// sigmoid(z) when `sigmoid` (hardware reciprocal).
__device__ __forceinline__ float rms_inv(float ss, int dim, float eps)
{
    return 1.0f / sqrtf(ss / (float)dim + eps);
}
__device__ __forceinline__ float gated_norm_out(float h, float inv, float w, float b, float z,
                                                bool sigmoid)
{
    const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-z));
    const float act = sigmoid ? sg : z * sg;
    return (h * inv * w + b) * act;
}

__device__ __forceinline__ bf16x8 pack_bf16x8(const float (&x)[8])
{
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = static_cast<bf16>(x[i]);
    return r;
}

}  // namespace kda
