// prefill.hip -- KDA chunk prefill over a varlen batch.
//
// Page "[Feature][KDA] Add Kimi K3 KDA execution", KDA execution step 3: the
// prefill builds the cumulative gate and then runs the chunked operator.
// Page "[KK] Prepare B12X Kimi KDA prefill ...", Behavior: states are read
// and written in place at their pool slot, scratch is caller-owned.
// Page "FlashKDA kernel upgrade supports bf16 checkpoint state": checkpoint
// states at segment boundaries, stored in the state dtype.
//
// Chunk algebra (exact up to rounding).  In a chunk of C tokens, with the
// inclusive cumulative gate G_r = sum_{s<=r} g_s (per key channel):
//   K~_r = e^{G_r} k_r,  Q~_r = e^{G_r} q_r,  K^_s = e^{-G_s} k_s,
//   Kb_s = e^{G_C - G_s} k_s,
//   M    = strict_lower(Diag(beta) K~ K^T),   X = (I + M)^{-1},
//   T    = X Diag(beta),  W = T K~,  U = T V,  Aqk = incl_lower(Q~ K^T);
// then, carrying S through the chunks of one sequence in order:
//   D   = U - W S                         (the chunk's rank-one writes)
//   O   = scale (Q~ S + Aqk D)
//   S  <- Diag(e^{G_C}) S + Kb^T D
// Every column of S (a d_v index) evolves independently.
//
// Two kernels:
//   intra_kernel  one workgroup per (chunk, head), all chunks in parallel:
//                 gate cumsum, Gram products on bf16 MFMA, the blocked
//                 triangular solve (16x16 forward substitution per diagonal
//                 block, off-diagonal blocks on fp32 MFMA), W and U on bf16
//                 MFMA.  Writes one record per (chunk, head) to the workspace.
//   chain_kernel  one workgroup per (sequence, head, 16-column d_v tile);
//                 walks the sequence's chunks in order with S held in fp32
//                 accumulators.  The four waves split the token rows of D and
//                 O and the key rows of S; D and a bf16 copy of S are shared
//                 through LDS (two barriers per chunk).  Reads S0 from
//                 pool[slot], writes checkpoints and the final state in place.
//
// Range of the decay factors.  Products e^{G_r - G_s} (r >= s) are at most 1,
// but the factors e^{-G_s} alone overflow fp32 for long strong decays, so the
// Gram products are formed per 16-token sub-chunk i with the reference point
// b_i = the token before the sub-chunk:  (e^{G_r - G_b} q_r) . (e^{G_b - G_s} k_s).
// Off-diagonal blocks have both factors <= 1; diagonal blocks grow at most by
// the decay accumulated inside one sub-chunk, which must stay above e^{-80}.

#include "kda_device.cuh"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kThreads = 256;   // four waves per workgroup

template <int D, int BT>
struct Shape {
    static constexpr int DKP = D < 32 ? 32 : D;      // key dim padded to the MFMA K step
    static constexpr int BTP = BT < 32 ? 32 : BT;    // token dim padded to the MFMA K step
    static constexpr int NS = BT / 16;               // 16-token sub-chunks (token m-tiles)
    static constexpr int NMT_K = DKP / 16;           // key-dim m-tiles of S
    static constexpr int NKK_K = DKP / 32;           // MFMA K steps over keys
    static constexpr int NKK_T = BTP / 32;           // MFMA K steps over tokens
    // Workspace record of one (chunk, head), bf16 arrays then fp32 decay:
    static constexpr int64_t OFF_Q = 0;                        // Q~   [BT][DKP]
    static constexpr int64_t OFF_W = OFF_Q + BT * DKP;         // W    [BT][DKP]
    static constexpr int64_t OFF_KB = OFF_W + BT * DKP;        // Kb^T [DKP][BTP]
    static constexpr int64_t OFF_U = OFF_KB + DKP * BTP;       // U^T  [D][BTP]
    static constexpr int64_t OFF_A = OFF_U + D * BTP;          // Aqk  [BT][BTP]
    static constexpr int64_t BF16_END = OFF_A + BT * BTP;
    static constexpr int64_t EG_BYTE_OFF = BF16_END * 2;       // e^{G_C} fp32 [DKP]
    static constexpr int64_t REC_BYTES = ((EG_BYTE_OFF + DKP * 4) + 255) / 256 * 256;
    static_assert(BT % 16 == 0 && BT <= 64, "chunk size");
    static_assert(D % 16 == 0 && D <= 128, "head dim");
};

int64_t max_chunks(int32_t num_seqs, int64_t total_tokens, int32_t chunk)
{
    return (total_tokens + chunk - 1) / chunk + num_seqs;
}

// Eight consecutive activations (16 B bf16 / 32 B fp32) widened to fp32.
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

__device__ __forceinline__ int num_chunks(int len, int bt) { return len > 0 ? (len + bt - 1) / bt : 0; }

// The sequence that owns global chunk x (chunks numbered sequence by sequence)
// and the index of that sequence's first chunk.  Whole-wave call; false if x
// is past the last chunk.
__device__ bool locate_chunk(const int32_t* __restrict__ cu, int n, int bt, int x, int lane,
                             int& seq, int& first)
{
    int base = 0;
    for (int i0 = 0; i0 < n; i0 += kWave) {
        const int i = i0 + lane;
        const int nch = i < n ? num_chunks(cu[i + 1] - cu[i], bt) : 0;
        const int incl = wave_inclusive_scan(nch, lane);
        const int excl = base + incl - nch;
        const unsigned long long hit = __ballot(i < n && x >= excl && x < excl + nch);
        if (hit) {
            const int src = __ffsll((long long)hit) - 1;
            seq = __shfl(i, src, kWave);
            first = __shfl(excl, src, kWave);
            return true;
        }
        base += __shfl(incl, kWave - 1, kWave);
    }
    return false;
}

// Sums over the sequences before `seq`: their chunk count and their
// checkpoint count.  Whole-wave call.
__device__ void sequence_bases(const int32_t* __restrict__ cu, int seq, int bt, int interval,
                               int lane, int& chunk_base, int64_t& ckpt_base)
{
    int cb = 0;
    int64_t kb = 0;
    for (int i0 = 0; i0 < seq; i0 += kWave) {
        const int i = i0 + lane;
        int nch = 0;
        int64_t nck = 0;
        if (i < seq) {
            const int len = cu[i + 1] - cu[i];
            nch = num_chunks(len, bt);
            nck = (interval > 0 && len > 0) ? len / interval : 0;
        }
        cb += nch;
        kb += nck;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        cb += __shfl_xor(cb, off, kWave);
        kb += __shfl_xor(kb, off, kWave);
    }
    chunk_base = cb;
    ckpt_base = kb;
}

// ---------------------------------------------------------------------------
// Eight activations as bf16 (fp32 inputs are rounded once, here).
__device__ __forceinline__ bf16x8 load8_bf16(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ bf16x8 load8_bf16(const float* p)
{
    float x[8];
    load8(p, x);
    return pack_bf16x8(x);
}
__device__ __forceinline__ bf16x4 pack_bf16x4(const f32x4& x)
{
    bf16x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = static_cast<bf16>(x[i]);
    return r;
}

// ---------------------------------------------------------------------------
// intra_kernel: everything in a chunk that does not depend on the state.
// Phase 0 stages the chunk's q, k, v, g, beta into LDS with every global
// load issued before the first use; all later phases read LDS only.
template <int D, int BT, typename AT>
__global__ __launch_bounds__(kThreads)
void intra_kernel(const AT* __restrict__ q, const AT* __restrict__ k, const AT* __restrict__ v,
                  int64_t qs, int64_t ks, int64_t vs, const float* __restrict__ g,
                  const float* __restrict__ beta, const int32_t* __restrict__ cu, int n_seqs,
                  int heads, const int32_t* __restrict__ slots, uint32_t flags,
                  uint8_t* __restrict__ ws)
{
    using P = Shape<D, BT>;
    constexpr int DKP = P::DKP, BTP = P::BTP, NS = P::NS;
    constexpr int GP = D + 4;                // fp32 pitch of sG (16-B rows)
    constexpr int RP = D + 8;                // bf16 pitch of sQ / sK
    constexpr int MP = BT + 4;               // fp32 pitch of sM / sX
    constexpr int TP = BTP + 8;              // bf16 pitch of the transposed tiles
    constexpr int VG = D / 8;                // 8-element groups per activation row

    __shared__ __attribute__((aligned(16))) float sG[BT][GP];    // g, then its inclusive cumsum
    __shared__ __attribute__((aligned(16))) bf16 sQ[BT][RP];     // raw q
    __shared__ __attribute__((aligned(16))) bf16 sK[BT][RP];     // raw k
    __shared__ __attribute__((aligned(16))) bf16 sVt[D][TP];     // V^T
    __shared__ __attribute__((aligned(16))) float sM[BT][MP];    // strict_lower(Diag(beta) K~ K^T)
    __shared__ __attribute__((aligned(16))) float sX[BT][MP];    // (I + M)^{-1}
    __shared__ __attribute__((aligned(16))) bf16 sKt[DKP][TP];   // K~^T
    __shared__ float sRq[BT], sRk[BT], sBeta[BT];
    __shared__ float sTmp[4][16][17];        // per-wave 16x16 scratch for the solve

    const int x = blockIdx.x, h = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int l16 = lane & 15, g4 = lane >> 4;

    int seq = 0, first = 0;
    if (!locate_chunk(cu, n_seqs, BT, x, lane, seq, first)) return;
    if (slots[seq] < 0) return;              // padding sequence: nothing to precompute
    const int64_t t0 = (int64_t)cu[seq] + (int64_t)(x - first) * BT;
    const int len = (int)min<int64_t>(BT, (int64_t)cu[seq + 1] - t0);

    uint8_t* rec = ws + ((int64_t)x * heads + h) * P::REC_BYTES;
    bf16* wQ = reinterpret_cast<bf16*>(rec) + P::OFF_Q;
    bf16* wW = reinterpret_cast<bf16*>(rec) + P::OFF_W;
    bf16* wKb = reinterpret_cast<bf16*>(rec) + P::OFF_KB;
    bf16* wU = reinterpret_cast<bf16*>(rec) + P::OFF_U;
    bf16* wA = reinterpret_cast<bf16*>(rec) + P::OFF_A;
    float* wEg = reinterpret_cast<float*>(rec + P::EG_BYTE_OFF);

    // 0. Stage q, k, v (as bf16), g and beta.
    {
        constexpr int NQ = (BT * VG + kThreads - 1) / kThreads;
        constexpr int NG = (BT * (D / 4) + kThreads - 1) / kThreads;
        bf16x8 rq[NQ], rk[NQ], rv[NQ];
        float4 rg[NG];
#pragma unroll
        for (int it = 0; it < NQ; ++it) {
            const int idx = tid + it * kThreads;
            const int r = idx / VG, c0 = 8 * (idx % VG);
            if (idx < BT * VG && r < len) {
                const int64_t t = t0 + r;
                rq[it] = load8_bf16(q + t * qs + (int64_t)h * D + c0);
                rk[it] = load8_bf16(k + t * ks + (int64_t)h * D + c0);
                rv[it] = load8_bf16(v + t * vs + (int64_t)h * D + c0);
            } else {
                rq[it] = bf16x8{}; rk[it] = bf16x8{}; rv[it] = bf16x8{};
            }
        }
#pragma unroll
        for (int it = 0; it < NG; ++it) {
            const int idx = tid + it * kThreads;
            const int r = idx / (D / 4), c0 = 4 * (idx % (D / 4));
            rg[it] = (idx < BT * (D / 4) && r < len)
                         ? *reinterpret_cast<const float4*>(g + ((t0 + r) * heads + h) * D + c0)
                         : make_float4(0.f, 0.f, 0.f, 0.f);
        }
        if (tid < BT) sBeta[tid] = tid < len ? beta[(t0 + tid) * heads + h] : 0.0f;
#pragma unroll
        for (int it = 0; it < NQ; ++it) {
            const int idx = tid + it * kThreads;
            if (idx < BT * VG) {
                const int r = idx / VG, c0 = 8 * (idx % VG);
                *reinterpret_cast<bf16x8*>(&sQ[r][c0]) = rq[it];
                *reinterpret_cast<bf16x8*>(&sK[r][c0]) = rk[it];
#pragma unroll
                for (int e = 0; e < 8; ++e) sVt[c0 + e][r] = rv[it][e];
            }
        }
#pragma unroll
        for (int it = 0; it < NG; ++it) {
            const int idx = tid + it * kThreads;
            if (idx < BT * (D / 4))
                *reinterpret_cast<float4*>(&sG[idx / (D / 4)][4 * (idx % (D / 4))]) = rg[it];
        }
        if (BTP > BT)
            for (int idx = tid; idx < D * (BTP - BT); idx += kThreads)
                sVt[idx / (BTP - BT)][BT + idx % (BTP - BT)] = static_cast<bf16>(0.0f);
    }
    __syncthreads();

    // 1. Inclusive cumulative gate per channel: NSPLIT threads per channel
    //    scan consecutive row segments, then add the totals before them.
    {
        constexpr int NSPLIT = kThreads / D;
        constexpr int RPC = BT / NSPLIT;
        static_assert(RPC >= 1 && BT % NSPLIT == 0, "gate split");
        const int c = tid % D, part = tid / D;
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < RPC; ++i) {
            acc += sG[part * RPC + i][c];
            sG[part * RPC + i][c] = acc;
        }
        __syncthreads();
        float pre = 0.0f;
        for (int p = 0; p < part; ++p) pre += sG[(p + 1) * RPC - 1][c];
        __syncthreads();
        if (part > 0)
#pragma unroll
            for (int i = 0; i < RPC; ++i) sG[part * RPC + i][c] += pre;
    }
    // Row norms for the optional q/k L2 normalisation.
    {
        constexpr int TPRN = kThreads / BT;
        const int r = tid / TPRN, part = tid % TPRN;
        float sq = 0.0f, sk = 0.0f;
        if (flags & KDA_FLAG_QK_L2NORM) {
            for (int c = part; c < D; c += TPRN) {
                const float a = static_cast<float>(sQ[r][c]), b = static_cast<float>(sK[r][c]);
                sq += a * a;
                sk += b * b;
            }
        }
#pragma unroll
        for (int off = TPRN / 2; off > 0; off >>= 1) {
            sq += __shfl_xor(sq, off, kWave);
            sk += __shfl_xor(sk, off, kWave);
        }
        if (part == 0) {
            const bool nrm = (flags & KDA_FLAG_QK_L2NORM) != 0;
            sRq[r] = nrm ? 1.0f / sqrtf(sq + 1e-6f) : 1.0f;
            sRk[r] = nrm ? 1.0f / sqrtf(sk + 1e-6f) : 1.0f;
        }
    }
    __syncthreads();

    // 2. Elementwise factors.  Q~ -> record (row-major); K~^T -> LDS and
    //    Kb^T -> record (8 consecutive tokens per thread, 16-B stores).
    for (int idx = tid; idx < BT * (DKP / 8); idx += kThreads) {
        const int r = idx / (DKP / 8), c0 = 8 * (idx % (DKP / 8));
        float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (r < len && c0 < D) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                o[e] = static_cast<float>(sQ[r][c0 + e]) * sRq[r] * __expf(sG[r][c0 + e]);
        }
        *reinterpret_cast<bf16x8*>(wQ + (int64_t)r * DKP + c0) = pack_bf16x8(o);
    }
    for (int idx = tid; idx < DKP * (BTP / 8); idx += kThreads) {
        const int c = idx / (BTP / 8), s0 = 8 * (idx % (BTP / 8));
        float kt[8], kb[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int s = s0 + e;
            kt[e] = 0.0f;
            kb[e] = 0.0f;
            if (s < len && c < D) {
                const float kv = static_cast<float>(sK[s][c]) * sRk[s];
                kt[e] = kv * __expf(sG[s][c]);
                kb[e] = kv * __expf(sG[BT - 1][c] - sG[s][c]);
            }
        }
        *reinterpret_cast<bf16x8*>(&sKt[c][s0]) = pack_bf16x8(kt);
        *reinterpret_cast<bf16x8*>(wKb + (int64_t)c * BTP + s0) = pack_bf16x8(kb);
    }
    for (int c = tid; c < DKP; c += kThreads) wEg[c] = c < D ? __expf(sG[BT - 1][c]) : 0.0f;
    // Zero the blocks above the diagonal of M and X, and of Aqk (with its
    // token padding).
    for (int idx = tid; idx < BT * BT; idx += kThreads) {
        const int r = idx / BT, s = idx % BT;
        if (s >= 16 * (r / 16 + 1)) { sM[r][s] = 0.0f; sX[r][s] = 0.0f; }
    }
    for (int idx = tid; idx < BT * (BTP / 8); idx += kThreads) {
        const int r = idx / (BTP / 8), s0 = 8 * (idx % (BTP / 8));
        if (s0 >= 16 * (r / 16 + 1)) *reinterpret_cast<bf16x8*>(wA + (int64_t)r * BTP + s0) = bf16x8{};
    }

    // 3. Gram blocks on bf16 MFMA (K = key dim), computed transposed so each
    //    lane ends up with 4 consecutive columns s of one row r:
    //    C[s][r] = (e^{G_b - G_s} k_s) . (e^{G_r - G_b} k_r or q_r), b = the
    //    token before sub-chunk i.  Wave w owns block row i = w.
    if (wave < NS) {
        const int i = wave;
        const int r = 16 * i + l16;
        bf16x8 bK[P::NKK_K], bQ[P::NKK_K];
#pragma unroll
        for (int kk = 0; kk < P::NKK_K; ++kk) {
            const int c0 = 32 * kk + 8 * g4;
            float fk[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            float fq[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            if (r < len && c0 < D) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float gb = i > 0 ? sG[16 * i - 1][c0 + e] : 0.0f;
                    const float ex = __expf(sG[r][c0 + e] - gb);
                    fk[e] = static_cast<float>(sK[r][c0 + e]) * sRk[r] * ex;
                    fq[e] = static_cast<float>(sQ[r][c0 + e]) * sRq[r] * ex;
                }
            }
            bK[kk] = pack_bf16x8(fk);
            bQ[kk] = pack_bf16x8(fq);
        }
        for (int j = 0; j <= i; ++j) {
            const int s = 16 * j + l16;
            f32x4 accK = {0.f, 0.f, 0.f, 0.f}, accQ = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < P::NKK_K; ++kk) {
                const int c0 = 32 * kk + 8 * g4;
                float fa[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
                if (s < len && c0 < D) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float gb = i > 0 ? sG[16 * i - 1][c0 + e] : 0.0f;
                        fa[e] = static_cast<float>(sK[s][c0 + e]) * sRk[s] * __expf(gb - sG[s][c0 + e]);
                    }
                }
                const bf16x8 a = pack_bf16x8(fa);
                accK = mfma16x16x32(a, bK[kk], accK);
                accQ = mfma16x16x32(a, bQ[kk], accQ);
            }
            const int rr = 16 * i + l16;
            f32x4 mk, aq;
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int ss = 16 * j + 4 * g4 + ii;
                mk[ii] = ss < rr ? sBeta[rr] * accK[ii] : 0.0f;
                aq[ii] = ss <= rr ? accQ[ii] : 0.0f;
            }
            *reinterpret_cast<f32x4*>(&sM[rr][16 * j + 4 * g4]) = mk;
            *reinterpret_cast<bf16x4*>(wA + (int64_t)rr * BTP + 16 * j + 4 * g4) = pack_bf16x4(aq);
        }
    }
    __syncthreads();

    // 4a. Diagonal blocks of X = (I + M)^{-1}: forward substitution, one wave
    //     per block, one lane per column.
    if (wave < NS && l16 == lane) {
        const int b0 = 16 * wave;
        float xcol[16];
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            float acc = rr == lane ? 1.0f : 0.0f;
#pragma unroll
            for (int s = 0; s < rr; ++s) acc -= sM[b0 + rr][b0 + s] * xcol[s];
            xcol[rr] = acc;
            sX[b0 + rr][b0 + lane] = acc;
        }
    }
    __syncthreads();

    // 4b. Off-diagonal blocks, block row by block row:
    //     X_ij = -X_ii sum_{j<=m<i} M_im X_mj  (fp32 MFMA); wave j does (i, j).
    for (int i = 1; i < NS; ++i) {
        if (wave < i) {
            const int j = wave;
            f32x4 y = {0.f, 0.f, 0.f, 0.f};
            for (int m = j; m < i; ++m) {
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    y = mfma16x16x4f32(sM[16 * i + l16][16 * m + 4 * kk + g4],
                                       sX[16 * m + 4 * kk + g4][16 * j + l16], y);
            }
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) sTmp[wave][4 * g4 + ii][l16] = y[ii];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                z = mfma16x16x4f32(sX[16 * i + l16][16 * i + 4 * kk + g4],
                                   sTmp[wave][4 * kk + g4][l16], z);
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) sX[16 * i + 4 * g4 + ii][16 * j + l16] = -z[ii];
        }
        __syncthreads();
    }

    // 5. With T = X Diag(beta): W^T = K~^T T^T (so each lane stores 4
    //    consecutive key channels of one W row) and U = T V (4 consecutive
    //    tokens of one U^T row), on bf16 MFMA up to the diagonal.
    {
        constexpr int NTW = (DKP / 16) * NS, NTU = NS * (D / 16);
        auto t_row = [&](int r, int s0) {           // T[r][s0 .. s0+7] as bf16
            float f[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int s = s0 + e;
                f[e] = s < BT ? sX[r][s] * sBeta[s] : 0.0f;
            }
            return pack_bf16x8(f);
        };
        for (int t = wave; t < NTW + NTU; t += 4) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            if (t < NTW) {
                const int mt = t / NS, nt = t % NS;             // key tile, token tile
                const int kmax = (16 * nt + 15) / 32;
                for (int kk = 0; kk <= kmax; ++kk) {
                    const int s0 = 32 * kk + 8 * g4;
                    acc = mfma16x16x32(*reinterpret_cast<const bf16x8*>(&sKt[16 * mt + l16][s0]),
                                       t_row(16 * nt + l16, s0), acc);
                }
                *reinterpret_cast<bf16x4*>(wW + (int64_t)(16 * nt + l16) * DKP + 16 * mt + 4 * g4) =
                    pack_bf16x4(acc);
            } else {
                const int tt = t - NTW;
                const int mt = tt / (D / 16), nt = tt % (D / 16);  // token tile, value tile
                const int kmax = (16 * mt + 15) / 32;
                for (int kk = 0; kk <= kmax; ++kk) {
                    const int s0 = 32 * kk + 8 * g4;
                    acc = mfma16x16x32(t_row(16 * mt + l16, s0),
                                       *reinterpret_cast<const bf16x8*>(&sVt[16 * nt + l16][s0]), acc);
                }
                *reinterpret_cast<bf16x4*>(wU + (int64_t)(16 * nt + l16) * BTP + 16 * mt + 4 * g4) =
                    pack_bf16x4(acc);
            }
        }
        if (BTP > BT)
            for (int idx = tid; idx < D * (BTP - BT) / 4; idx += kThreads) {
                const int row = idx / ((BTP - BT) / 4), c4 = idx % ((BTP - BT) / 4);
                *reinterpret_cast<bf16x4*>(wU + (int64_t)row * BTP + BT + 4 * c4) = bf16x4{};
            }
    }
}

// ---------------------------------------------------------------------------
// chain_kernel: the state-dependent part, serial over a sequence's chunks.
//
// One workgroup per (sequence, head, 16-column d_v tile) with eleven waves in
// four roles.  Each role runs its own loop over the chunks and every role
// executes the same two barriers per chunk (B1: D is ready; B2: the next S and
// the next operand stage are ready):
//   state waves 0-3    D = U - W S for token tile w; then S <- e^{G_C} S + Kb^T D
//                      for key tiles w, w+4.  S stays in fp32 accumulators and
//                      is shared as bf16 S^T through a ping-pong LDS tile.
//   output waves 4-7   O = scale (Q~ S + Aqk D) for token tile w-4, with their
//                      Q~ and Aqk rows prefetched into registers 3 chunks ahead.
//   loader waves 8-9   stream each chunk's W, Kb^T, U tile and e^{G_C} into a
//                      3-stage LDS ring with asynchronous global->LDS loads.
//   warmer wave 10     asks for this tile's share of the record WARM chunks
//                      ahead, so that the L2 of the XCD (shared by all tiles of
//                      the pair) holds each record before it is streamed; a CU
//                      reads its L2 several times faster than it pulls from HBM.
// State waves issue no global loads, and loads with different latencies sit
// in different waves, so no wave waits on another's prefetch.
constexpr int kChainWaves = 11;
constexpr int kChainThreads = kChainWaves * kWave;
constexpr int kStages = 3;
constexpr int kWarm = 4;

template <int D, int BT>
struct ChainStage {
    using P = Shape<D, BT>;
    static constexpr int W_OFF = 0;                                   // W    [BT][DKP]
    static constexpr int KB_OFF = W_OFF + BT * P::DKP * 2;            // Kb^T [DKP][BTP]
    static constexpr int U_OFF = KB_OFF + P::DKP * P::BTP * 2;        // U^T tile [16][BTP]
    static constexpr int EG_OFF = U_OFF + 16 * P::BTP * 2;            // e^{G_C} [DKP] fp32
    static constexpr int BYTES = (EG_OFF + P::DKP * 4 + 1023) / 1024 * 1024;
    // asynchronous 1-KB copies per stage (64 lanes x 16 B)
    static constexpr int OPS_W = (BT * P::DKP * 2 + 1023) / 1024;
    static constexpr int OPS_KB = (P::DKP * P::BTP * 2 + 1023) / 1024;
    static constexpr int OPS_U = (16 * P::BTP * 2 + 1023) / 1024;
    static constexpr int OPS_EG = (P::DKP * 4 + 1023) / 1024;
    static constexpr int OPS = OPS_W + OPS_KB + OPS_U + OPS_EG;
};

typedef __attribute__((address_space(3))) void lds_void;

// Copy `bytes` (a multiple of 16) from global `src` to LDS `dst` in 1-KB
// asynchronous pieces; every piece is issued (lanes past the end idle), so the
// number of memory operations is fixed.
__device__ __forceinline__ void copy_async(uint8_t* dst, const uint8_t* src, int bytes, int lane)
{
    for (int off = 0; off < bytes; off += kWave * 16) {
        if (off + lane * 16 < bytes)
            __builtin_amdgcn_global_load_lds((const void*)(src + off + lane * 16), (lds_void*)(dst + off), 16, 0, 0);
    }
}

template <int D, int BT, typename AT, typename ST>
__global__ __launch_bounds__(kChainThreads)
void chain_kernel(const int32_t* __restrict__ cu, int n_seqs, int heads,
                  ST* __restrict__ pool, int64_t num_slots, const int32_t* __restrict__ slots,
                  const uint8_t* __restrict__ has_init, ST* __restrict__ ckpt, int64_t ckpt_cap,
                  int interval, float scale, AT* __restrict__ out, int64_t os,
                  const uint8_t* __restrict__ ws)
{
    using P = Shape<D, BT>;
    using SG = ChainStage<D, BT>;
    constexpr int DKP = P::DKP, BTP = P::BTP, NS = P::NS;
    constexpr int TILES = D / 16;                 // column tiles of one (sequence, head)
    constexpr int NKT_W = (P::NMT_K + 3) / 4;     // key m-tiles per state wave
    constexpr int SP = DKP + 8, DP = BTP + 8;     // bf16 pitches of the exchange tiles

    __shared__ __attribute__((aligned(1024))) uint8_t sStage[kStages][SG::BYTES];
    __shared__ __attribute__((aligned(16))) bf16 sS[2][16][SP];   // bf16 S^T (ping-pong)
    __shared__ __attribute__((aligned(16))) bf16 sD[16][DP];      // bf16 D^T
    __shared__ __attribute__((aligned(1024))) uint8_t sWarm[kWave * 16];   // discarded

    // blockIdx.x enumerates (sequence, head) pairs, padded to a multiple of 8,
    // and blockIdx.y the column tile: workgroups are dealt to the 8 XCDs
    // round-robin by linear id, so all tiles of one pair share an XCD and its L2.
    const int pair = blockIdx.x;
    if (pair >= n_seqs * heads) return;
    const int seq = pair / heads, h = pair % heads, tile = blockIdx.y, n0 = tile * 16;
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    __builtin_assume(wave >= 0 && wave < kChainWaves);
    const int l16 = lane & 15, g4 = lane >> 4;
    const int col = n0 + l16;

    const int64_t s_begin = cu[seq];
    const int len = max(0, cu[seq + 1] - cu[seq]);
    const int slot = slots[seq];
    if (slot < 0) {                                // graph padding: zero output rows
        for (int idx = tid; idx < len * 16; idx += kChainThreads)
            out[(s_begin + idx / 16) * os + (int64_t)h * D + n0 + idx % 16] = from_f32<AT>(0.0f);
        return;
    }
    if (len == 0 || slot >= num_slots) return;

    int chunk_base = 0;
    int64_t ckpt_base = 0;
    sequence_bases(cu, seq, BT, interval, lane, chunk_base, ckpt_base);
    const int nch = num_chunks(len, BT);
    auto record = [&](int lc) {
        return ws + ((int64_t)(chunk_base + min(lc, nch - 1)) * heads + h) * P::REC_BYTES;
    };

    if (wave < 4) {
        // ---------------- state waves ----------------
        const bool init = has_init ? has_init[seq] != 0 : true;
        ST* home = pool + ((int64_t)slot * heads + h) * (int64_t)(D * D);
        float S[NKT_W][4];
#pragma unroll
        for (int j = 0; j < NKT_W; ++j) {
            const int kt = wave + 4 * j;
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int row = 16 * kt + 4 * g4 + ii;
                S[j][ii] = (init && kt < P::NMT_K && row < D) ? to_f32(home[(int64_t)row * D + col]) : 0.0f;
            }
            if (kt < P::NMT_K) {
                bf16x4 s4;
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) s4[ii] = static_cast<bf16>(S[j][ii]);
                *reinterpret_cast<bf16x4*>(&sS[0][l16][16 * kt + 4 * g4]) = s4;
            }
        }
        if (BTP > BT && wave == 0)                 // token padding of D^T stays zero
            *reinterpret_cast<bf16x4*>(&sD[l16][BT + 4 * g4]) = bf16x4{};
        lds_barrier();                             // B0: S_0 published, stage 0 loaded

        for (int lc = 0; lc < nch; ++lc) {
            const uint8_t* stg = sStage[lc % kStages];
            const bf16* sW = reinterpret_cast<const bf16*>(stg + SG::W_OFF);
            const bf16* sKb = reinterpret_cast<const bf16*>(stg + SG::KB_OFF);
            const bf16* sU = reinterpret_cast<const bf16*>(stg + SG::U_OFF);
            const float* sEg = reinterpret_cast<const float*>(stg + SG::EG_OFF);
            const int cur = lc & 1;
            if (wave < NS) {                       // D = U - W S, token tile `wave`
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < P::NKK_K; ++kk)
                    acc = mfma16x16x32(
                        *reinterpret_cast<const bf16x8*>(sW + (16 * wave + l16) * DKP + 32 * kk + 8 * g4),
                        *reinterpret_cast<const bf16x8*>(&sS[cur][l16][32 * kk + 8 * g4]), acc);
                const bf16x4 u4 = *reinterpret_cast<const bf16x4*>(sU + l16 * BTP + 16 * wave + 4 * g4);
                bf16x4 d4;
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) d4[ii] = static_cast<bf16>(static_cast<float>(u4[ii]) - acc[ii]);
                *reinterpret_cast<bf16x4*>(&sD[l16][16 * wave + 4 * g4]) = d4;
            }
            lds_barrier();                         // B1
#pragma unroll
            for (int j = 0; j < NKT_W; ++j) {      // S <- Diag(e^{G_C}) S + Kb^T D
                const int kt = wave + 4 * j;
                if (kt >= P::NMT_K) continue;
                const f32x4 eg = *reinterpret_cast<const f32x4*>(sEg + 16 * kt + 4 * g4);
                f32x4 acc;
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) acc[ii] = S[j][ii] * eg[ii];
#pragma unroll
                for (int kk = 0; kk < P::NKK_T; ++kk)
                    acc = mfma16x16x32(
                        *reinterpret_cast<const bf16x8*>(sKb + (16 * kt + l16) * BTP + 32 * kk + 8 * g4),
                        *reinterpret_cast<const bf16x8*>(&sD[l16][32 * kk + 8 * g4]), acc);
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) S[j][ii] = acc[ii];
                bf16x4 s4;
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) s4[ii] = static_cast<bf16>(S[j][ii]);
                *reinterpret_cast<bf16x4*>(&sS[cur ^ 1][l16][16 * kt + 4 * g4]) = s4;
            }
            const int pos = (lc + 1) * BT;         // checkpoint at this chunk's end
            if (ckpt && interval > 0 && pos <= len && pos % interval == 0) {
                const int64_t row = ckpt_base + pos / interval - 1;
                if (row < ckpt_cap) {
                    ST* dst = ckpt + (row * heads + h) * (int64_t)(D * D);
#pragma unroll
                    for (int j = 0; j < NKT_W; ++j) {
                        const int kt = wave + 4 * j;
#pragma unroll
                        for (int ii = 0; ii < 4; ++ii) {
                            const int rr = 16 * kt + 4 * g4 + ii;
                            if (kt < P::NMT_K && rr < D) dst[(int64_t)rr * D + col] = from_f32<ST>(S[j][ii]);
                        }
                    }
                }
            }
            lds_barrier();                         // B2
        }
#pragma unroll
        for (int j = 0; j < NKT_W; ++j) {          // final state, in place
            const int kt = wave + 4 * j;
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int rr = 16 * kt + 4 * g4 + ii;
                if (kt < P::NMT_K && rr < D) home[(int64_t)rr * D + col] = from_f32<ST>(S[j][ii]);
            }
        }
    } else if (wave < 8) {
        // ---------------- output waves ----------------
        const int tt = wave - 4;                   // token tile
        const bool active = tt < NS;
        const int kmax = (16 * tt + 15) / 32;
        struct OutOps { bf16x8 q[P::NKK_K]; bf16x8 a[P::NKK_T]; };
        auto load_ops = [&](OutOps& o, int lc) {
            const uint8_t* rec = record(lc);
            const bf16* wQ = reinterpret_cast<const bf16*>(rec) + P::OFF_Q;
            const bf16* wA = reinterpret_cast<const bf16*>(rec) + P::OFF_A;
            const int64_t row = 16 * (active ? tt : 0) + l16;
#pragma unroll
            for (int kk = 0; kk < P::NKK_K; ++kk)
                o.q[kk] = *reinterpret_cast<const bf16x8*>(wQ + row * DKP + 32 * kk + 8 * g4);
#pragma unroll
            for (int kk = 0; kk < P::NKK_T; ++kk)
                o.a[kk] = *reinterpret_cast<const bf16x8*>(wA + row * BTP + 32 * kk + 8 * g4);
        };
        auto step = [&](const OutOps& o, int lc) {
            const int cur = lc & 1;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            if (active) {
#pragma unroll
                for (int kk = 0; kk < P::NKK_K; ++kk)
                    acc = mfma16x16x32(o.q[kk], *reinterpret_cast<const bf16x8*>(&sS[cur][l16][32 * kk + 8 * g4]), acc);
            }
            lds_barrier();                         // B1
            if (active) {
#pragma unroll
                for (int kk = 0; kk < P::NKK_T; ++kk)
                    if (kk <= kmax)
                        acc = mfma16x16x32(o.a[kk], *reinterpret_cast<const bf16x8*>(&sD[l16][32 * kk + 8 * g4]), acc);
                const int64_t tc = s_begin + (int64_t)lc * BT;
                const int clen = min(BT, len - lc * BT);
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    const int r = 16 * tt + 4 * g4 + ii;
                    if (r < clen) out[(tc + r) * os + (int64_t)h * D + col] = from_f32<AT>(scale * acc[ii]);
                }
            }
        };
        OutOps o0, o1, o2;
        load_ops(o0, 0);
        load_ops(o1, 1);
        lds_barrier();                             // B0
        for (int lc = 0; lc < nch; lc += 3) {
            load_ops(o2, lc + 2);
            step(o0, lc);
            lds_barrier();                         // B2
            if (lc + 1 >= nch) break;
            load_ops(o0, lc + 3);
            step(o1, lc + 1);
            lds_barrier();
            if (lc + 2 >= nch) break;
            load_ops(o1, lc + 4);
            step(o2, lc + 2);
            lds_barrier();
        }
    } else if (wave < 10) {
        // ---------------- loader waves ----------------
        // Stage copies are split between the two loader waves; each wave waits
        // only for its own copies (vmcnt counts per wave, in issue order).
        const int lw = wave - 8;
        auto issue_stage = [&](int lc) {
            uint8_t* dst = sStage[lc % kStages];
            const uint8_t* rec = record(lc);
            if (lw == 0) {
                copy_async(dst + SG::W_OFF, rec + P::OFF_W * 2, BT * DKP * 2, lane);
                copy_async(dst + SG::U_OFF, rec + (P::OFF_U + (int64_t)n0 * BTP) * 2, 16 * BTP * 2, lane);
            } else {
                copy_async(dst + SG::KB_OFF, rec + P::OFF_KB * 2, DKP * BTP * 2, lane);
                copy_async(dst + SG::EG_OFF, rec + P::EG_BYTE_OFF, DKP * 4, lane);
            }
        };
        // Copies one loader wave issues per stage (the larger of the two halves).
        issue_stage(0);
        issue_stage(1);
        // wait for stage 0: at most one stage's copies outstanding
        if (lw == 0) wait_vmcnt<SG::OPS_W + SG::OPS_U>();
        else wait_vmcnt<SG::OPS_KB + SG::OPS_EG>();
        lds_barrier();                             // B0
        for (int lc = 0; lc < nch; ++lc) {
            lds_barrier();                         // B1
            issue_stage(lc + 2);                   // into the stage chunk lc-1 used
            if (lw == 0) wait_vmcnt<SG::OPS_W + SG::OPS_U>();   // stage lc+1 complete
            else wait_vmcnt<SG::OPS_KB + SG::OPS_EG>();
            lds_barrier();                         // B2
        }
        wait_vmcnt<0>();
    } else {
        // ---------------- warmer wave ----------------
        constexpr int SHARE = (int)((P::REC_BYTES + TILES - 1) / TILES / 16 * 16);
        auto warm = [&](int lc) {
            if (lc >= nch) return;                 // uniform
            const uint8_t* base = record(lc) + (int64_t)tile * SHARE;
            for (int off = 0; off < SHARE; off += kWave * 16) {
                const int o = off + lane * 16;
                if (o < SHARE && tile * SHARE + o + 16 <= P::REC_BYTES)
                    __builtin_amdgcn_global_load_lds((const void*)(base + o), (lds_void*)sWarm, 16, 0, 0);
            }
        };
        for (int lc = 2; lc < 2 + kWarm; ++lc) warm(lc);
        lds_barrier();                             // B0
        for (int lc = 0; lc < nch; ++lc) {
            warm(lc + 2 + kWarm);
            lds_barrier();                         // B1
            lds_barrier();                         // B2
        }
        wait_vmcnt<0>();
    }
}

// ---------------------------------------------------------------------------
template <int D, int BT, typename AT, typename ST>
hipError_t launch_typed(const PrefillArgs& a, hipStream_t stream)
{
    const int64_t chunks = max_chunks(a.num_seqs, a.total_tokens, BT);
    if (chunks > INT32_MAX) return hipErrorInvalidValue;
    const int64_t pairs = ((int64_t)a.num_seqs * a.heads + 7) / 8 * 8;
    if (pairs > INT32_MAX) return hipErrorInvalidValue;
    if (a.ev[0]) {
        const hipError_t e = hipEventRecord(a.ev[0], stream);
        if (e != hipSuccess) return e;
    }
    if (a.total_tokens > 0) {
        hipLaunchKernelGGL((intra_kernel<D, BT, AT>), dim3((unsigned)chunks, (unsigned)a.heads),
                           dim3(kThreads), 0, stream, static_cast<const AT*>(a.q),
                           static_cast<const AT*>(a.k), static_cast<const AT*>(a.v), a.q_stride,
                           a.k_stride, a.v_stride, a.g, a.beta, a.cu_seqlens, a.num_seqs, a.heads,
                           a.slots, a.flags, static_cast<uint8_t*>(a.workspace));
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (a.ev[1]) {
        const hipError_t e = hipEventRecord(a.ev[1], stream);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((chain_kernel<D, BT, AT, ST>), dim3((unsigned)pairs, (unsigned)(D / 16)),
                       dim3(kChainThreads), 0, stream, a.cu_seqlens, a.num_seqs, a.heads,
                       static_cast<ST*>(a.pool), a.num_slots, a.slots, a.has_init,
                       static_cast<ST*>(a.ckpt), a.ckpt_capacity, a.ckpt_interval, a.scale,
                       static_cast<AT*>(a.out), a.out_stride,
                       static_cast<const uint8_t*>(a.workspace));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || !a.ev[2]) return e;
    return hipEventRecord(a.ev[2], stream);
}

template <int D, int BT>
hipError_t launch_types(const PrefillArgs& a, hipStream_t stream)
{
    if (a.act == KDA_BF16)
        return a.state == KDA_BF16 ? launch_typed<D, BT, bf16, bf16>(a, stream)
                                   : launch_typed<D, BT, bf16, float>(a, stream);
    return a.state == KDA_BF16 ? launch_typed<D, BT, float, bf16>(a, stream)
                               : launch_typed<D, BT, float, float>(a, stream);
}

template <int D>
hipError_t launch_chunk(const PrefillArgs& a, hipStream_t stream)
{
    switch (a.chunk) {
        case 16: return launch_types<D, 16>(a, stream);
        case 32: return launch_types<D, 32>(a, stream);
        case 64: return launch_types<D, 64>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

template <int D, int BT>
int64_t record_bytes() { return Shape<D, BT>::REC_BYTES; }

template <int D>
int64_t record_bytes_chunk(int32_t chunk)
{
    switch (chunk) {
        case 16: return record_bytes<D, 16>();
        case 32: return record_bytes<D, 32>();
        case 64: return record_bytes<D, 64>();
        default: return 0;
    }
}

}  // namespace

size_t prefill_workspace_bytes(int32_t num_seqs, int64_t total_tokens, int32_t heads, int32_t dk,
                               int32_t dv, int32_t chunk)
{
    if (dk != dv) return 0;
    int64_t rec = 0;
    switch (dk) {
        case 16: rec = record_bytes_chunk<16>(chunk); break;
        case 32: rec = record_bytes_chunk<32>(chunk); break;
        case 64: rec = record_bytes_chunk<64>(chunk); break;
        case 128: rec = record_bytes_chunk<128>(chunk); break;
        default: return 0;
    }
    if (rec == 0) return 0;
    return (size_t)(max_chunks(num_seqs, total_tokens, chunk) * heads * rec);
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream)
{
    switch (a.dk) {
        case 16: return launch_chunk<16>(a, stream);
        case 32: return launch_chunk<32>(a, stream);
        case 64: return launch_chunk<64>(a, stream);
        case 128: return launch_chunk<128>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kda
