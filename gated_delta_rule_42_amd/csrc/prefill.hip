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
// intra_kernel: everything in a chunk that does not depend on the state.
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
    constexpr int GP = D + 4;                // fp32 pitch of sG
    constexpr int MP = BT + 4;               // fp32 pitch of sM / sX
    constexpr int TP = BTP + 8;              // bf16 pitch of the transposed tiles

    __shared__ float sG[BT][GP];             // inclusive cumulative gate
    __shared__ float sM[BT][MP];             // strict_lower(Diag(beta) K~ K^T)
    __shared__ float sX[BT][MP];             // (I + M)^{-1}, lower triangular
    __shared__ __attribute__((aligned(16))) bf16 sKt[DKP][TP];   // K~^T
    __shared__ __attribute__((aligned(16))) bf16 sVt[D][TP];     // V^T
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

    auto qrow = [&](int r) { return q + (t0 + r) * qs + (int64_t)h * D; };
    auto krow = [&](int r) { return k + (t0 + r) * ks + (int64_t)h * D; };

    // 1. Cumulative gate: NSPLIT threads per channel scan consecutive row
    //    segments, then each segment adds the totals of the segments before it.
    {
        constexpr int NSPLIT = kThreads / D;
        constexpr int RP = BT / NSPLIT;
        static_assert(RP >= 1 && BT % NSPLIT == 0, "gate split");
        const int c = tid % D, part = tid / D;
        float acc = 0.0f;
        for (int i = 0; i < RP; ++i) {
            const int r = part * RP + i;
            const float gv = r < len ? g[((t0 + r) * heads + h) * D + c] : 0.0f;
            acc += gv;
            sG[r][c] = acc;
        }
        __syncthreads();
        float pre = 0.0f;
        for (int p = 0; p < part; ++p) pre += sG[(p + 1) * RP - 1][c];
        __syncthreads();
        if (part > 0)
            for (int i = 0; i < RP; ++i) sG[part * RP + i][c] += pre;
    }

    // 2. Row norms (optional q/k L2 normalisation), beta, V^T.
    {
        constexpr int TPRN = kThreads / BT;          // threads per row
        const int r = tid / TPRN, part = tid % TPRN;
        float sq = 0.0f, sk = 0.0f;
        if ((flags & KDA_FLAG_QK_L2NORM) && r < len) {
            for (int c = part * 8; c < D; c += TPRN * 8) {
                float a[8], b[8];
                load8(qrow(r) + c, a);
                load8(krow(r) + c, b);
#pragma unroll
                for (int e = 0; e < 8; ++e) { sq += a[e] * a[e]; sk += b[e] * b[e]; }
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
            sBeta[r] = r < len ? beta[(t0 + r) * heads + h] : 0.0f;
        }
        for (int idx = tid; idx < BTP * D; idx += kThreads) {
            const int rr = idx / D, c = idx % D;
            const float val = rr < len ? to_f32(v[(t0 + rr) * vs + (int64_t)h * D + c]) : 0.0f;
            sVt[c][rr] = static_cast<bf16>(val);
        }
    }
    __syncthreads();

    // 3. Elementwise factors: K~^T into LDS; Q~, Kb^T, e^{G_C} into the record.
    for (int idx = tid; idx < BTP * DKP; idx += kThreads) {
        const int r = idx / DKP, c = idx % DKP;
        float kt = 0.0f, qt = 0.0f, kb = 0.0f;
        if (r < len && c < D) {
            const float kv = to_f32(krow(r)[c]) * sRk[r];
            const float qv = to_f32(qrow(r)[c]) * sRq[r];
            const float eg = __expf(sG[r][c]);
            kt = kv * eg;
            qt = qv * eg;
            kb = kv * __expf(sG[BT - 1][c] - sG[r][c]);
        }
        sKt[c][r] = static_cast<bf16>(kt);
        wKb[(int64_t)c * BTP + r] = static_cast<bf16>(kb);
        if (r < BT) wQ[(int64_t)r * DKP + c] = static_cast<bf16>(qt);
    }
    for (int c = tid; c < DKP; c += kThreads) wEg[c] = c < D ? __expf(sG[BT - 1][c]) : 0.0f;
    // Zero the blocks above the diagonal of M, X and Aqk (and Aqk's padding).
    for (int idx = tid; idx < BT * BTP; idx += kThreads) {
        const int r = idx / BTP, s = idx % BTP;
        if (s >= 16 * (r / 16 + 1)) {
            if (s < BT) { sM[r][s] = 0.0f; sX[r][s] = 0.0f; }
            wA[(int64_t)r * BTP + s] = static_cast<bf16>(0.0f);
        }
    }

    // 4. Gram blocks (i, j <= i) on bf16 MFMA, K = key dim.  Wave w owns
    //    block row i = w.  Reference point: the token before sub-chunk i.
    if (wave < NS) {
        const int i = wave;
        const int r = 16 * i + l16;
        bf16x8 aK[P::NKK_K], aQ[P::NKK_K];
#pragma unroll
        for (int kk = 0; kk < P::NKK_K; ++kk) {
            const int c0 = 32 * kk + 8 * g4;
            float fk[8] = {}, fq[8] = {};
            if (r < len && c0 < D) {
                load8(krow(r) + c0, fk);
                load8(qrow(r) + c0, fq);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float gb = i > 0 ? sG[16 * i - 1][c0 + e] : 0.0f;
                    const float ex = __expf(sG[r][c0 + e] - gb);
                    fk[e] *= sRk[r] * ex;
                    fq[e] *= sRq[r] * ex;
                }
            }
            aK[kk] = pack_bf16x8(fk);
            aQ[kk] = pack_bf16x8(fq);
        }
        for (int j = 0; j <= i; ++j) {
            const int s = 16 * j + l16;
            f32x4 accK = {0.f, 0.f, 0.f, 0.f}, accQ = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < P::NKK_K; ++kk) {
                const int c0 = 32 * kk + 8 * g4;
                float fb[8] = {};
                if (s < len && c0 < D) {
                    load8(krow(s) + c0, fb);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float gb = i > 0 ? sG[16 * i - 1][c0 + e] : 0.0f;
                        fb[e] *= sRk[s] * __expf(gb - sG[s][c0 + e]);
                    }
                }
                const bf16x8 b = pack_bf16x8(fb);
                accK = mfma16x16x32(aK[kk], b, accK);
                accQ = mfma16x16x32(aQ[kk], b, accQ);
            }
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int rr = 16 * i + 4 * g4 + ii, ss = 16 * j + l16;
                sM[rr][ss] = ss < rr ? sBeta[rr] * accK[ii] : 0.0f;
                wA[(int64_t)rr * BTP + ss] = static_cast<bf16>(ss <= rr ? accQ[ii] : 0.0f);
            }
        }
    }
    __syncthreads();

    // 5a. Diagonal blocks of X = (I + M)^{-1}: forward substitution, one wave
    //     per block, one lane per column.
    if (wave < NS && l16 == lane) {
        const int i = wave, b0 = 16 * i;
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

    // 5b. Off-diagonal blocks, row by row:  X_ij = -X_ii sum_{j<=m<i} M_im X_mj,
    //     on fp32 MFMA.  Wave j computes block (i, j).
    for (int i = 1; i < NS; ++i) {
        if (wave < i) {
            const int j = wave;
            f32x4 y = {0.f, 0.f, 0.f, 0.f};
            for (int m = j; m < i; ++m) {
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const float a = sM[16 * i + l16][16 * m + 4 * kk + g4];
                    const float b = sX[16 * m + 4 * kk + g4][16 * j + l16];
                    y = mfma16x16x4f32(a, b, y);
                }
            }
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) sTmp[wave][4 * g4 + ii][l16] = y[ii];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const float a = sX[16 * i + l16][16 * i + 4 * kk + g4];
                const float b = sTmp[wave][4 * kk + g4][l16];
                z = mfma16x16x4f32(a, b, z);
            }
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) sX[16 * i + 4 * g4 + ii][16 * j + l16] = -z[ii];
        }
        __syncthreads();
    }

    // 6. W = T K~ and U = T V with T = X Diag(beta), on bf16 MFMA (K = tokens,
    //    only up to the diagonal).  Tiles are dealt round-robin to the waves.
    {
        constexpr int NTW = NS * (DKP / 16), NTU = NS * (D / 16);
        for (int t = wave; t < NTW + NTU; t += 4) {
            const bool isW = t < NTW;
            const int tt = isW ? t : t - NTW;
            const int nt_count = isW ? DKP / 16 : D / 16;
            const int mt = tt / nt_count, nt = tt % nt_count;
            const int kmax = (16 * mt + 15) / 32;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int kk = 0; kk <= kmax; ++kk) {
                const int s0 = 32 * kk + 8 * g4;
                float fa[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int s = s0 + e;
                    fa[e] = s < BT ? sX[16 * mt + l16][s] * sBeta[s] : 0.0f;
                }
                const bf16x8 a = pack_bf16x8(fa);
                const bf16x8 b = isW ? *reinterpret_cast<const bf16x8*>(&sKt[16 * nt + l16][s0])
                                     : *reinterpret_cast<const bf16x8*>(&sVt[16 * nt + l16][s0]);
                acc = mfma16x16x32(a, b, acc);
            }
            if (isW) {
#pragma unroll
                for (int ii = 0; ii < 4; ++ii)
                    wW[(int64_t)(16 * mt + 4 * g4 + ii) * DKP + 16 * nt + l16] =
                        static_cast<bf16>(acc[ii]);
            } else {
                bf16x4 u4;
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) u4[ii] = static_cast<bf16>(acc[ii]);
                *reinterpret_cast<bf16x4*>(&wU[(int64_t)(16 * nt + l16) * BTP + 16 * mt + 4 * g4]) = u4;
            }
        }
        // Token padding of U^T (only when the chunk is shorter than a K step).
        if (BTP > BT)
            for (int idx = tid; idx < D * (BTP - BT); idx += kThreads)
                wU[(int64_t)(idx / (BTP - BT)) * BTP + BT + idx % (BTP - BT)] = static_cast<bf16>(0.0f);
    }
}

// ---------------------------------------------------------------------------
// chain_kernel: the state-dependent part, serial over a sequence's chunks.
template <int D, int BT, typename AT, typename ST>
__global__ __launch_bounds__(kThreads)
void chain_kernel(const int32_t* __restrict__ cu, int n_seqs, int heads,
                  ST* __restrict__ pool, int64_t num_slots, const int32_t* __restrict__ slots,
                  const uint8_t* __restrict__ has_init, ST* __restrict__ ckpt, int64_t ckpt_cap,
                  int interval, float scale, AT* __restrict__ out, int64_t os,
                  const uint8_t* __restrict__ ws)
{
    using P = Shape<D, BT>;
    constexpr int DKP = P::DKP, BTP = P::BTP, NS = P::NS;
    constexpr int NKT_W = (P::NMT_K + 3) / 4;     // key m-tiles per wave
    constexpr int SP = DKP + 8, DP = BTP + 8;     // bf16 pitches

    __shared__ __attribute__((aligned(16))) bf16 sS[16][SP];   // bf16 S^T of this column tile
    __shared__ __attribute__((aligned(16))) bf16 sD[16][DP];   // bf16 D^T of this column tile

    const int seq = blockIdx.x, h = blockIdx.y, n0 = blockIdx.z * 16;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int col = n0 + l16;

    const int64_t s_begin = cu[seq];
    const int len = max(0, cu[seq + 1] - cu[seq]);
    const int slot = slots[seq];
    if (slot < 0) {                                // graph padding: zero output rows
        for (int idx = tid; idx < len * 16; idx += kThreads)
            out[(s_begin + idx / 16) * os + (int64_t)h * D + n0 + idx % 16] = from_f32<AT>(0.0f);
        return;
    }
    if (len == 0 || slot >= num_slots) return;

    int chunk_base = 0;
    int64_t ckpt_base = 0;
    sequence_bases(cu, seq, BT, interval, lane, chunk_base, ckpt_base);
    const int nch = num_chunks(len, BT);
    const bool init = has_init ? has_init[seq] != 0 : true;
    ST* home = pool + ((int64_t)slot * heads + h) * (int64_t)(D * D);

    // S rows 16*kt + 4*g4 + ii (kt = wave + 4*j), column col, in fp32.
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
            *reinterpret_cast<bf16x4*>(&sS[l16][16 * kt + 4 * g4]) = s4;
        }
    }
    __syncthreads();

    for (int lc = 0; lc < nch; ++lc) {
        const uint8_t* rec = ws + ((int64_t)(chunk_base + lc) * heads + h) * P::REC_BYTES;
        const bf16* wQ = reinterpret_cast<const bf16*>(rec) + P::OFF_Q;
        const bf16* wW = reinterpret_cast<const bf16*>(rec) + P::OFF_W;
        const bf16* wKb = reinterpret_cast<const bf16*>(rec) + P::OFF_KB;
        const bf16* wU = reinterpret_cast<const bf16*>(rec) + P::OFF_U;
        const bf16* wA = reinterpret_cast<const bf16*>(rec) + P::OFF_A;
        const float* wEg = reinterpret_cast<const float*>(rec + P::EG_BYTE_OFF);
        const int64_t tc = s_begin + (int64_t)lc * BT;
        const int clen = min(BT, len - lc * BT);

        // D = U - W S and Q~ S for token tile `wave`.
        f32x4 accO = {0.f, 0.f, 0.f, 0.f};
        if (wave < NS) {
            f32x4 accW = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < P::NKK_K; ++kk) {
                const bf16x8 b = *reinterpret_cast<const bf16x8*>(&sS[l16][32 * kk + 8 * g4]);
                const int64_t ao = (int64_t)(16 * wave + l16) * DKP + 32 * kk + 8 * g4;
                accW = mfma16x16x32(*reinterpret_cast<const bf16x8*>(wW + ao), b, accW);
                accO = mfma16x16x32(*reinterpret_cast<const bf16x8*>(wQ + ao), b, accO);
            }
            const bf16x4 u4 = *reinterpret_cast<const bf16x4*>(wU + (int64_t)col * BTP + 16 * wave + 4 * g4);
            bf16x4 d4;
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) d4[ii] = static_cast<bf16>(static_cast<float>(u4[ii]) - accW[ii]);
            *reinterpret_cast<bf16x4*>(&sD[l16][16 * wave + 4 * g4]) = d4;
        }
        if (BTP > BT && wave == 0 && g4 * 4 + 4 <= BTP - BT) {
            bf16x4 z4 = {};
            *reinterpret_cast<bf16x4*>(&sD[l16][BT + 4 * g4]) = z4;
        }
        __syncthreads();

        // O = scale (Q~ S + Aqk D) for token tile `wave`.
        if (wave < NS) {
            const int kmax = (16 * wave + 15) / 32;
            for (int kk = 0; kk <= kmax; ++kk) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(
                    wA + (int64_t)(16 * wave + l16) * BTP + 32 * kk + 8 * g4);
                const bf16x8 b = *reinterpret_cast<const bf16x8*>(&sD[l16][32 * kk + 8 * g4]);
                accO = mfma16x16x32(a, b, accO);
            }
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int r = 16 * wave + 4 * g4 + ii;
                if (r < clen) out[(tc + r) * os + (int64_t)h * D + col] = from_f32<AT>(scale * accO[ii]);
            }
        }

        // S <- Diag(e^{G_C}) S + Kb^T D for key tiles wave, wave + 4, ...
#pragma unroll
        for (int j = 0; j < NKT_W; ++j) {
            const int kt = wave + 4 * j;
            if (kt >= P::NMT_K) continue;
            f32x4 acc;
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) acc[ii] = S[j][ii] * wEg[16 * kt + 4 * g4 + ii];
#pragma unroll
            for (int kk = 0; kk < P::NKK_T; ++kk) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(
                    wKb + (int64_t)(16 * kt + l16) * BTP + 32 * kk + 8 * g4);
                const bf16x8 b = *reinterpret_cast<const bf16x8*>(&sD[l16][32 * kk + 8 * g4]);
                acc = mfma16x16x32(a, b, acc);
            }
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) S[j][ii] = acc[ii];
        }

        // Checkpoint at this chunk's end if it is a multiple of the interval.
        const int pos = (lc + 1) * BT;
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

        // Publish bf16 S for the next chunk.
#pragma unroll
        for (int j = 0; j < NKT_W; ++j) {
            const int kt = wave + 4 * j;
            if (kt >= P::NMT_K) continue;
            bf16x4 s4;
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) s4[ii] = static_cast<bf16>(S[j][ii]);
            *reinterpret_cast<bf16x4*>(&sS[l16][16 * kt + 4 * g4]) = s4;
        }
        __syncthreads();
    }

    // Final state, in place.
#pragma unroll
    for (int j = 0; j < NKT_W; ++j) {
        const int kt = wave + 4 * j;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int rr = 16 * kt + 4 * g4 + ii;
            if (kt < P::NMT_K && rr < D) home[(int64_t)rr * D + col] = from_f32<ST>(S[j][ii]);
        }
    }
}

// ---------------------------------------------------------------------------
template <int D, int BT, typename AT, typename ST>
hipError_t launch_typed(const PrefillArgs& a, hipStream_t stream)
{
    const int64_t chunks = max_chunks(a.num_seqs, a.total_tokens, BT);
    if (chunks > INT32_MAX) return hipErrorInvalidValue;
    if (a.total_tokens > 0) {
        hipLaunchKernelGGL((intra_kernel<D, BT, AT>), dim3((unsigned)chunks, (unsigned)a.heads),
                           dim3(kThreads), 0, stream, static_cast<const AT*>(a.q),
                           static_cast<const AT*>(a.k), static_cast<const AT*>(a.v), a.q_stride,
                           a.k_stride, a.v_stride, a.g, a.beta, a.cu_seqlens, a.num_seqs, a.heads,
                           a.slots, a.flags, static_cast<uint8_t*>(a.workspace));
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((chain_kernel<D, BT, AT, ST>),
                       dim3((unsigned)a.num_seqs, (unsigned)a.heads, (unsigned)(D / 16)),
                       dim3(kThreads), 0, stream, a.cu_seqlens, a.num_seqs, a.heads,
                       static_cast<ST*>(a.pool), a.num_slots, a.slots, a.has_init,
                       static_cast<ST*>(a.ckpt), a.ckpt_capacity, a.ckpt_interval, a.scale,
                       static_cast<AT*>(a.out), a.out_stride,
                       static_cast<const uint8_t*>(a.workspace));
    return hipGetLastError();
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
