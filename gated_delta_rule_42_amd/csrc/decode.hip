// decode.hip -- KDA recurrent decode: one token per (row, head), state in place.
//
// Page "[Feature][KDA] Add Kimi K3 KDA execution", KDA execution step 4
// (decode calls the recurrent operator) and Metadata construction (a one-token
// request with an existing state is decode); page "[KK] Prepare B12X Kimi KDA
// prefill ...", Behavior (states read and written in place at their pool
// slot, no gather/scatter).
//
// Per (row b, head h), with S the d_k x d_v state at pool[slot_b, h]:
//     S~ = Diag(exp g) S                  decay the key-channel rows
//     u  = S~^T k,  w = S~^T q,  kq = k.q
//     d  = beta (v - u)
//     S' = S~ + k d^T                     = (I - beta k k^T) S~ + beta k v^T
//     o  = scale S'^T q = scale (w + d kq)
// The step is HBM-bound (0.87 flop per state byte): each workgroup streams
// one head's state through registers exactly once -- read, update, write back
// to the same address -- with every load of the state issued before any
// arithmetic so the whole 64 KiB (fp32, d = 128) is in flight at once.  The
// state stream uses nontemporal loads and stores (touched once per step).
//
// Thread layout: TPR threads cover one state row (4 columns each, 16 B fp32 /
// 8 B bf16 vectors); RG row groups; thread (rg, c) owns rows rg, rg+RG, ...
// A wave therefore reads 64/TPR whole adjacent rows per instruction.  The two
// column reductions (u, w) are summed inside each thread over its rows, then
// across row groups through LDS in a fixed order (deterministic).

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

template <int DK, int DV>
struct DecodeShape {
    static constexpr int CPT = 4;                                    // columns per thread
    static constexpr int TPR = DV / CPT;                             // threads per row
    static constexpr int RG = (DK < 1024 / TPR) ? DK : 1024 / TPR;   // row groups
    static constexpr int NT = TPR * RG;                              // block size
    static constexpr int RPT = DK / RG;                              // rows per thread
    static_assert(CPT == 4, "each thread moves one 4-column vector per row");
    static_assert(DV % CPT == 0 && DK % RG == 0 && NT % kWave == 0, "decode shape");
};

// One workgroup per (row b, head h).  The state is read from pool[slot_b]
// once and kept in registers while the row's ntok tokens (rows b*ntok + t of
// the token arrays) are applied in order.  After token t the state goes to
// dst + t * dst_step, where dst is the pool slot itself for decode (ntok = 1,
// update in place) and the row's token-state buffer for speculative decode
// (the pool is then only read).
template <int DK, int DV, typename AT, typename ST>
__global__ __launch_bounds__((DecodeShape<DK, DV>::NT))
void kda_decode_kernel(const AT* __restrict__ q, const AT* __restrict__ k,
                       const AT* __restrict__ v, int64_t qs, int64_t ks, int64_t vs,
                       const float* __restrict__ g, const float* __restrict__ beta,
                       int heads, int ntok, ST* __restrict__ pool, int64_t num_slots,
                       const int32_t* __restrict__ slots, ST* __restrict__ token_states,
                       float scale, uint32_t flags, AT* __restrict__ out, int64_t os)
{
    using Sh = DecodeShape<DK, DV>;
    __shared__ float s_q[DK], s_k[DK], s_a[DK];
    __shared__ float s_u[Sh::RG][DV], s_w[Sh::RG][DV], s_kq[Sh::RG];
    __shared__ float s_ut[DV], s_wt[DV], s_kqt;
    __shared__ float s_norm[2];

    const int b = blockIdx.x / heads, h = blockIdx.x % heads;
    const int tid = threadIdx.x;
    const int c0 = (tid % Sh::TPR) * Sh::CPT;
    const int rg = tid / Sh::TPR;

    const int slot = slots[b];
    if (slot < 0) {                                    // graph padding: zero output
        for (int t = 0; t < ntok; ++t) {
            AT* ob = out + ((int64_t)b * ntok + t) * os + (int64_t)h * DV;
            for (int c = tid; c < DV; c += Sh::NT) ob[c] = from_f32<AT>(0.0f);
        }
        return;
    }
    if (slot >= num_slots) return;                     // contract violation: touch nothing

    // Issue the state loads first: they are the whole cost of a decode step.
    ST* S = pool + ((int64_t)slot * heads + h) * (int64_t)(DK * DV);
    ST* dst = S;
    int64_t dst_step = 0;
    if (token_states) {
        dst = token_states + ((int64_t)b * ntok * heads + h) * (int64_t)(DK * DV);
        dst_step = (int64_t)heads * DK * DV;
    }
    float s[Sh::RPT][4];
#pragma unroll
    for (int i = 0; i < Sh::RPT; ++i) load4_stream(S + (int64_t)(rg + i * Sh::RG) * DV + c0, s[i]);

    for (int t = 0; t < ntok; ++t) {
        const int64_t row = (int64_t)b * ntok + t;
        const int64_t bh = row * heads + h;
        for (int i = tid; i < DK; i += Sh::NT) {
            s_q[i] = to_f32(q[row * qs + (int64_t)h * DK + i]);
            s_k[i] = to_f32(k[row * ks + (int64_t)h * DK + i]);
            s_a[i] = __expf(g[bh * DK + i]);
        }
        float vv[4];
        load4(v + row * vs + (int64_t)h * DV + c0, vv);
        const float bt = beta[bh];
        __syncthreads();

        if (flags & KDA_FLAG_QK_L2NORM) {
            if (tid < kWave) {
                float sq = 0.0f, sk = 0.0f;
                for (int i = tid; i < DK; i += kWave) { sq += s_q[i] * s_q[i]; sk += s_k[i] * s_k[i]; }
                sq = wave_sum(sq);
                sk = wave_sum(sk);
                if (tid == 0) { s_norm[0] = 1.0f / sqrtf(sq + 1e-6f); s_norm[1] = 1.0f / sqrtf(sk + 1e-6f); }
            }
            __syncthreads();
            const float rq = s_norm[0], rk = s_norm[1];
            __syncthreads();
            for (int i = tid; i < DK; i += Sh::NT) { s_q[i] *= rq; s_k[i] *= rk; }
            __syncthreads();
        }

        float u[4] = {0.f, 0.f, 0.f, 0.f}, w[4] = {0.f, 0.f, 0.f, 0.f}, kq = 0.0f;
#pragma unroll
        for (int i = 0; i < Sh::RPT; ++i) {
            const int r = rg + i * Sh::RG;
            const float a = s_a[r], kr = s_k[r], qr = s_q[r];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                s[i][c] *= a;
                u[c] += kr * s[i][c];
                w[c] += qr * s[i][c];
            }
            kq += kr * qr;
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) { s_u[rg][c0 + c] = u[c]; s_w[rg][c0 + c] = w[c]; }
        if (c0 == 0) s_kq[rg] = kq;
        __syncthreads();

        // Column totals over the row groups, each summed once (fixed order).
        for (int i = tid; i < 2 * DV + 1; i += Sh::NT) {
            float acc = 0.0f;
            if (i < DV) {
#pragma unroll
                for (int gi = 0; gi < Sh::RG; ++gi) acc += s_u[gi][i];
                s_ut[i] = acc;
            } else if (i < 2 * DV) {
#pragma unroll
                for (int gi = 0; gi < Sh::RG; ++gi) acc += s_w[gi][i - DV];
                s_wt[i - DV] = acc;
            } else {
#pragma unroll
                for (int gi = 0; gi < Sh::RG; ++gi) acc += s_kq[gi];
                s_kqt = acc;
            }
        }
        __syncthreads();

        float d[4], o[4];
        const float kqt = s_kqt;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            d[c] = bt * (vv[c] - s_ut[c0 + c]);
            o[c] = scale * (s_wt[c0 + c] + d[c] * kqt);
        }
        if (rg == 0) {
            AT* ob = out + row * os + (int64_t)h * DV;
#pragma unroll
            for (int c = 0; c < 4; ++c) ob[c0 + c] = from_f32<AT>(o[c]);
        }
        ST* St = dst + t * dst_step;
#pragma unroll
        for (int i = 0; i < Sh::RPT; ++i) {
            const int r = rg + i * Sh::RG;
            const float kr = s_k[r];
#pragma unroll
            for (int c = 0; c < 4; ++c) s[i][c] += kr * d[c];
            store4_stream(St + (int64_t)r * DV + c0, s[i]);
        }
        if (t + 1 < ntok) __syncthreads();             // LDS is reused by the next token
    }
}

// Commit of a speculative step: pool[slot_b] = token_states[b, n_b - 1] for
// 0 < n_b <= ntok.  One workgroup per (row, head), a streaming copy.
// 1024 threads, each with all its vectors' loads in flight before it stores
// any: 512 rows x 16 heads of 128 x 128 fp32 states commit in 148.8 us on
// MI355X (155 us with one load in flight per thread; 166 us with 256
// threads, 159 with 512).
constexpr int kCommitThreads = 1024;
constexpr int kCommitUnroll = 4;

template <typename ST>
__global__ __launch_bounds__(kCommitThreads)
void kda_spec_commit_kernel(const ST* __restrict__ token_states, int heads, int ntok, int64_t elems,
                            const int32_t* __restrict__ accepted, ST* __restrict__ pool,
                            int64_t num_slots, const int32_t* __restrict__ slots)
{
    const int b = blockIdx.x / heads, h = blockIdx.x % heads;
    const int slot = slots[b];
    const int n = accepted[b];
    if (slot < 0 || slot >= num_slots || n <= 0 || n > ntok) return;
    const ST* src = token_states + (((int64_t)b * ntok + n - 1) * heads + h) * elems;
    ST* dstp = pool + ((int64_t)slot * heads + h) * elems;
    // kCommitUnroll vectors per thread in flight before any is stored.
    constexpr int64_t kStep = 4 * (int64_t)kCommitThreads;
    for (int64_t i0 = 4 * (int64_t)threadIdx.x; i0 < elems; i0 += kStep * kCommitUnroll) {
        float x[kCommitUnroll][4];
#pragma unroll
        for (int u = 0; u < kCommitUnroll; ++u)
            if (i0 + u * kStep < elems) load4_stream(src + i0 + u * kStep, x[u]);
#pragma unroll
        for (int u = 0; u < kCommitUnroll; ++u)
            if (i0 + u * kStep < elems) store4_stream(dstp + i0 + u * kStep, x[u]);
    }
}

template <int D, typename AT, typename ST>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t stream)
{
    using Sh = DecodeShape<D, D>;
    dim3 grid((unsigned)((int64_t)a.batch * a.heads)), block(Sh::NT);
    hipLaunchKernelGGL((kda_decode_kernel<D, D, AT, ST>), grid, block, 0, stream,
                       static_cast<const AT*>(a.q), static_cast<const AT*>(a.k),
                       static_cast<const AT*>(a.v), a.q_stride, a.k_stride, a.v_stride,
                       a.g, a.beta, a.heads, a.ntok, static_cast<ST*>(a.pool), a.num_slots,
                       a.slots, static_cast<ST*>(a.token_states), a.scale, a.flags,
                       static_cast<AT*>(a.out), a.out_stride);
    return hipGetLastError();
}

template <int D>
hipError_t launch_dim(const DecodeArgs& a, hipStream_t stream)
{
    if (a.act == KDA_BF16)
        return a.state == KDA_BF16 ? launch_typed<D, bf16, bf16>(a, stream)
                                   : launch_typed<D, bf16, float>(a, stream);
    return a.state == KDA_BF16 ? launch_typed<D, float, bf16>(a, stream)
                               : launch_typed<D, float, float>(a, stream);
}

}  // namespace

hipError_t launch_spec_commit(const SpecCommitArgs& a, hipStream_t stream)
{
    const int64_t elems = (int64_t)a.dk * a.dv;
    dim3 grid((unsigned)((int64_t)a.batch * a.heads)), block(kCommitThreads);
    if (a.state == KDA_BF16)
        hipLaunchKernelGGL((kda_spec_commit_kernel<bf16>), grid, block, 0, stream,
                           static_cast<const bf16*>(a.token_states), a.heads, a.ntok, elems,
                           a.accepted, static_cast<bf16*>(a.pool), a.num_slots, a.slots);
    else
        hipLaunchKernelGGL((kda_spec_commit_kernel<float>), grid, block, 0, stream,
                           static_cast<const float*>(a.token_states), a.heads, a.ntok, elems,
                           a.accepted, static_cast<float*>(a.pool), a.num_slots, a.slots);
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream)
{
    switch (a.dk) {
        case 16: return launch_dim<16>(a, stream);
        case 32: return launch_dim<32>(a, stream);
        case 64: return launch_dim<64>(a, stream);
        case 128: return launch_dim<128>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kda
