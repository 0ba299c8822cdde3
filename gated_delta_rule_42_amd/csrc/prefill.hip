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
//                 accumulators.  Its waves split the token rows of D and O
//                 and the key rows of S; D and a bf16 copy of S are shared
//                 through LDS (two barriers per chunk).  Reads S0 from
//                 pool[slot], writes checkpoints and the final state in place.
//
// Range of the decay factors.  Products e^{G_r - G_s} (r >= s) are at most 1,
// but the factors e^{-G_s} alone overflow fp32 for long strong decays, so the
// Gram products are formed per 16-token sub-chunk i with the reference point
// b_i = the token before the sub-chunk:  (e^{G_r - G_b} q_r) . (e^{G_b - G_s} k_s).
// Off-diagonal blocks have both factors <= 1; diagonal blocks grow at most by
// the decay accumulated inside one sub-chunk, which must stay above e^{-80}.

#include <algorithm>
#include <type_traits>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kThreads = 256;   // four waves per workgroup
// Largest total log-decay of one chunk (per channel) for which the Gram
// products use the chunk start as the only reference point: e^{80} and
// e^{-80} are far inside the fp32 / bf16 range.
constexpr float kMaxLogDecay = 80.0f;
// Bound on a wave's wait for another wave of its workgroup (that wave writes
// within a few hundred cycles; the bound only keeps every wait finite).
constexpr int kMaxRowWait = 1 << 20;
// The workspace starts with a header whose first word is the call's status:
// a bounded wait that ran out sets a bit in it (its results are then NaN, not
// stale values), and the host reads it back on request.  The kernels get the
// rest of the workspace, past the header.
constexpr int64_t kHeaderBytes = 256;
constexpr uint32_t kStatusTimeout = 1u;     // a bounded wait ran out
constexpr uint32_t kStatusPlacement = 2u;   // the two workgroups of a tile ran on different XCDs
__device__ __forceinline__ void raise_status(uint32_t* status, uint32_t bits)
{
    __hip_atomic_fetch_or(status, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

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
    // Aqk keeps only the columns its products read: token tile t stores
    // columns 0 .. aq_width(t) - 1 (the 32-wide K steps up to its diagonal
    // block), tiles one after another.
    static constexpr int aq_width(int t) { return 32 * ((16 * t + 15) / 32 + 1); }
    static constexpr int aq_base(int t)
    {
        int b = 0;
        for (int i = 0; i < t; ++i) b += 16 * aq_width(i);
        return b;
    }
    static constexpr int AQ_ELEMS = aq_base(NS);
    static constexpr int64_t REC_BYTES = ((EG_BYTE_OFF + DKP * 4) + 255) / 256 * 256;
    static_assert(BT % 16 == 0 && BT <= 64, "chunk size");
    static_assert(D % 16 == 0 && D <= 128, "head dim");
};

// Upper bound on the chunks of a call: with absolute start positions a
// sequence of L tokens spans at most floor(L / chunk) + 2 chunks (a partial
// one at each end).
int64_t max_chunks(int32_t num_seqs, int64_t total_tokens, int32_t chunk)
{
    return (total_tokens + chunk - 1) / chunk + 2 * (int64_t)num_seqs;
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

// Chunk geometry.  Chunk boundaries fall on absolute multiples of bt: a
// sequence whose first token sits at absolute position p0 (tokens processed
// before this call; 0 without positions) has a first chunk of bt - p0 % bt
// tokens, then full chunks, then a partial one.  off = p0 % bt; negative
// positions count as 0.
__device__ __forceinline__ int64_t start_pos(const int64_t* __restrict__ pos, int i)
{
    return pos ? max<int64_t>(pos[i], 0) : 0;
}
__device__ __forceinline__ int num_chunks(int len, int bt, int off)
{
    return len > 0 ? (len + off + bt - 1) / bt : 0;
}
__device__ __forceinline__ int chunk_begin(int c, int bt, int off) { return c == 0 ? 0 : c * bt - off; }
__device__ __forceinline__ int chunk_end(int c, int len, int bt, int off) { return min(len, (c + 1) * bt - off); }

// The sequence that owns global chunk x (chunks numbered sequence by sequence)
// and the index of that sequence's first chunk.  Whole-wave call; false if x
// is past the last chunk.
__device__ bool locate_chunk(const int32_t* __restrict__ cu, const int64_t* __restrict__ pos, int n,
                             int bt, int x, int lane, int& seq, int& first)
{
    int base = 0;
    for (int i0 = 0; i0 < n; i0 += kWave) {
        const int i = i0 + lane;
        const int nch = i < n ? num_chunks(cu[i + 1] - cu[i], bt, (int)(start_pos(pos, i) % bt)) : 0;
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
// checkpoint count (the multiples of the interval in (p0, p0 + len]).
// Whole-wave call.
__device__ void sequence_bases(const int32_t* __restrict__ cu, const int64_t* __restrict__ pos, int seq,
                               int bt, int interval, int lane, int& chunk_base, int64_t& ckpt_base)
{
    int cb = 0;
    int64_t kb = 0;
    for (int i0 = 0; i0 < seq; i0 += kWave) {
        const int i = i0 + lane;
        int nch = 0;
        int64_t nck = 0;
        if (i < seq) {
            const int len = cu[i + 1] - cu[i];
            const int64_t p0 = start_pos(pos, i);
            nch = num_chunks(len, bt, (int)(p0 % bt));
            nck = (interval > 0 && len > 0) ? (p0 + len) / interval - p0 / interval : 0;
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

// Element offset of (row, col) in a record tile with COLS columns stored as
// MFMA operand fragments: the 16 x 32 block (row / 16, col / 32) is
// fragment row / 16 * COLS / 32 + col / 32, 512 elements long, and lane
// l = row % 16 + 16 ((col % 32) / 8) of it holds the 8 elements of that row
// from column col & ~7 at element 8 l.  The wave that reads a 16 x 32
// operand block of the tile then reads 1 KB of consecutive bytes.
template <int COLS>
__device__ __forceinline__ int frag(int row, int col)
{
    static_assert(COLS % 32 == 0, "fragment columns");
    return (((row >> 4) * (COLS / 32) + (col >> 5)) * 64 + (row & 15) + 16 * ((col >> 3) & 3)) * 8 + (col & 7);
}

// Element offset of (row r, col) in the compact Aqk tile (aq_width above):
// token tile t = r / 16 keeps its aq_width(t) / 32 fragments, laid out as in
// frag, after those of the tiles before it.
__device__ __forceinline__ int aq_frag(int r, int col)
{
    const int t = r >> 4;
    const int base = t == 0 ? 0 : t == 1 ? 512 : t == 2 ? 1024 : 2048;
    return base + ((col >> 5) * 64 + (r & 15) + 16 * ((col >> 3) & 3)) * 8 + (col & 7);
}

// ---------------------------------------------------------------------------
// Lane-level helpers for the MFMA operand layouts (16x16x32 bf16): an
// "A fragment" of a 16-row tile holds, in lane l, row l % 16 and the 8
// consecutive K-elements 8 * (l / 16) .. + 7 of one 32-wide K block.

// Inclusive prefix sum over the 16 lanes of each DPP row (lanes 16r..16r+15).
template <int N>
__device__ __forceinline__ float dpp_row_shr(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        0, __builtin_bit_cast(int, x), 0x110 + N, 0xf, 0xf, true));
}
// Lane QL of each group of four lanes, broadcast to the group.
template <int QL>
__device__ __forceinline__ float quad_bcast(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(
        __builtin_bit_cast(int, x), QL * 0x55, 0xf, 0xf, false));
}
__device__ __forceinline__ float row_scan16(float x)
{
    x += dpp_row_shr<1>(x);
    x += dpp_row_shr<2>(x);
    x += dpp_row_shr<4>(x);
    x += dpp_row_shr<8>(x);
    return x;
}

// B operands of the identity products that transpose an A fragment: with
// B = E_half (the 32x16 matrix with ones at (n + 16 * half, n)), the product
// A[16x32] * E_half is columns 16*half .. 16*half+15 of A, returned in the
// accumulator layout (lane l: column l % 16, rows 4 * (l / 16) .. + 3).  The
// products are exact: every output is one bf16 value times 1 plus zeros.
__device__ __forceinline__ bf16x8 identity_half(int half, int lane)
{
    const int e = (lane & 15) + 16 * half - 8 * (lane >> 4);
    bf16x8 b;
#pragma unroll
    for (int i = 0; i < 8; ++i) b[i] = static_cast<bf16>(i == e ? 1.0f : 0.0f);
    return b;
}

// ---------------------------------------------------------------------------
// intra_kernel: everything in a chunk that does not depend on the state.
//
// Wave w < NS owns token tile w (tokens 16w .. 16w+15).  Each lane keeps one
// token's q, k, v, g as A fragments (8 consecutive channels per 32-channel
// block) for the whole kernel, so the elementwise work happens in registers:
//   1. gate cumsum: a DPP scan over the tile's 16 lanes, plus the totals of
//      the tiles before (LDS).
//   2. decay factors relative to the tile's reference point b_w (the token
//      before the tile): f_w = e^{G_r - G_{b_w}} <= 1, and for earlier
//      reference points f_j = f_w * prod_{j<=m<w} e^{tile total m}, products
//      of factors <= 1 (no exponential of a positive number).  Q~ and K~ use
//      f_0; the Gram blocks (w, j) use f_j on this tile's rows and
//      K^_s = k_s e^{G_{b_j} - G_s} (written by wave j) on the other side.
//   3. Gram blocks on bf16 MFMA, computed transposed so each lane holds 4
//      consecutive columns of one row: M (to LDS, fp32) and Aqk (record).
//   4. X = (I + M)^{-1}: forward substitution on each 16x16 diagonal block
//      (one lane per column), then the off-diagonal blocks row by row on
//      fp32 MFMA.  T = X Diag(beta) in bf16.
//   5. W = T K~ and U = T V on bf16 MFMA from LDS tiles, K~^T and V^T having
//      been transposed with identity MFMA products in step 2.
// Record stores are 8- or 16-byte vector stores in the swizzled layout.

typedef int v2i32 __attribute__((ext_vector_type(2)));
typedef int v4i32 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
constexpr int kBufferRsrcWord3 = 0x00020000;       // raw 32-bit buffer descriptor
constexpr int kDeviceScope = 16;                   // cache policy: device scope (sc1)

// Stores into one record.  A record is written once, by its intra workgroup,
// and read by the chain kernel after the kernel boundary.  The stores are
// device-scope buffer stores: each goes through the XCD's L2 to the
// memory-side cache when it is made, so the intra kernel ends with no dirty
// record lines in L2 that the end of the kernel would first have to write
// back (the intra kernel takes 3 us less at T = 4096, H = 16, d = 128 than
// with write-back stores; the chain kernel is unchanged).
struct RecordOut {
    __amdgpu_buffer_rsrc_t rsrc;
    const uint8_t* base;
    __device__ RecordOut(uint8_t* rec, int bytes)
        : rsrc(__builtin_amdgcn_make_buffer_rsrc(rec, 0, bytes, kBufferRsrcWord3)), base(rec) {}
    __device__ int offset(const void* p) const { return (int)(reinterpret_cast<const uint8_t*>(p) - base); }
    __device__ void put(const void* p, bf16x4 v) const
    {
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2i32, v), rsrc, offset(p), 0, kDeviceScope);
    }
    __device__ void put(const void* p, bf16x8 v) const
    {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i32, v), rsrc, offset(p), 0, kDeviceScope);
    }
    __device__ void put(const void* p, float v) const
    {
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, v), rsrc, offset(p), 0, kDeviceScope);
    }
};
// Causal conv1d of the fused front end (the operation of kda_causal_conv1d on
// the packed [q | k | v] projection), evaluated where the intra kernel loads
// its activations.
template <typename AT>
struct ConvIn {
    const AT* w;            // [channels, width]
    const AT* b;            // [channels] or null
    AT* state;              // [num_slots, width - 1, channels] (row width - 2 = newest)
    const uint8_t* has_init;    // [num_seqs] or null (= all 1)
    int64_t num_slots;
    int64_t channels;       // 3 H d
    int width;              // 2 .. 8
    bool silu;
};

constexpr int kMaxConvWidth = 8;

// Eight consecutive activations as raw 32-bit words (bf16 pairs or fp32), the
// unit the conv front end moves between lanes.
template <typename AT>
struct Raw8 {
    static constexpr int N = 2 * (int)sizeof(AT);
    uint32_t u[N];
};

template <typename AT>
__device__ __forceinline__ Raw8<AT> load_raw8(const AT* p)
{
    Raw8<AT> r;
    const uint4* s = reinterpret_cast<const uint4*>(p);
#pragma unroll
    for (int i = 0; i < Raw8<AT>::N / 4; ++i) {
        const uint4 t = s[i];
        r.u[4 * i] = t.x; r.u[4 * i + 1] = t.y; r.u[4 * i + 2] = t.z; r.u[4 * i + 3] = t.w;
    }
    return r;
}

template <typename AT>
__device__ __forceinline__ void store_raw8(AT* p, const Raw8<AT>& r)
{
    uint4* d = reinterpret_cast<uint4*>(p);
#pragma unroll
    for (int i = 0; i < Raw8<AT>::N / 4; ++i)
        d[i] = make_uint4(r.u[4 * i], r.u[4 * i + 1], r.u[4 * i + 2], r.u[4 * i + 3]);
}

template <typename AT>
__device__ __forceinline__ Raw8<AT> zero_raw8()
{
    Raw8<AT> r;
#pragma unroll
    for (int i = 0; i < Raw8<AT>::N; ++i) r.u[i] = 0u;
    return r;
}

__device__ __forceinline__ void widen8(const Raw8<bf16>& r, float (&x)[8])
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(r.u[i] << 16);
        x[2 * i + 1] = __uint_as_float(r.u[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ void widen8(const Raw8<float>& r, float (&x)[8])
{
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = __uint_as_float(r.u[i]);
}

// The conv inputs of one 8-channel group for this lane's token row r: its own
// row (token tr) and, in lanes 17 - W .. 15 of each 16-lane row group, the row
// 16 tokens earlier (token tr - 16, which may precede the sequence and then
// comes from its conv state).  Tap m of lane l then reads row r - m from lane
// (l - m) mod 16 of a DPP row rotation: the own row of lane l - m when l >= m,
// else the early row of lane l + 16 - m, which is token tr - m as well.
template <typename AT>
struct ConvRows {
    Raw8<AT> own, early;
};

template <typename AT>
__device__ __forceinline__ void conv_fetch(ConvRows<AT>& cr, const AT* __restrict__ xp, int64_t xs,
                                           int64_t tr, bool own_ok, bool early_ok, int64_t s0,
                                           const AT* __restrict__ st_row0, int64_t channels,
                                           int width)
{
    cr.own = own_ok ? load_raw8(xp + tr * xs) : zero_raw8<AT>();
    cr.early = zero_raw8<AT>();
    if (early_ok) {
        const int64_t p = tr - 16;
        if (p >= s0)
            cr.early = load_raw8(xp + p * xs);
        else if (st_row0)                         // s0 - p is 1 .. width - 1 here
            cr.early = load_raw8(st_row0 + (int64_t)((width - 1) - (s0 - p)) * channels);
    }
}

// Element u of a 16-byte vector of AT (bf16 or fp32), widened to fp32 and
// stored to p (u a constant after unrolling).
__device__ __forceinline__ uint32_t vec_word(const uint4& v, int i)
{
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}
template <typename AT>
__device__ __forceinline__ void store_elem_f32(float* p, const uint4& v, int u)
{
    if constexpr (sizeof(AT) == 2)
        *p = __uint_as_float(((vec_word(v, u >> 1) >> (16 * (u & 1))) & 0xffffu) << 16);
    else
        *p = __uint_as_float(vec_word(v, u));
}

// Taps M, M - 1, .. 0 of the conv (tap m reads row r - m with weight
// W - 1 - m); taps at or past the width are skipped.  WC > 0 is the width
// known at compile time (no branches, so the weight reads of all taps are
// issued together); WC = 0 takes it from `width`.
template <int M, int D, int WC, typename AT>
__device__ __forceinline__ void conv_taps(float (&acc)[8], const ConvRows<AT>& cr, const float* wt,
                                          int width, int l16)
{
    const bool live = WC > 0 ? M <= WC - 1 : M <= width - 1;
    if (live) {
        const int W = WC > 0 ? WC : width;
        float xv[8], wv[8];
        if constexpr (M == 0) {
            widen8(cr.own, xv);
        } else {
            Raw8<AT> t;
            const bool early = l16 >= 16 - M;
#pragma unroll
            for (int i = 0; i < Raw8<AT>::N; ++i)
                t.u[i] = (uint32_t)__builtin_amdgcn_mov_dpp(
                    (int)(early ? cr.early.u[i] : cr.own.u[i]), 0x120 + M /* row_ror:M */, 0xF, 0xF,
                    false);
            widen8(t, xv);
        }
        load8(wt + (W - 1 - M) * D, wv);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += wv[i] * xv[i];
    }
    if constexpr (M > 0) conv_taps<M - 1, D, WC>(acc, cr, wt, width, l16);
}

// Conv output of the group: bias, then the taps from the oldest input (row
// r - (W-1)) to the current one, then SiLU, rounded to bf16 as the
// activations are.  The same operations in the same order as the conv kernel.
// wt: the group's tap-major weights in LDS, widened to fp32 (tap j at wt[j * D]).
template <int D, int WC, typename AT>
__device__ __forceinline__ bf16x8 conv_eval(const ConvRows<AT>& cr, const AT* bias, const float* wt,
                                            int width, bool silu, int l16)
{
    float acc[8];
    if (bias) {
        load8(bias, acc);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    }
    conv_taps<(WC > 0 ? WC : kMaxConvWidth) - 1, D, WC>(acc, cr, wt, width, l16);
    if (silu) {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = silu_f32(acc[i]);
    }
    return pack_bf16x8(acc);
}

template <int D, int BT, typename AT, bool CONV>
__global__ __launch_bounds__(kThreads, 2)
void intra_kernel(const AT* __restrict__ q, const AT* __restrict__ k, const AT* __restrict__ v,
                  int64_t qs, int64_t ks, int64_t vs, const float* __restrict__ g,
                  const float* __restrict__ beta, const int32_t* __restrict__ cu, int n_seqs,
                  int heads, const int32_t* __restrict__ slots, uint32_t flags,
                  const int64_t* __restrict__ pos, uint8_t* __restrict__ ws, int64_t flag_off,
                  int64_t n_flags, uint32_t* __restrict__ status, ConvIn<AT> cv)
{
    using P = Shape<D, BT>;
    constexpr int DKP = P::DKP, BTP = P::BTP, NS = P::NS, NKK = P::NKK_K;
    constexpr int XP = BT + 4;               // fp32 pitch of the X / M tiles
    constexpr int TP = BTP + 8;              // bf16 pitch of the token-contiguous tiles

    // LDS regions are reused once the phase that reads them has passed a
    // barrier, so that two workgroups fit on one CU:
    //   R1: K^ fragments (Gram)  ->  X^T (solve)  ->  K~^T (W)
    //   R2: M (solve)                             ->  V^T (U)
    constexpr int KH_BYTES = NS * NKK * kWave * 16;
    constexpr int XT_BYTES = BT * XP * 4;
    constexpr int KT_BYTES = DKP * TP * 2;
    constexpr int R1_BYTES = KH_BYTES > XT_BYTES ? (KH_BYTES > KT_BYTES ? KH_BYTES : KT_BYTES)
                                                 : (XT_BYTES > KT_BYTES ? XT_BYTES : KT_BYTES);
    constexpr int R2_BYTES = XT_BYTES > KT_BYTES ? XT_BYTES : KT_BYTES;
    __shared__ __attribute__((aligned(16))) uint8_t sR1[R1_BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t sR2[R2_BYTES];
    auto sKh = reinterpret_cast<bf16x8 (*)[NKK][kWave]>(sR1);            // [NS][NKK][64]
    auto sXt = reinterpret_cast<float (*)[XP]>(sR1);                     // X^T [BT][XP]
    auto sKt = reinterpret_cast<bf16 (*)[TP]>(sR1);                      // K~^T [DKP][TP]
    auto sM = reinterpret_cast<float (*)[XP]>(sR2);                      // M [BT][XP]
    auto sVt = reinterpret_cast<bf16 (*)[TP]>(sR2);                      // V^T [DKP][TP]
    __shared__ __attribute__((aligned(16))) float sXd[NS][16][20];       // diagonal blocks of X
    __shared__ __attribute__((aligned(16))) bf16 sT[BT][TP];             // T = X Diag(beta)
    // Per-tile factors of the gate (dead once the Gram phase starts, when the
    // same bytes hold the last token tile's row fragments).
    __shared__ __attribute__((aligned(16))) float sFac[4][4][DKP];
    auto& sTot = sFac[0];                                                // tile totals of g
    __shared__ __attribute__((aligned(16))) float sE[4][DKP];            // e^{tile total}
    auto& sBef = sFac[1];                                                // e^{G_b}
    auto& sAft = sFac[2];                                                // e^{G_C - G_b}
    auto& sInv = sFac[3];                                                // e^{-G_b}
    __shared__ int sRowsReady;                                           // sKr written
    __shared__ __attribute__((aligned(16))) float sBeta[BTP];
    __shared__ __attribute__((aligned(16))) float sCw[CONV ? 3 * kMaxConvWidth * D : 1];   // conv weights

    // One workgroup per (chunk slot x, head h), heads fastest in the linear
    // id: workgroups are dealt to the XCDs round-robin by linear id, so
    // record (x, h) is written on XCD h mod 8 (with H a multiple of 8, the
    // XCD whose L2 the chain of head h reads from), and the chunks are
    // dispatched in order.
    const int x = (int)(blockIdx.x / (unsigned)heads), h = (int)(blockIdx.x % (unsigned)heads);
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int l16 = lane & 15, g4 = lane >> 4;

    if (wave == 0) {
        // The chain kernel's flags start at zero, and so does the call's
        // status word.  Workgroup 0 is dispatched before every other one and
        // clears the word first thing; a bounded wait elsewhere takes
        // milliseconds to run out, so no bit raised in this call is lost.
        if (blockIdx.x == 0) *status = 0u;
        uint32_t* fl = reinterpret_cast<uint32_t*>(ws + flag_off);
        const int64_t nwg = gridDim.x;
        for (int64_t i = (int64_t)blockIdx.x * kWave + lane; i < n_flags; i += nwg * kWave) fl[i] = 0;
    }
    int seq = 0, first = 0;
    if (!locate_chunk(cu, pos, n_seqs, BT, x, lane, seq, first)) return;
    if (slots[seq] < 0) return;              // padding sequence: nothing to precompute
    const int off = (int)(start_pos(pos, seq) % BT);
    const int cb = chunk_begin(x - first, BT, off);
    const int64_t t0 = (int64_t)cu[seq] + cb;
    const int len = chunk_end(x - first, cu[seq + 1] - cu[seq], BT, off) - cb;

    uint8_t* rec = ws + ((int64_t)x * heads + h) * P::REC_BYTES;
    bf16* wQ = reinterpret_cast<bf16*>(rec) + P::OFF_Q;
    bf16* wW = reinterpret_cast<bf16*>(rec) + P::OFF_W;
    bf16* wKb = reinterpret_cast<bf16*>(rec) + P::OFF_KB;
    bf16* wU = reinterpret_cast<bf16*>(rec) + P::OFF_U;
    bf16* wA = reinterpret_cast<bf16*>(rec) + P::OFF_A;
    float* wEg = reinterpret_cast<float*>(rec + P::EG_BYTE_OFF);
    const RecordOut ro(rec, (int)P::REC_BYTES);

    const bool tok_wave = wave < NS;
    const int r = 16 * (tok_wave ? wave : 0) + l16;  // this lane's token row
    const bool valid = tok_wave && r < len;

    // 0. Loads: this lane's token, channels 32 kk + 8 g4 .. + 7, in the
    //    order of first use (g for the scan, then k and q, v last) so each
    //    phase waits only for what it reads.
    bf16x8 kq[NKK], kk8[NKK], kv[NKK];
    float gv[NKK][8];
    float b_r = 0.0f;
    const int64_t tr = t0 + r;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        const int c0 = 32 * kk + 8 * g4;
        if (valid && c0 < D) {
            load8(g + (tr * heads + h) * D + c0, gv[kk]);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) gv[kk][e] = 0.0f;
        }
    }
    if (valid) b_r = beta[tr * heads + h];
    if constexpr (CONV) {
        // q, k, v are the conv outputs of channels h d + c of the packed
        // projection's three parts (q = x, k = x + H d, v = x + 2 H d).
        const int W = cv.width;
        const int64_t hd = (int64_t)heads * D;
        // The weights of this head's channels are staged in LDS tap-major per
        // part and widened to fp32, sCw[(part W + j) D + c].  Each part's weights are one
        // contiguous block of D W elements (channel-major, W taps per
        // channel), read as 16-byte vectors: all loads are issued first (with
        // the conv rows behind them), the LDS writes come after.
        constexpr int kVec = 16 / (int)sizeof(AT);
        constexpr int kWIt = (3 * kMaxConvWidth * D / kVec + kThreads - 1) / kThreads;
        const int per_part = W * D / kVec;
        uint4 wreg[kWIt];
        auto wload = [&]() {
#pragma unroll
            for (int i = 0; i < kWIt; ++i) {
                const int e = tid + i * kThreads;
                if (e < 3 * per_part) {
                    const int part = e / per_part, o = e - part * per_part;
                    wreg[i] = *reinterpret_cast<const uint4*>(cv.w + (part * hd + (int64_t)h * D) * W +
                                                              (int64_t)o * kVec);
                }
            }
        };
        auto wstore = [&]() {
#pragma unroll
            for (int i = 0; i < kWIt; ++i) {
                const int e = tid + i * kThreads;
                if (e < 3 * per_part) {
                    const int part = e / per_part, o = e - part * per_part;
#pragma unroll
                    for (int u = 0; u < kVec; ++u) {
                        const int f = o * kVec + u, c = f / W, j = f - c * W;
                        store_elem_f32<AT>(sCw + (part * W + j) * D + c, wreg[i], u);
                    }
                }
            }
        };
        const int64_t s0 = cu[seq];
        const int cslot = slots[seq];
        const bool cinit = cslot < cv.num_slots && (cv.has_init ? cv.has_init[seq] != 0 : true);
        const AT* st = cinit ? cv.state + (int64_t)cslot * (W - 1) * cv.channels : nullptr;
        const bool early_lane = tok_wave && l16 >= 17 - W && r - 16 < len;
        const AT* xpart[3] = {q, k, v};
        const int64_t xstr[3] = {qs, ks, vs};
        auto fetch = [&](int part, ConvRows<AT> (&cr)[NKK]) {
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                const int c0 = 32 * kk + 8 * g4;
                const bool ok = c0 < D;
                const int64_t ch = (int64_t)h * D + c0;
                conv_fetch(cr[kk], xpart[part] + ch, xstr[part], tr, valid && ok, early_lane && ok, s0,
                           st ? st + part * hd + ch : nullptr, cv.channels, W);
            }
        };
        auto eval_w = [&](auto wc, int part, const ConvRows<AT> (&cr)[NKK], bf16x8 (&dst)[NKK]) {
            constexpr int WC = decltype(wc)::value;
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                const int c0 = 32 * kk + 8 * g4;
                const bool ok = valid && c0 < D;
                const int cc = c0 < D ? c0 : 0;
                const bf16x8 y = conv_eval<D, WC>(cr[kk], cv.b ? cv.b + part * hd + (int64_t)h * D + cc : nullptr,
                                                  sCw + part * W * D + cc, W, cv.silu, l16);
                dst[kk] = ok ? y : bf16x8{};
            }
        };
        // Widths 2 .. 4 (the common short convolutions) with the width fixed
        // at compile time; wider ones through the general path.
        auto eval = [&](int part, const ConvRows<AT> (&cr)[NKK], bf16x8 (&dst)[NKK]) {
            switch (W) {
                case 2: eval_w(std::integral_constant<int, 2>{}, part, cr, dst); break;
                case 3: eval_w(std::integral_constant<int, 3>{}, part, cr, dst); break;
                case 4: eval_w(std::integral_constant<int, 4>{}, part, cr, dst); break;
                default: eval_w(std::integral_constant<int, 0>{}, part, cr, dst); break;
            }
        };
        // k is evaluated first, then q, then v (the order of first use).
        if constexpr (sizeof(AT) == 2) {
            // All rows are requested before the first evaluation, so the
            // chunk waits for one round of load latency.
            ConvRows<AT> rk[NKK], rq[NKK], rv[NKK];
            wload();
            fetch(1, rk);
            fetch(0, rq);
            fetch(2, rv);
            wstore();
            lds_barrier();                   // the staged weights
            eval(1, rk, kk8);
            eval(0, rq, kq);
            eval(2, rv, kv);
        } else {
            // fp32 rows take twice the registers: one part ahead.
            ConvRows<AT> ra[NKK], rb[NKK];
            wload();
            fetch(1, ra);
            fetch(0, rb);
            wstore();
            lds_barrier();                   // the staged weights
            eval(1, ra, kk8);
            fetch(2, ra);
            eval(0, rb, kq);
            eval(2, ra, kv);
        }
    } else {
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            const int c0 = 32 * kk + 8 * g4;
            const bool ok = valid && c0 < D;
            kk8[kk] = ok ? load8_bf16(k + tr * ks + (int64_t)h * D + c0) : bf16x8{};
            kq[kk] = ok ? load8_bf16(q + tr * qs + (int64_t)h * D + c0) : bf16x8{};
        }
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            const int c0 = 32 * kk + 8 * g4;
            kv[kk] = (valid && c0 < D) ? load8_bf16(v + tr * vs + (int64_t)h * D + c0) : bf16x8{};
        }
    }
    if (tok_wave && g4 == 0) sBeta[r] = b_r;
    if (BTP > BT && tid < BTP - BT) sBeta[BT + tid] = 0.0f;
    if (tid == 0) sRowsReady = 0;

    // 1. Cumulative gate inside the tile (DPP scan over the 16 token lanes).
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
        for (int e = 0; e < 8; ++e) gv[kk][e] = row_scan16(gv[kk][e]);
    if (tok_wave && l16 == 15) {
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            const int c0 = 32 * kk + 8 * g4;
            *reinterpret_cast<float4*>(&sTot[wave][c0]) = make_float4(gv[kk][0], gv[kk][1], gv[kk][2], gv[kk][3]);
            *reinterpret_cast<float4*>(&sTot[wave][c0 + 4]) = make_float4(gv[kk][4], gv[kk][5], gv[kk][6], gv[kk][7]);
        }
    }
    // L2 norms of q and k over the token's channels (4 lanes share a token).
    float rq = 1.0f, rk = 1.0f;
    if (flags & KDA_FLAG_QK_L2NORM) {
        float sq = 0.0f, sk = 0.0f;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float a = static_cast<float>(kq[kk][e]), b = static_cast<float>(kk8[kk][e]);
                sq += a * a;
                sk += b * b;
            }
        sq += __shfl_xor(sq, 16, kWave); sq += __shfl_xor(sq, 32, kWave);
        sk += __shfl_xor(sk, 16, kWave); sk += __shfl_xor(sk, 32, kWave);
        rq = 1.0f / sqrtf(sq + 1e-6f);
        rk = 1.0f / sqrtf(sk + 1e-6f);
    }
    __syncthreads();

    // Per-tile reference points and the chunk's total decay, per channel c:
    //   sBef[w][c] = e^{G_{b_w}},  sAft[w][c] = e^{G_C - G_{b_w}},
    //   sInv[w][c] = e^{-G_{b_w}},  sE[w][c] = e^{tile total w},  e^{G_C} -> record.
    // A chunk whose total decay stays above e^{-kMaxLogDecay} on every channel
    // takes the single-reference path: e^{G} and e^{-G} are then both
    // representable and one factor pair serves every Gram block.
    bool strong = false;
    for (int c = tid; c < DKP; c += kThreads) {
        float tot = 0.0f;
        for (int j = 0; j < NS; ++j) tot += sTot[j][c];
        float pre = 0.0f;
        for (int j = 0; j < NS; ++j) {
            const float tj = sTot[j][c];
            sBef[j][c] = __expf(pre);
            sInv[j][c] = __expf(-pre);
            sAft[j][c] = __expf(tot - pre);
            sE[j][c] = __expf(tj);
            pre += tj;
        }
        ro.put(wEg + c, c < D ? __expf(tot) : 0.0f);
        strong |= tot < -kMaxLogDecay;
    }
    strong = __syncthreads_or(strong) != 0;

    // 2. Factors, with f_w = e^{G_r - G_{b_w}} (the scan is tile-relative):
    //    K^ = k / f_w (tile reference; times e^{-G_{b_w}} for the chunk-start
    //    reference of the single-reference path) -> LDS;
    //    Kb = k e^{G_C - G_r} -> record (transposed);
    //    Q~ = q e^{G_r} -> record;  K~ = k e^{G_r} -> LDS (transposed).
    bf16x8 qt0[NKK], kt0[NKK];
    if (tok_wave) {
        const bf16x8 id0 = identity_half(0, lane), id1 = identity_half(1, lane);
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            const int c0 = 32 * kk + 8 * g4;
            const float4 bf0 = *reinterpret_cast<const float4*>(&sBef[wave][c0]);
            const float4 bf1 = *reinterpret_cast<const float4*>(&sBef[wave][c0 + 4]);
            const float4 af0 = *reinterpret_cast<const float4*>(&sAft[wave][c0]);
            const float4 af1 = *reinterpret_cast<const float4*>(&sAft[wave][c0 + 4]);
            const float4 iv0 = *reinterpret_cast<const float4*>(&sInv[wave][c0]);
            const float4 iv1 = *reinterpret_cast<const float4*>(&sInv[wave][c0 + 4]);
            const float bef[8] = {bf0.x, bf0.y, bf0.z, bf0.w, bf1.x, bf1.y, bf1.z, bf1.w};
            const float aft[8] = {af0.x, af0.y, af0.z, af0.w, af1.x, af1.y, af1.z, af1.w};
            const float inb[8] = {iv0.x, iv0.y, iv0.z, iv0.w, iv1.x, iv1.y, iv1.z, iv1.w};
            float kh[8], kb[8], qt[8], kt[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float fw = __expf(gv[kk][e]);
                const float inv = __builtin_amdgcn_rcpf(fw);
                const float f0 = fw * bef[e];
                const float kn = static_cast<float>(kk8[kk][e]) * rk;
                const float khw = kn * inv;
                kh[e] = strong ? khw : khw * inb[e];
                kb[e] = khw * aft[e];
                qt[e] = static_cast<float>(kq[kk][e]) * rq * f0;
                kt[e] = kn * f0;
                gv[kk][e] = fw;                 // keep f_w for the multi-reference path
            }
            sKh[wave][kk][lane] = pack_bf16x8(kh);
            qt0[kk] = pack_bf16x8(qt);
            kt0[kk] = pack_bf16x8(kt);
            ro.put(wQ + frag<DKP>(r, c0), qt0[kk]);
            // Kb^T through the identity products: lane l gets channel
            // 32 kk + 16 half + l % 16, tokens 16 w + 4 (l / 16) .. + 3.
            const bf16x8 akb = pack_bf16x8(kb);
            const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const f32x4 tb = mfma16x16x32(akb, half ? id1 : id0, zero);
                ro.put(wKb + frag<BTP>(32 * kk + 16 * half + l16, 16 * wave + 4 * g4), pack_bf16x4(tb));
            }
        }
    }
    if (BTP > BT) {                           // token padding of Kb^T
        for (int idx = tid; idx < DKP * (BTP - BT) / 4; idx += kThreads) {
            const int c = idx / ((BTP - BT) / 4), s = BT + 4 * (idx % ((BTP - BT) / 4));
            ro.put(wKb + frag<BTP>(c, s), bf16x4{});
        }
    }
    __syncthreads();                          // sKh ready

    // 3. Gram blocks (w, j), j <= w, computed transposed: C[s][r], lane l
    //    holding row r = 16 w + l % 16 and columns s = 16 j + 4 (l / 16) .. + 3.
    //    Single reference: C = K^_s . K~_r with K^ = k e^{-G}, K~ = k e^{G}.
    //    Multi-reference (strong decay): the reference of block (w, j) is
    //    b_j; the row side is k_r f_j with f_j = f_{j+1} e^{tile total j} <= 1,
    //    the column side K^_s = k_s e^{G_{b_j} - G_s} written by wave j.
    //    With four token tiles and a single reference, blocks (3, 0) and
    //    (3, 1) go to waves 0 and 1, which read tile 3's row fragments from
    //    LDS: no wave then does more than three blocks (instead of 1 .. 4).
    auto gram_store = [&](int w, int j, const f32x4& ck, const f32x4& cq, float br) {
        const int rr = 16 * w + l16;
        f32x4 mk, aq;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int sc = 16 * j + 4 * g4 + ii;
            mk[ii] = sc < rr ? br * ck[ii] : 0.0f;
            aq[ii] = sc <= rr ? cq[ii] : 0.0f;
        }
        *reinterpret_cast<f32x4*>(&sM[rr][16 * j + 4 * g4]) = mk;
        ro.put(wA + aq_frag(rr, 16 * j + 4 * g4), pack_bf16x4(aq));
    };
    const bool split_gram = NS == 4 && !strong;
    auto sKr = reinterpret_cast<bf16x8 (*)[NKK][kWave]>(&sFac[0][0][0]);   // [2][NKK][64]: K~, Q~ of tile 3
    static_assert(sizeof(sFac) >= 2 * NKK * kWave * sizeof(bf16x8), "row fragments fit");
    if (tok_wave) {
        if (split_gram && wave == 3) {
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                sKr[0][kk][lane] = kt0[kk];
                sKr[1][kk][lane] = qt0[kk];
            }
            __hip_atomic_store(&sRowsReady, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        const int jmin = split_gram && wave == 3 ? 2 : 0;
        for (int j = wave; j >= jmin; --j) {
            f32x4 ck = {0.f, 0.f, 0.f, 0.f}, cq = {0.f, 0.f, 0.f, 0.f};
            if (!strong) {
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk) {
                    const bf16x8 a = sKh[j][kk][lane];
                    ck = mfma16x16x32(a, kt0[kk], ck);
                    cq = mfma16x16x32(a, qt0[kk], cq);
                }
            } else {
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk) {
                    const int c0 = 32 * kk + 8 * g4;
                    if (j < wave) {             // gv holds f_{j+1}; advance to f_j
                        const float4 a = *reinterpret_cast<const float4*>(&sE[j][c0]);
                        const float4 b = *reinterpret_cast<const float4*>(&sE[j][c0 + 4]);
                        const float em[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
                        for (int e = 0; e < 8; ++e) gv[kk][e] *= em[e];
                    }
                    float bk[8], bq[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        bk[e] = static_cast<float>(kk8[kk][e]) * rk * gv[kk][e];
                        bq[e] = static_cast<float>(kq[kk][e]) * rq * gv[kk][e];
                    }
                    const bf16x8 a = sKh[j][kk][lane];
                    ck = mfma16x16x32(a, pack_bf16x8(bk), ck);
                    cq = mfma16x16x32(a, pack_bf16x8(bq), cq);
                }
            }
            gram_store(wave, j, ck, cq, b_r);
        }
        if (split_gram && wave < 2) {           // block (3, wave)
            int spin = 0;
            for (; spin < kMaxRowWait &&
                   __hip_atomic_load(&sRowsReady, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) == 0;
                 ++spin)
                __builtin_amdgcn_s_sleep(1);
            f32x4 ck = {0.f, 0.f, 0.f, 0.f}, cq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                const bf16x8 a = sKh[wave][kk][lane];
                ck = mfma16x16x32(a, sKr[0][kk][lane], ck);
                cq = mfma16x16x32(a, sKr[1][kk][lane], cq);
            }
            if (spin == kMaxRowWait) {           // the fragments never came: poison, not garbage
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) ck[ii] = cq[ii] = __builtin_nanf("");
                raise_status(status, kStatusTimeout);
            }
            gram_store(3, wave, ck, cq, sBeta[48 + l16]);
        }
        for (int j = wave + 1; j < P::aq_width(wave) / 16; ++j)   // above the diagonal
            ro.put(wA + aq_frag(r, 16 * j + 4 * g4), bf16x4{});
        // T is zero above the diagonal blocks (and in the token padding).
        for (int cc = 16 * (wave + 1) + 4 * g4; cc < BTP; cc += 16)
            *reinterpret_cast<bf16x4*>(&sT[r][cc]) = bf16x4{};
    }
    __syncthreads();                          // sM ready

    // 4a. Diagonal blocks of X = (I + M)^{-1}: forward substitution, lane c
    //     of wave w solves column c of X_ww; T = X Diag(beta) alongside.
    if (tok_wave && lane < 16) {
        const int b0 = 16 * wave, c = lane;
        float xc[16];
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            float acc = rr == c ? 1.0f : 0.0f;
#pragma unroll
            for (int s = 0; s < rr; ++s) acc -= sM[b0 + rr][b0 + s] * xc[s];
            xc[rr] = acc;
            sXd[wave][rr][c] = acc;
            sT[b0 + rr][b0 + c] = static_cast<bf16>(acc * b_r);   // b_r: beta of token b0 + c
        }
#pragma unroll
        for (int rr = 0; rr < 16; rr += 4)
            *reinterpret_cast<float4*>(&sXt[b0 + c][b0 + rr]) = make_float4(xc[rr], xc[rr + 1], xc[rr + 2], xc[rr + 3]);
    }
    // 4b. Off-diagonal blocks, block row by block row:
    //     X_ij = -X_ii sum_{j<=m<i} M_im X_mj  (fp32 MFMA); wave j does (i, j).
    //     MFMA step kb uses K index 4 (l/16) + kb in lane l, so A and B are
    //     read as float4 rows of M, X and X^T.
    for (int i = 1; i < NS; ++i) {
        __syncthreads();
        if (wave < i) {
            const int j = wave;
            f32x4 y = {0.f, 0.f, 0.f, 0.f};
            for (int m = j; m < i; ++m) {
                const f32x4 a = *reinterpret_cast<const f32x4*>(&sM[16 * i + l16][16 * m + 4 * g4]);
                const f32x4 b = *reinterpret_cast<const f32x4*>(&sXt[16 * j + l16][16 * m + 4 * g4]);
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) y = mfma16x16x4f32(a[kb], b[kb], y);
            }
            const f32x4 a = *reinterpret_cast<const f32x4*>(&sXd[i][l16][4 * g4]);
            f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) z = mfma16x16x4f32(a[kb], y[kb], z);
            const float bs = sBeta[16 * j + l16];
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                z[ii] = -z[ii];
                sT[16 * i + 4 * g4 + ii][16 * j + l16] = static_cast<bf16>(z[ii] * bs);
            }
            *reinterpret_cast<f32x4*>(&sXt[16 * j + l16][16 * i + 4 * g4]) = z;
        }
    }
    __syncthreads();                          // X and T complete; M and X^T dead

    // K~^T and V^T through the identity products (into the regions of X^T and M).
    if (tok_wave) {
        const bf16x8 id0 = identity_half(0, lane), id1 = identity_half(1, lane);
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const bf16x8 id = half ? id1 : id0;
                const f32x4 tk = mfma16x16x32(kt0[kk], id, zero);
                const f32x4 tv = mfma16x16x32(kv[kk], id, zero);
                const int c = 32 * kk + 16 * half + l16;
                *reinterpret_cast<bf16x4*>(&sKt[c][16 * wave + 4 * g4]) = pack_bf16x4(tk);
                *reinterpret_cast<bf16x4*>(&sVt[c][16 * wave + 4 * g4]) = pack_bf16x4(tv);
            }
    }
    if (BTP > BT) {                           // token padding of the transposed tiles
        for (int idx = tid; idx < DKP * (BTP - BT) / 4; idx += kThreads) {
            const int c = idx / ((BTP - BT) / 4), s = BT + 4 * (idx % ((BTP - BT) / 4));
            *reinterpret_cast<bf16x4*>(&sKt[c][s]) = bf16x4{};
            *reinterpret_cast<bf16x4*>(&sVt[c][s]) = bf16x4{};
        }
    }
    __syncthreads();                          // K~^T, V^T ready

    // 5. W^T = K~^T T^T (lane: 4 consecutive channels of one W row) and
    //    U = T V (lane: 4 consecutive tokens of one U^T row), K stopping at
    //    each token tile's diagonal block.  Wave w takes the key tiles and the
    //    value tiles w, w + 4, ... for every token tile: a later token tile
    //    needs more K steps, so this spreads the products evenly, and each
    //    K~^T or V^T fragment is read from LDS once per wave.
    {
        bf16x8 tf[NS][P::NKK_T];
#pragma unroll
        for (int t = 0; t < NS; ++t)
#pragma unroll
            for (int kk = 0; kk < P::NKK_T; ++kk)
                tf[t][kk] = kk <= (16 * t + 15) / 32
                                ? *reinterpret_cast<const bf16x8*>(&sT[16 * t + l16][32 * kk + 8 * g4]) : bf16x8{};
#pragma unroll
        for (int mt = wave; mt < DKP / 16; mt += kThreads / kWave) {
            bf16x8 kf[P::NKK_T];
#pragma unroll
            for (int kk = 0; kk < P::NKK_T; ++kk)
                kf[kk] = *reinterpret_cast<const bf16x8*>(&sKt[16 * mt + l16][32 * kk + 8 * g4]);
#pragma unroll
            for (int t = 0; t < NS; ++t) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < P::NKK_T; ++kk)
                    if (kk <= (16 * t + 15) / 32) acc = mfma16x16x32(kf[kk], tf[t][kk], acc);
                ro.put(wW + frag<DKP>(16 * t + l16, 16 * mt + 4 * g4), pack_bf16x4(acc));
            }
        }
#pragma unroll
        for (int nt = wave; nt < D / 16; nt += kThreads / kWave) {
            bf16x8 vf[P::NKK_T];
#pragma unroll
            for (int kk = 0; kk < P::NKK_T; ++kk)
                vf[kk] = *reinterpret_cast<const bf16x8*>(&sVt[16 * nt + l16][32 * kk + 8 * g4]);
#pragma unroll
            for (int t = 0; t < NS; ++t) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < P::NKK_T; ++kk)
                    if (kk <= (16 * t + 15) / 32) acc = mfma16x16x32(tf[t][kk], vf[kk], acc);
                ro.put(wU + frag<BTP>(16 * nt + l16, 16 * t + 4 * g4), pack_bf16x4(acc));
            }
        }
    }
    if (BTP > BT)
        for (int idx = tid; idx < D * (BTP - BT) / 4; idx += kThreads) {
            const int row = idx / ((BTP - BT) / 4), c4 = idx % ((BTP - BT) / 4);
            ro.put(wU + frag<BTP>(row, BT + 4 * c4), bf16x4{});
        }

    if constexpr (CONV) {
        // The sequence's new conv state, this head's channels of q, k and v:
        // its last W - 1 inputs (for a sequence shorter than that, the newest
        // rows of the old state before them).  The sequence's first chunk
        // writes it: that workgroup is the only reader of the old rows, and
        // its reads completed before the conv evaluation.  Each thread reads
        // all rows of its channels before writing any (the rows shift in
        // place when the sequence is short).  In the fused front end q is the
        // packed projection x (k and v are q + H d and q + 2 H d, one stride).
        const int cslot = slots[seq];
        if (x == first && cv.state && cslot < cv.num_slots) {
            const int W = cv.width;
            const int64_t hd = (int64_t)heads * D;
            const int64_t s0 = cu[seq], s1 = cu[seq + 1];
            const bool cinit = cv.has_init ? cv.has_init[seq] != 0 : true;
            AT* stw = cv.state + (int64_t)cslot * (W - 1) * cv.channels;
            constexpr int kG = D / 8;                      // 8-channel groups per part
            for (int e = tid; e < 3 * kG; e += kThreads) {
                const int part = e / kG;
                const int64_t ch = part * hd + (int64_t)h * D + 8 * (e - part * kG);
                Raw8<AT> rows[kMaxConvWidth - 1];
#pragma unroll
                for (int j = 0; j < kMaxConvWidth - 1; ++j) {
                    if (j < W - 1) {
                        const int64_t p = s1 - (W - 1) + j;
                        rows[j] = p >= s0 ? load_raw8(q + p * qs + ch)
                                : cinit   ? load_raw8(stw + (int64_t)((W - 1) - (s0 - p)) * cv.channels + ch)
                                          : zero_raw8<AT>();
                    }
                }
#pragma unroll
                for (int j = 0; j < kMaxConvWidth - 1; ++j)
                    if (j < W - 1) store_raw8(stw + (int64_t)j * cv.channels + ch, rows[j]);
            }
        }
    }
}

// Gated RMSNorm fused into the chain kernel's output workgroups (page
// "[Feature][KDA] Add Kimi K3 KDA execution", What this PR does: the KDA
// output goes through a fused normalisation-and-gating step; the result is
// a separate buffer, o is kept).  Per (token, head) row of o as stored:
//     y = o * rsqrt(mean(o^2) + eps) * w * SiLU(gate)
// computed exactly as kda_gated_rmsnorm computes it (same lane layout, sum
// chain, shuffle tree and helpers), so y is that call's result bit for bit.
template <typename AT>
struct NormIn {
    const AT* gate; int64_t gs;     // [tokens, heads, D], token stride gs
    const AT* w;                    // [D] or null (= 1)
    AT* y; int64_t ys;              // [tokens, heads, D], token stride ys
    float eps;
    int64_t flag_off;               // workspace offset of the per-(pair, tile) o-stored flags
};

// Eight consecutive elements of one row, as loaded.
template <typename AT> struct Vec8;
template <> struct Vec8<bf16> {
    bf16x8 v;
    __device__ float operator[](int i) const { return static_cast<float>(v[i]); }
};
template <> struct Vec8<float> {
    f32x4 a, b;
    __device__ float operator[](int i) const { return i < 4 ? a[i] : b[i - 4]; }
};
__device__ __forceinline__ void load_vec8(const bf16* p, Vec8<bf16>& x) { x.v = *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ void load_vec8(const float* p, Vec8<float>& x)
{
    x.a = *reinterpret_cast<const f32x4*>(p);
    x.b = *reinterpret_cast<const f32x4*>(p + 4);
}
// Stores of the norm's output rows: written once and read by no one in the
// launch, so nontemporal (faster than write-back stores here, while
// nontemporal loads of the gate were slower).
__device__ __forceinline__ void store_vec8(bf16* p, const float (&x)[8])
{
    __builtin_nontemporal_store(__builtin_bit_cast(f32x4, pack_bf16x8(x)), reinterpret_cast<f32x4*>(p));
}
__device__ __forceinline__ void store_vec8(float* p, const float (&x)[8])
{
    __builtin_nontemporal_store(f32x4{x[0], x[1], x[2], x[3]}, reinterpret_cast<f32x4*>(p));
    __builtin_nontemporal_store(f32x4{x[4], x[5], x[6], x[7]}, reinterpret_cast<f32x4*>(p + 4));
}

// ---------------------------------------------------------------------------
// chain_kernel: the state-dependent part, serial over a sequence's chunks.
//
// Two workgroups per (sequence, head, 16-column d_v tile), on two CUs of one
// XCD:
//   state workgroup    8 waves, two barriers per chunk.  Phase 1: wave w <
//                      BT / 16 computes D = U - W S for token tile w; phase 2:
//                      every wave w computes S <- e^{G_C} S + Kb^T D for key
//                      tile w (and w + 8, ... for d_k > 128).  S stays in fp32
//                      accumulators and is shared as bf16 through LDS.
//                      Each chunk's S (at its start) and D go, in bf16, to the
//                      chunk's exchange slot in the workspace; once they have
//                      landed in L2 the chunk count is published in a flag.
//   output workgroup   4 output waves and a loader wave, one barrier per
//                      chunk.  The loader waits for the flag and copies the
//                      chunk's S and D from its slot into LDS, two chunks
//                      ahead; output wave t writes O = scale (Q~ S + Aqk D)
//                      for token tile t, computed transposed so each lane
//                      stores 4 consecutive columns.  Waves 5-7 end at once,
//                      or, with the gated norm fused (NORM), waves 5 and 6
//                      normalise this tile's share of the rows nine chunks
//                      behind (norm_rows).
// Every byte of a record is an MFMA operand of exactly one wave, so each
// compute wave loads its own record operands straight into a register ring
// kChainBufs - 1 chunks ahead.  Splitting the roles halves what one CU pulls
// from L2 per chunk, which is what bounds the chain (W, Kb^T, U, e^{G_C} on
// one CU; Q~, Aqk and the 6 KB of S and D on the other).  Eight state waves
// rather than four spread that CU's loads over twice the waves and halve the
// MFMA chain of phase 2: the chain kernel takes 38 us instead of 44 us at
// T = 4096, H = 16, d = 128.
//
// The exchange goes through the XCD's L2: plain stores, and loads issued only
// after the flag, at addresses the CU has not read before in the launch.
// Workgroups are dealt to the XCDs round-robin by linear id and
// the two roles of a tile are 8 * k ids apart, so they share an XCD.  The
// flag carries the state workgroup's XCD id and the output workgroup checks
// it; if the two ever ran on different XCDs the output workgroup would never
// see the flag move and writes NaN after a bounded wait instead of stale
// results.  A pair's state workgroups come before its output workgroups in
// the grid, so every output workgroup's producer is already running when it
// starts waiting.
constexpr int kChainWaves = 8;
constexpr int kChainThreads = kChainWaves * kWave;
constexpr int kChainBufs = 3;                      // register ring depth (chunks)
constexpr int kXchStages = 3;                      // LDS stages of S and D (output workgroup)
// Spin limit of the output workgroup's loader waiting for a chunk; the state
// workgroup publishes one every microsecond or so, so this is a safety net.
constexpr int kMaxSpin = 1 << 20;
// Longest average sequence (in chunks) for which a grid that does not fit on
// the chip at one workgroup per CU runs two per CU (d = 128).  Packing lets
// the chains of more sequences run at once, which hides each chain's fixed
// start and end (a few microseconds), but each CU then serves two
// workgroups' loads, so every step is slower: on MI355X (H = 16) the packed
// grid was faster up to ~22 chunks per sequence and slower from 32.
constexpr int kPackMaxChunks = 24;

// Cache policy sc0 (workgroup scope) of the loader's copies: they read each
// exchange slot once, after its flag, at an address this CU has not read
// before in the launch, so no stale L1 line can answer them.
constexpr int kSkipL1 = 1;
typedef __attribute__((address_space(3))) void lds_void;

// Marks every register of `x` as read here, so that the loads that wrote it
// are waited for at this point (and not later, behind a branch).
template <typename T>
__device__ __forceinline__ void consume(const T& x)
{
    constexpr int N = sizeof(T) / 16, R = sizeof(T) % 16 / 4;
    static_assert(sizeof(T) % 4 == 0, "4-byte pieces");
    const uint32_t* p = reinterpret_cast<const uint32_t*>(&x);
#pragma unroll
    for (int i = 0; i < N; ++i) {
        uint32_t a = p[4 * i], b = p[4 * i + 1], c = p[4 * i + 2], d = p[4 * i + 3];
        asm volatile("" : : "v"(a), "v"(b), "v"(c), "v"(d));
    }
#pragma unroll
    for (int i = 0; i < R; ++i) {
        uint32_t a = p[4 * N + i];
        asm volatile("" : : "v"(a));
    }
}

// Loads of 4, 8 or 16 bytes at base + byte_off, coherent at device scope
// (sc1: they miss in the CU's L1 and read the XCD's L2): for data another
// workgroup, or this one, wrote in the same launch at an address this CU may
// already hold in L1.  (The workgroup-scope policy, sc0, is not enough for
// that: such a load can still return a line the L1 fetched before the
// write.)  base must be the same for the whole wave.  Callers reinterpret the result as a float or
// bf16 vector: indexing an integer-vector reinterpretation of it compiled,
// with this toolchain, to one loaded element copied into every lane of the
// vector.
template <int BYTES>
__device__ __forceinline__ auto load_l2(const void* base, int byte_off)
{
    // The base is the wave's own (the caller guarantees it); taken from the
    // first lane so that the compiler keeps the descriptor in scalar
    // registers instead of looping over the lanes' values.
    // (readfirstlane returns a signed int: each half is widened through
    // uint32_t so that a low word at or above 2^31 is not sign-extended.)
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    const uint64_t ub = ((uint64_t)hi << 32) | (uint64_t)lo;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(ub), 0, 0x7fffffff,
                                                                         kBufferRsrcWord3);
    if constexpr (BYTES == 16) return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kDeviceScope);
    else if constexpr (BYTES == 8) return __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, kDeviceScope);
    else return __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, kDeviceScope);
}
__device__ __forceinline__ void load_vec8_l2(const bf16* base, int byte_off, Vec8<bf16>& x)
{
    x.v = __builtin_bit_cast(bf16x8, __builtin_bit_cast(f32x4, load_l2<16>(base, byte_off)));
}
__device__ __forceinline__ void load_vec8_l2(const float* base, int byte_off, Vec8<float>& x)
{
    x.a = __builtin_bit_cast(f32x4, load_l2<16>(base, byte_off));
    x.b = __builtin_bit_cast(f32x4, load_l2<16>(base, byte_off + 16));
}

// The chunk loop of one wave with a register ring of NB chunks, steps first
// to nch - 1 (first a multiple of NB; the buffer of chunk lc is buf[lc % NB]).
// The loop runs whole groups of NB steps (so every buffer is used at a fixed
// place in the body) and the last steps after it.  Step lc runs on the buffer
// of chunk lc and calls `refill`, which starts the loads of chunk lc + NB - 1
// into the buffer that step lc - 1 used (its arguments go on to `fetch`, so a
// step may start them in parts).
template <int NB, typename Ops, typename Fetch, typename Step>
__device__ __forceinline__ void run_steps(int first, int nch, Ops (&buf)[NB], Fetch fetch, Step step)
{
    int c0 = first;
    for (; c0 + NB <= nch; c0 += NB) {
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            consume(buf[u]);
            step(c0 + u, buf[u], [&](auto... part) { fetch(c0 + u + NB - 1, buf[(u + NB - 1) % NB], part...); });
        }
    }
#pragma unroll
    for (int u = 0; u < NB - 1; ++u) {
        if (c0 + u < nch) {
            consume(buf[u]);
            step(c0 + u, buf[u], [&](auto... part) { fetch(c0 + u + NB - 1, buf[(u + NB - 1) % NB], part...); });
        }
    }
}
template <int NB, typename Ops, typename Fetch, typename Step>
__device__ __forceinline__ void run_steps(int nch, Ops (&buf)[NB], Fetch fetch, Step step)
{
    run_steps<NB>(0, nch, buf, fetch, step);
}

// The o-stored flags of a pair's D/16 output workgroups (with the norm
// fused): tile t's flag holds (XCD id << 24) | the number of chunks whose o
// that workgroup has stored.  Lane t of a wave reads tile t's, so one load
// polls them all.
template <int D>
struct StoredFlags {
    const uint32_t* f0;
    uint32_t xcc;
    bool mine;                                     // this lane reads a flag
    __device__ StoredFlags(const uint32_t* f, uint32_t x, int lane) : f0(f), xcc(x), mine(lane < D / 16) {}
    __device__ uint32_t load(int lane) const
    {
        return mine ? __hip_atomic_load(f0 + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
    }
    __device__ bool at(uint32_t f, int n) const    // every tile has stored n chunks
    {
        return __all(!mine || ((f >> 24) == xcc && (int)(f & 0xffffff) >= n));
    }
    // Until every tile has stored n chunks; false, with the status word
    // raised, if the bounded wait ran out.
    __device__ bool wait(int n, int lane, int max_spin, uint32_t* status) const
    {
        uint32_t f = 0;
        for (int spin = 0; spin < max_spin; ++spin) {
            f = load(lane);
            if (at(f, n)) return true;
            __builtin_amdgcn_s_sleep(2);
        }
        const bool elsewhere = __any(mine && f != 0 && (f >> 24) != xcc);
        raise_status(status, elsewhere ? kStatusPlacement : kStatusTimeout);
        return false;
    }
};

// Norm waves of an output workgroup (the norm fused into the prefill).  The
// pair's D/16 output workgroups split each chunk's BT rows into runs of
// RW = 16 BT / D rows in tile order, and each normalises its run with
// kda_gated_rmsnorm's lane layout for these head dims: D/8 lanes per row, one
// 8-element vector each, the lane's sum of squares in element order, then
// the shuffle tree over the row's lanes.  So y is that kernel's result bit
// for bit.
// The waves trail the output waves by kNormLag chunks, one step per barrier
// of the workgroup.  In step lc a wave starts the loads of o and the gate of
// chunk lc + 2 - kNormLag and writes y of chunk lc - kNormLag from what it
// loaded two steps earlier.  The loader has made sure, by the barrier that
// began the step, that every tile has stored lc - 5 chunks (it checks flags
// it loaded a step before, so it rarely waits), which covers the chunk with a
// step to spare.  After the loop the waves wait until every tile has stored
// all its chunks and write the rest.
// The steps before the first write and the steps after it run as two loops,
// and every step of a loop issues the same memory operations (the y store
// included: a lane without a row of its own stores the value of a row that
// exists, which another lane stores too), so the compiler's waits for the
// loads of one step never hold for those of a later one.
constexpr int kNormLag = 9;   // a multiple of kChainBufs: the write steps start on a ring boundary
constexpr int kNormCheckLag = 4;   // the loader's check at the end of step c covers c - 4 chunks

template <int D, int BT, typename AT>
__device__ __forceinline__ void norm_rows(int nw, int lane, int tile, int nch, int off, int len, int64_t s_begin,
                                          int h, const AT* out, int64_t os, const NormIn<AT>& nrm,
                                          const StoredFlags<D>& flags, const int* sbroken, uint32_t* status,
                                          int max_spin)
{
    constexpr int NB = kChainBufs;
    constexpr int LPR = D / 8;                     // lanes per row
    constexpr int RP = kWave / LPR;                // rows per wave
    constexpr int RW = BT * 16 / D;                // rows of a chunk per tile
    static_assert(kNormLag % NB == 0, "ring boundary");
    // Step s loads chunk s + NB - 1 - kNormLag; the loader's check at the end
    // of step s - 1 has every tile's chunks up to s - 2 - kNormCheckLag stored.
    static_assert(kNormLag >= NB + 1 + kNormCheckLag, "norm lag");
    static_assert((RW + RP - 1) / RP <= kChainWaves - 5, "norm waves");
    if (nw * RP >= RW) return;
    const int rl = min(nw * RP + lane / LPR, RW - 1);   // row in this tile's run
    const int c8 = (lane % LPR) * 8;               // first column of this lane's vector
    const int rrow = tile * RW + rl;               // row of the chunk
    bool broken = false;
    float wv[8];
    if (nrm.w) {
        Vec8<AT> t;
        load_vec8(nrm.w + c8, t);
#pragma unroll
        for (int i = 0; i < 8; ++i) wv[i] = t[i];
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) wv[i] = 1.0f;
    }
    struct Rows {
        Vec8<AT> o, g;
    };
    // This lane's row of chunk c, clamped into the chunk (a run past a short
    // last chunk reads, and later writes, the chunk's last row).
    auto row_of = [&](int c, int64_t& t0) {
        const int cb = chunk_begin(c, BT, off);
        t0 = s_begin + cb;
        return min(rrow, chunk_end(c, len, BT, off) - cb - 1);
    };
    auto load_rows = [&](int c, Rows& e) {
        int64_t t0;
        const int rr = row_of(c, t0);
        load_vec8_l2(out + t0 * os + (int64_t)h * D, (int)(((int64_t)rr * os + c8) * (int64_t)sizeof(AT)), e.o);
        load_vec8(nrm.gate + (t0 + rr) * nrm.gs + (int64_t)h * D + c8, e.g);
    };
    auto write_rows = [&](int c, const Rows& e) {
        float hv[8];
        float ss = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) hv[i] = e.o[i];
#pragma unroll
        for (int i = 0; i < 8; ++i) ss = __builtin_fmaf(hv[i], hv[i], ss);
#pragma unroll
        for (int o = LPR / 2; o > 0; o >>= 1) ss += __shfl_xor(ss, o, LPR);
        const float inv = rms_inv(ss, D, nrm.eps);
        const float bad = broken || *sbroken ? __builtin_nanf("") : 1.0f;
        float y[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] = bad * gated_norm_out(hv[i], inv, wv[i], 0.0f, e.g[i], false);
        int64_t t0;
        const int rr = row_of(c, t0);
        store_vec8(nrm.y + (t0 + rr) * nrm.ys + (int64_t)h * D + c8, y);
    };
    // Loads of chunk lc - kNormLag (of chunk 0 before the first, unused).
    auto fetch = [&](int lc, Rows& e) { load_rows(max(lc - kNormLag, 0), e); };
    Rows buf[NB];
#pragma unroll
    for (int b = 0; b < NB - 1; ++b) fetch(b, buf[b]);
    lds_barrier();                                 // the output waves' first barrier
    const int lead = min(nch, kNormLag);
    run_steps<NB>(0, lead, buf, fetch, [&](int lc, const Rows&, auto refill) {
        refill();
        lds_barrier();                             // end of step lc
    });
    run_steps<NB>(kNormLag, nch, buf, fetch, [&](int lc, const Rows& e, auto refill) {
        refill();
        write_rows(lc - kNormLag, e);
        lds_barrier();                             // end of step lc
    });
    lds_barrier();                                 // the output waves' last barrier
    // The last kNormLag chunks (fewer in a short sequence), loaded together.
    broken = !flags.wait(nch, lane, max_spin, status);
    const int j0 = nch - lead;
    Rows rest[kNormLag];
#pragma unroll
    for (int i = 0; i < kNormLag; ++i) load_rows(min(j0 + i, nch - 1), rest[i]);
#pragma unroll
    for (int i = 0; i < kNormLag; ++i)
        if (j0 + i < nch) write_rows(j0 + i, rest[i]);
}

// PACK caps the registers at 128 per lane (four waves per SIMD), so that two
// workgroups fit on one CU; the host picks it for grids of short sequences
// that do not fit on the chip at one workgroup per CU (see launch_typed).
template <int D, int BT, typename AT, typename ST, bool NORM, bool PACK>
__global__ __launch_bounds__(kChainThreads, PACK ? 4 : 2)
void chain_kernel(const int32_t* __restrict__ cu, const int64_t* __restrict__ pos, int n_seqs, int heads,
                  ST* __restrict__ pool, int64_t num_slots, const int32_t* __restrict__ slots,
                  const uint8_t* __restrict__ has_init, ST* __restrict__ ckpt, int64_t ckpt_cap,
                  int interval, float scale, AT* __restrict__ out, int64_t os,
                  uint8_t* __restrict__ ws, int64_t xch_off, int64_t xch_chunks, int64_t flag_off,
                  uint32_t* __restrict__ status, int max_spin, NormIn<AT> nrm)
{
    using P = Shape<D, BT>;
    constexpr int DKP = P::DKP, BTP = P::BTP, NS = P::NS, NB = kChainBufs;
    constexpr int NKT_W = (P::NMT_K + 7) / 8;     // key m-tiles per state wave
    constexpr int SP = DKP + 8, DP = BTP + 8;     // bf16 pitches of the LDS tiles
    // Exchange slot of one chunk: S^T [16][DKP] then D^T [16][BTP], bf16, in
    // operand-fragment order.
    constexpr int XS_BYTES = 16 * DKP * 2, XSLOT = XS_BYTES + 16 * BTP * 2;
    static_assert(XSLOT % (kWave * 16) == 0, "exchange slot in 1 KB pieces");

    __shared__ __attribute__((aligned(16))) bf16 sS[16][SP];      // state: bf16 S^T of the tile
    __shared__ __attribute__((aligned(16))) bf16 sD[16][DP];      // state: bf16 D^T
    __shared__ __attribute__((aligned(1024))) uint8_t sX[kXchStages][XSLOT];   // output: S, D

    // One-dimensional grid in blocks of 8 (sequence, head) pairs (padded to a
    // multiple of 8): a block holds the state workgroups of its pairs' D/16
    // tiles, then their output workgroups, pair fastest in both.  So a pair's
    // workgroups are 8 * k ids apart (one XCD), every output workgroup comes
    // after its producer, and the chip works through the pairs block by
    // block: the eight tiles of a pair read its records from L2 at about the
    // same time and its output workgroups run beside its state workgroups.
    // (With the state workgroups of all pairs first, a batch larger than the
    // chip ran its state roles tile by tile in rounds, each round reading the
    // records again, and the output roles only after them.)  The blocks run
    // last pair first: the intra kernel writes the records in pair order, so
    // the last pairs' records are the newest and most likely still in the
    // memory-side cache when a large batch's records do not all fit there.
    // With the norm
    // the output workgroups of a pair also wait for one another; they sit in
    // one block, blocks are dispatched in order, and a workgroup waits only
    // for its own block and earlier ones, so the earliest unfinished block
    // always gets the next free slots.
    constexpr int TB = 8 * (D / 16);               // workgroups of one role in a block
    const int blk = (int)(gridDim.x / (2u * TB)) - 1 - (int)(blockIdx.x / (2u * TB));
    const int rb = (int)(blockIdx.x % (2u * TB));
    const bool state_role = rb < TB;
    const int rr = state_role ? rb : rb - TB;
    const int pair = blk * 8 + rr % 8, tile = rr / 8;
    if (pair >= n_seqs * heads) return;
    const int seq = pair / heads, h = pair % heads, n0 = tile * 16;
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    __builtin_assume(wave >= 0 && wave < kChainWaves);
    const int l16 = lane & 15, g4 = lane >> 4;
    const int col = n0 + l16;
    const uint32_t xcc = __builtin_amdgcn_s_getreg((31 << 11) | 20) & 15;   // HW_REG_XCC_ID

    const int64_t s_begin = cu[seq];
    const int len = max(0, cu[seq + 1] - cu[seq]);
    const int slot = slots[seq];
    if (slot < 0) {                                // graph padding: zero output rows
        if (!state_role)
            for (int idx = tid; idx < len * 16; idx += kChainThreads) {
                const int64_t at = (s_begin + idx / 16);
                const int c = n0 + idx % 16;
                out[at * os + (int64_t)h * D + c] = from_f32<AT>(0.0f);
                if constexpr (NORM) {              // the norm of a zero row
                    const float g = to_f32(nrm.gate[at * nrm.gs + (int64_t)h * D + c]);
                    const float w = nrm.w ? to_f32(nrm.w[c]) : 1.0f;
                    nrm.y[at * nrm.ys + (int64_t)h * D + c] =
                        from_f32<AT>(gated_norm_out(0.0f, rms_inv(0.0f, D, nrm.eps), w, 0.0f, g, false));
                }
            }
        return;
    }
    if (len == 0 || slot >= num_slots) return;

    int chunk_base = 0;
    int64_t ckpt_base = 0;
    sequence_bases(cu, pos, seq, BT, interval, lane, chunk_base, ckpt_base);
    const int64_t p0 = start_pos(pos, seq);
    const int off = (int)(p0 % BT);
    const int nch = num_chunks(len, BT, off);
    // Chunks past the last are clamped to it, so prefetches stay in bounds.
    auto record = [&](int lc) {
        return reinterpret_cast<const bf16*>(
            ws + ((int64_t)(chunk_base + min(lc, nch - 1)) * heads + h) * P::REC_BYTES);
    };
    uint8_t* const xch = ws + xch_off + ((int64_t)(h * (D / 16) + tile) * xch_chunks + chunk_base) * XSLOT;
    uint32_t* const flag = reinterpret_cast<uint32_t*>(ws + flag_off) + ((int64_t)seq * heads + h) * (D / 16) + tile;

    if (state_role) {
        // ---------------- state workgroup ----------------
        const bool init = has_init ? has_init[seq] != 0 : true;
        ST* home = pool + ((int64_t)slot * heads + h) * (int64_t)(D * D);
        const bool dwave = wave < NS;              // owns a token tile of D
        const int tt = dwave ? wave : 0;
        // The initial state, every address clamped into the state so that the
        // loads carry no per-element branch and issue together (a branch per
        // element makes each load wait for the one before).
        ST s0[NKT_W][4];
#pragma unroll
        for (int j = 0; j < NKT_W; ++j)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int row = min(16 * (wave + 8 * j) + 4 * g4 + ii, D - 1);
                s0[j][ii] = init ? home[(int64_t)row * D + col] : from_f32<ST>(0.0f);
            }
        float S[NKT_W][4];
#pragma unroll
        for (int j = 0; j < NKT_W; ++j) {
            const int kt = wave + 8 * j;
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int row = 16 * kt + 4 * g4 + ii;
                S[j][ii] = (kt < P::NMT_K && row < D) ? to_f32(s0[j][ii]) : 0.0f;
            }
            if (kt < P::NMT_K) {
                bf16x4 s4;
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) s4[ii] = static_cast<bf16>(S[j][ii]);
                *reinterpret_cast<bf16x4*>(&sS[l16][16 * kt + 4 * g4]) = s4;
            }
        }
        if (BTP > BT && wave == 0)                 // token padding of D^T stays zero
            *reinterpret_cast<bf16x4*>(&sD[l16][BT + 4 * g4]) = bf16x4{};

        struct Ops {
            bf16x8 w[P::NKK_K];                    // W rows of token tile tt
            bf16x4 u;                              // U^T: column col, 4 tokens of tile tt
            bf16x8 kb[NKT_W][P::NKK_T];            // Kb^T rows of key tiles wave + 8 j
            float eg[NKT_W];                       // e^{G_C} of row 16 kt + 4 g4 + l16 % 4
        };
        // A chunk's operands are fetched in three parts, spread over a step
        // so that no one burst of loads fills the CU's memory queue and
        // stalls the wave: W (part 0), U and e^{G_C} (part 1), Kb^T (part 2);
        // part -1 is all three.  Token-tile waves (phase 1) load all of it,
        // the other waves e^{G_C} and Kb^T only.  Each kind of wave runs its
        // own copy of the chunk loop (`run`, on a compile-time flag), so within
        // a copy every load is unconditional and the counts below are exact.
        constexpr int LOADS1 = 1 + NKT_W, LOADS2 = NKT_W * P::NKK_T;
        constexpr int LOADS = P::NKK_K + LOADS1 + LOADS2;                 // loads per chunk
        auto run = [&](auto is_d) {
            constexpr bool ISD = decltype(is_d)::value;
            auto fetch = [&](int lc, Ops& o, auto part) {
                constexpr int PART = decltype(part)::value;
                const bf16* rec = record(lc);
                if constexpr (ISD && (PART < 0 || PART == 0)) {
#pragma unroll
                    for (int kk = 0; kk < P::NKK_K; ++kk)
                        o.w[kk] = *reinterpret_cast<const bf16x8*>(rec + P::OFF_W + frag<DKP>(16 * tt + l16, 32 * kk + 8 * g4));
                }
                if constexpr (PART < 0 || PART == 1) {
                    if constexpr (ISD) o.u = *reinterpret_cast<const bf16x4*>(rec + P::OFF_U + frag<BTP>(col, 16 * tt + 4 * g4));
#pragma unroll
                    for (int j = 0; j < NKT_W; ++j) {
                        const int kt = min(wave + 8 * j, P::NMT_K - 1);
                        // One float per lane, spread over the quad in the update:
                        // a 16-byte load per lane would move 16 times the bytes.
                        o.eg[j] = *reinterpret_cast<const float*>(
                            reinterpret_cast<const uint8_t*>(rec) + P::EG_BYTE_OFF + (16 * kt + 4 * g4 + (l16 & 3)) * 4);
                    }
                }
                if constexpr (PART < 0 || PART == 2) {
#pragma unroll
                    for (int j = 0; j < NKT_W; ++j) {
                        const int kt = min(wave + 8 * j, P::NMT_K - 1);
#pragma unroll
                        for (int kk = 0; kk < P::NKK_T; ++kk)
                            o.kb[j][kk] = *reinterpret_cast<const bf16x8*>(rec + P::OFF_KB + frag<BTP>(16 * kt + l16, 32 * kk + 8 * g4));
                    }
                }
            };
            using Part0 = std::integral_constant<int, 0>;
            using Part1 = std::integral_constant<int, 1>;
            using Part2 = std::integral_constant<int, 2>;
            using AllParts = std::integral_constant<int, -1>;
            // Checkpoint of chunk c (S holds the state after it) where the chunk
            // ends on an absolute multiple of the interval, written at the start
            // of the next step.
            auto checkpoint = [&](int c) {
                const int64_t at = p0 + chunk_end(c, len, BT, off);
                if (!ckpt || interval <= 0 || at % interval != 0) return;
                const int64_t row = ckpt_base + at / interval - p0 / interval - 1;
                if (row >= ckpt_cap) return;
                ST* dst = ckpt + (row * heads + h) * (int64_t)(D * D);
#pragma unroll
                for (int j = 0; j < NKT_W; ++j) {
                    const int kt = wave + 8 * j;
#pragma unroll
                    for (int ii = 0; ii < 4; ++ii) {
                        const int rr = 16 * kt + 4 * g4 + ii;
                        if (kt < P::NMT_K && rr < D) dst[(int64_t)rr * D + col] = from_f32<ST>(S[j][ii]);
                    }
                }
            };
            // Publishes that chunks 0 .. n - 1 are in their exchange slots.
            // The flag is written with a plain store (a workgroup-scope atomic):
            // the vector L1 is write-through, so the store lands in this XCD's
            // L2, which the output workgroup (same XCD, checked through the id in
            // the flag) polls past its own L1.  An agent-scope store would be
            // written through to memory for the other XCDs' sake, which makes
            // every publish wait on the memory-side round trip.
            auto publish = [&](int n) {
                if (wave == 0)
                    __hip_atomic_store(flag, (xcc << 24) | (uint32_t)n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            };
            auto step = [&](int lc, const Ops& o, auto refill) {
                uint8_t* const slot_x = xch + (int64_t)lc * XSLOT;
                if (lc > 0) checkpoint(lc - 1);
                // This chunk's S (its start state) to the exchange slot.
#pragma unroll
                for (int j = 0; j < NKT_W; ++j) {
                    const int kt = wave + 8 * j;
                    if (kt >= P::NMT_K) continue;
                    bf16x4 s4;
#pragma unroll
                    for (int ii = 0; ii < 4; ++ii) s4[ii] = static_cast<bf16>(S[j][ii]);
                    *reinterpret_cast<bf16x4*>(slot_x + 2 * frag<DKP>(l16, 16 * kt + 4 * g4)) = s4;
                }
                refill(Part0{});
                if constexpr (ISD) {                   // D = U - W S, token tile tt
                    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < P::NKK_K; ++kk) {
                        const bf16x8 b = *reinterpret_cast<const bf16x8*>(&sS[l16][32 * kk + 8 * g4]);
                        if (kk & 1) acc1 = mfma16x16x32(o.w[kk], b, acc1);
                        else acc0 = mfma16x16x32(o.w[kk], b, acc0);
                    }
                    bf16x4 d4;
#pragma unroll
                    for (int ii = 0; ii < 4; ++ii)
                        d4[ii] = static_cast<bf16>(static_cast<float>(o.u[ii]) - (acc0[ii] + acc1[ii]));
                    *reinterpret_cast<bf16x4*>(&sD[l16][16 * tt + 4 * g4]) = d4;
                    *reinterpret_cast<bf16x4*>(slot_x + XS_BYTES + 2 * frag<BTP>(l16, 16 * tt + 4 * g4)) = d4;
                }
                if (BTP > BT && wave == 0)             // token padding of D^T
                    *reinterpret_cast<bf16x4*>(slot_x + XS_BYTES + 2 * frag<BTP>(l16, BT + 4 * g4)) = bf16x4{};
                asm volatile("" ::: "memory");         // parts 1 and 2 come after the stores
                refill(Part1{});
                lds_barrier();                         // B1
                refill(Part2{});
#pragma unroll
                for (int j = 0; j < NKT_W; ++j) {      // S <- Diag(e^{G_C}) S + Kb^T D
                    const int kt = wave + 8 * j;
                    if (kt >= P::NMT_K) continue;
                    f32x4 acc;
                    acc[0] = S[j][0] * quad_bcast<0>(o.eg[j]);
                    acc[1] = S[j][1] * quad_bcast<1>(o.eg[j]);
                    acc[2] = S[j][2] * quad_bcast<2>(o.eg[j]);
                    acc[3] = S[j][3] * quad_bcast<3>(o.eg[j]);
#pragma unroll
                    for (int kk = 0; kk < P::NKK_T; ++kk)
                        acc = mfma16x16x32(o.kb[j][kk], *reinterpret_cast<const bf16x8*>(&sD[l16][32 * kk + 8 * g4]), acc);
                    bf16x4 s4;
#pragma unroll
                    for (int ii = 0; ii < 4; ++ii) {
                        S[j][ii] = acc[ii];
                        s4[ii] = static_cast<bf16>(acc[ii]);
                    }
                    *reinterpret_cast<bf16x4*>(&sS[l16][16 * kt + 4 * g4]) = s4;
                }
                // Chunk lc - 1 is published one step late, so that its stores are
                // long done and the wait costs nothing: they are older than the
                // previous step's parts 1 and 2 and all of this step's loads, so
                // they have reached L2 once at most that many operations remain
                // outstanding.  A wave without a token tile issues only its S
                // stores and parts 1 and 2 in a step, so allowing two steps' loads
                // outstanding leaves the previous step's stores done.
                asm volatile("" ::: "memory");
                if constexpr (ISD) wait_vmcnt<LOADS1 + LOADS2 + LOADS>();
                else wait_vmcnt<2 * (NKT_W + LOADS2)>();
                lds_barrier();                         // B2
                if (lc > 0) publish(lc);
            };
            Ops buf[NB];
#pragma unroll
            for (int b = 0; b < NB - 1; ++b) fetch(b, buf[b], AllParts{});
            lds_barrier();                             // B0: S_0 published
            run_steps<NB>(nch, buf, fetch, step);
            wait_vmcnt<0>();
            lds_barrier();
            publish(nch);
            checkpoint(nch - 1);
#pragma unroll
            for (int j = 0; j < NKT_W; ++j) {          // final state, in place
                const int kt = wave + 8 * j;
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    const int rr = 16 * kt + 4 * g4 + ii;
                    if (kt < P::NMT_K && rr < D) home[(int64_t)rr * D + col] = from_f32<ST>(S[j][ii]);
                }
            }
        };
        if (dwave) run(std::true_type{}); else run(std::false_type{});
        return;
    }

    // ---------------- output workgroup ----------------
    // With the norm fused the pair's output workgroups also publish, per
    // tile, how many chunks of o are stored (in L2, two steps late), and each
    // normalises its share of every chunk's rows once all tiles have stored
    // them: waves 5 and on (norm_rows, above).  Other waves past the loader
    // have no work.
    uint32_t* const nflag0 = NORM ? reinterpret_cast<uint32_t*>(ws + nrm.flag_off) + ((int64_t)seq * heads + h) * (D / 16)
                                  : nullptr;
    const StoredFlags<D> stored(nflag0, xcc, lane);
    __shared__ int sBroken;                        // a flag never came: write NaN
    if (wave > 4) {
        if constexpr (NORM) norm_rows<D, BT, AT>(wave - 5, lane, tile, nch, off, len, s_begin, h, out, os, nrm,
                                                 stored, &sBroken, status, max_spin);
        return;
    }
    if (wave == 4) {
        // Loader: chunk c's S and D land in stage c % kXchStages before the
        // barrier that ends step c - 1 (the prologue's barrier for c = 0).
        bool broken = false;
        auto wait_chunk = [&](int c) {             // until chunk c is published
            if (broken) return;
            uint32_t f = 0;
            for (int spin = 0; spin < max_spin; ++spin) {
                // Polled with device-scope atomic loads: a plain load can keep
                // hitting the CU's own cached copy of the flag.
                f = __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if ((f >> 24) == xcc && (f & 0xffffff) > (uint32_t)c) return;
                __builtin_amdgcn_s_sleep(2);
            }
            // A flag carrying another XCD's id: the pair was split across
            // XCDs; otherwise the producer never got this far.
            broken = true;
            raise_status(status, f != 0 && (f >> 24) != xcc ? kStatusPlacement : kStatusTimeout);
        };
        auto copy = [&](int c) {                   // 1 KB pieces, device-coherent at L2
            const uint8_t* src = xch + (int64_t)min(c, nch - 1) * XSLOT;
            uint8_t* dst = sX[c % kXchStages];
#pragma unroll
            for (int off = 0; off < XSLOT; off += kWave * 16)
                __builtin_amdgcn_global_load_lds((const void*)(src + off + lane * 16), (lds_void*)(dst + off), 16, 0,
                                                 kSkipL1);
        };
        constexpr int OPS = XSLOT / (kWave * 16);
        // With the norm fused: the o-stored flags, loaded at the end of a
        // step and checked at the end of the next.
        uint32_t fnext = 0;
        wait_chunk(0); copy(0);
        wait_chunk(min(1, nch - 1)); copy(1);
        wait_vmcnt<OPS>();                         // chunk 0 landed
        if (lane == 0) sBroken = broken;
        lds_barrier();                             // publishes chunk 0
        for (int c = 0; c < nch; ++c) {
            // Stage (c + 2) % 3 was read in step c - 1, which ended at the
            // barrier above.
            wait_chunk(min(c + 2, nch - 1));
            copy(c + 2);
            wait_vmcnt<OPS>();                     // chunk c + 1 landed
            if constexpr (NORM) {
                // Every tile has stored c - kNormCheckLag chunks before this
                // step ends (the norm waves' loads of the next step need it).
                const int n = c - kNormCheckLag;
                if (n > 0 && !broken && !stored.at(fnext, n)) broken = !stored.wait(n, lane, max_spin, status);
                fnext = stored.load(lane);
            }
            if (lane == 0 && broken) sBroken = 1;
            lds_barrier();                         // end of step c
        }
        wait_vmcnt<0>();
        return;
    }
    // Output waves.
    // O^T = S^T Q~^T + D^T Aqk^T: with the operands of O = Q~ S + Aqk D
    // swapped, lane l holds 4 consecutive columns of output row
    // 16 tt + l % 16 and writes them with one vector store.
    const bool active = wave < NS;
    const int tt = active ? wave : 0;              // token tile
    const int kmax = (16 * tt + 15) / 32;          // Aqk is zero beyond the diagonal
    const int r = 16 * tt + l16;
    struct Ops {
        bf16x8 q[P::NKK_K];                        // Q~ rows of token tile tt
        bf16x8 a[P::NKK_T];                        // Aqk rows of token tile tt
    };
    auto fetch = [&](int lc, Ops& o) {
        const bf16* rec = record(lc);
#pragma unroll
        for (int kk = 0; kk < P::NKK_K; ++kk)
            o.q[kk] = *reinterpret_cast<const bf16x8*>(rec + P::OFF_Q + frag<DKP>(r, 32 * kk + 8 * g4));
#pragma unroll
        for (int kk = 0; kk < P::NKK_T; ++kk)
            o.a[kk] = *reinterpret_cast<const bf16x8*>(rec + P::OFF_A + aq_frag(r, 32 * min(kk, kmax) + 8 * g4));
    };
    // Loads per step of an output wave (all unconditional).
    constexpr int LOADS_O = P::NKK_K + P::NKK_T;
    // With the norm fused, this tile's o-stored count goes out at the end of
    // each step: o of step lc - 2 is in L2 once at most two steps' loads
    // remain outstanding (its store is older than both).  Like the chain's
    // own flag, a workgroup-scope store that lands in the XCD's L2, where the
    // pair's other workgroups read it: an agent-scope store would be written
    // through to memory and hold up this wave's later waits.
    auto publish_o = [&](int n) {
        if (wave == 0 && lane == 0)
            __hip_atomic_store(nflag0 + tile, (xcc << 24) | (uint32_t)n, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_WORKGROUP);
    };
    auto step = [&](int lc, const Ops& o, auto refill) {
        refill();
        if (active) {
            const uint8_t* x = sX[lc % kXchStages];
            f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < P::NKK_K; ++kk) {
                const bf16x8 sf = *reinterpret_cast<const bf16x8*>(x + (kk * kWave + lane) * 16);
                if (kk & 1) acc1 = mfma16x16x32(sf, o.q[kk], acc1);
                else acc0 = mfma16x16x32(sf, o.q[kk], acc0);
            }
#pragma unroll
            for (int kk = 0; kk < P::NKK_T; ++kk)
                if (kk <= kmax)
                    acc0 = mfma16x16x32(*reinterpret_cast<const bf16x8*>(x + XS_BYTES + (kk * kWave + lane) * 16),
                                        o.a[kk], acc0);
            const int cbeg = chunk_begin(lc, BT, off);
            const int64_t tc = s_begin + cbeg;
            if (r < chunk_end(lc, len, BT, off) - cbeg) {
                const float bad = sBroken ? __builtin_nanf("") : 1.0f;
                float o4[4];
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) o4[ii] = bad * scale * (acc0[ii] + acc1[ii]);
                store4(out + (tc + r) * os + (int64_t)h * D + n0 + 4 * g4, o4);
            }
        }
        if constexpr (NORM) wait_vmcnt<2 * LOADS_O>();
        lds_barrier();                             // end of step lc
        if constexpr (NORM)
            if (lc >= 1) publish_o(lc - 1);
    };
    Ops buf[NB];
#pragma unroll
    for (int b = 0; b < NB - 1; ++b) fetch(b, buf[b]);
    lds_barrier();                                 // chunk 0 of S and D in LDS
    run_steps<NB>(nch, buf, fetch, step);
    if constexpr (NORM) {
        wait_vmcnt<0>();
        lds_barrier();                             // every output wave's stores done
        publish_o(nch);
    }
}

// Clears the status word and the chain kernel's flags for a call without
// tokens (otherwise the intra kernel does it).
__global__ __launch_bounds__(kThreads)
void prefill_clear_kernel(uint32_t* __restrict__ status, uint32_t* __restrict__ flags, int64_t n_flags)
{
    if (threadIdx.x == 0) *status = 0u;
    for (int64_t i = threadIdx.x; i < n_flags; i += kThreads) flags[i] = 0u;
}

// ---------------------------------------------------------------------------
// Workspace, past the header: the records, then the chain's exchange slots
// (per head and column tile, one per chunk slot), then one flag per
// (sequence, head, tile).
struct WorkspaceLayout {
    int64_t chunks, xch_off, flag_off, n_flags, nflag_off, bytes;
};
// With the norm fused the flags are followed by as many o-stored flags (so
// the intra kernel clears both in one sweep).
template <int D, int BT>
WorkspaceLayout workspace_layout(int32_t num_seqs, int64_t total_tokens, int32_t heads, bool norm = false)
{
    using P = Shape<D, BT>;
    WorkspaceLayout l;
    l.chunks = max_chunks(num_seqs, total_tokens, BT);
    const int64_t xslot = 16 * (P::DKP + P::BTP) * 2;
    l.xch_off = l.chunks * heads * P::REC_BYTES;
    l.flag_off = l.xch_off + (int64_t)heads * (D / 16) * l.chunks * xslot;
    l.n_flags = (int64_t)num_seqs * heads * (D / 16);
    l.nflag_off = l.flag_off + l.n_flags * 4;
    l.bytes = kHeaderBytes + l.flag_off + ((norm ? 2 : 1) * l.n_flags * 4 + 255) / 256 * 256;
    return l;
}

template <int D, int BT, typename AT, typename ST>
hipError_t launch_typed(const PrefillArgs& a, hipStream_t stream)
{
    const bool norm = a.norm_y != nullptr;
    const WorkspaceLayout lay = workspace_layout<D, BT>(a.num_seqs, a.total_tokens, a.heads, norm);
    const int64_t chunks = lay.chunks;
    const int64_t n_clear = norm ? 2 * lay.n_flags : lay.n_flags;   // chain (and norm) flags
    if (chunks * a.heads * kThreads > (int64_t)UINT32_MAX) return hipErrorInvalidValue;   // 1-D intra grid
    const int64_t pairs = ((int64_t)a.num_seqs * a.heads + 7) / 8 * 8;
    if (pairs > INT32_MAX) return hipErrorInvalidValue;
    uint32_t* const status = static_cast<uint32_t*>(a.workspace);
    uint8_t* const ws = static_cast<uint8_t*>(a.workspace) + kHeaderBytes;
    if (a.total_tokens > 0) {
        ConvIn<AT> cv;
        cv.w = static_cast<const AT*>(a.conv_w);
        cv.b = static_cast<const AT*>(a.conv_b);
        cv.state = static_cast<AT*>(a.conv_state);
        cv.has_init = a.has_init;
        cv.num_slots = a.num_slots;
        cv.channels = 3 * (int64_t)a.heads * D;
        cv.width = a.conv_width;
        cv.silu = (a.conv_flags & KDA_CONV_SILU) != 0;
        const dim3 grid((unsigned)(chunks * a.heads));
        if (a.conv_width > 0)
            hipLaunchKernelGGL((intra_kernel<D, BT, AT, true>), grid, dim3(kThreads), 0, stream,
                               static_cast<const AT*>(a.q), static_cast<const AT*>(a.k),
                               static_cast<const AT*>(a.v), a.q_stride, a.k_stride, a.v_stride, a.g,
                               a.beta, a.cu_seqlens, a.num_seqs, a.heads, a.slots, a.flags,
                               a.seq_pos, ws, lay.flag_off, n_clear, status, cv);
        else
            hipLaunchKernelGGL((intra_kernel<D, BT, AT, false>), grid, dim3(kThreads), 0, stream,
                               static_cast<const AT*>(a.q), static_cast<const AT*>(a.k),
                               static_cast<const AT*>(a.v), a.q_stride, a.k_stride, a.v_stride, a.g,
                               a.beta, a.cu_seqlens, a.num_seqs, a.heads, a.slots, a.flags,
                               a.seq_pos, ws, lay.flag_off, n_clear, status, cv);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    } else {
        // No tokens, so no intra kernel to clear the flags and the status
        // word: a one-workgroup kernel does it.
        hipLaunchKernelGGL(prefill_clear_kernel, dim3(1), dim3(kThreads), 0, stream, status,
                           reinterpret_cast<uint32_t*>(ws + lay.flag_off), n_clear);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    NormIn<AT> nrm;
    nrm.gate = static_cast<const AT*>(a.norm_gate);
    nrm.gs = a.norm_gate_stride;
    nrm.w = static_cast<const AT*>(a.norm_weight);
    nrm.y = static_cast<AT*>(a.norm_y);
    nrm.ys = a.norm_y_stride;
    nrm.eps = a.norm_eps;
    nrm.flag_off = lay.nflag_off;
    const int spin = (a.flags & KDA_FLAG_DIAG_GIVE_UP) ? 0 : kMaxSpin;
    const int64_t plane = pairs * (D / 16);         // workgroups of one role
    if (2 * plane > (int64_t)UINT32_MAX) return hipErrorInvalidValue;
    bool pack = false;
    if constexpr (D == 128) {
        // At d = 128 the chain kernel needs more than 128 registers per lane,
        // so it runs one workgroup per CU unless compiled with PACK (not for
        // fp32 activations with the fused norm, whose build needs ~190).
        const bool packable = !norm || std::is_same<AT, bf16>::value;
        if (packable && a.total_tokens <= (int64_t)kPackMaxChunks * BT * a.num_seqs) {
            int dev = 0, cus = 0;
            if (hipGetDevice(&dev) == hipSuccess &&
                hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
                pack = 2 * plane > (int64_t)cus;
            else
                (void)hipGetLastError();            // fall back to one workgroup per CU
        }
    }
    if (norm && pack) {
        if constexpr (D == 128 && std::is_same<AT, bf16>::value)
            hipLaunchKernelGGL((chain_kernel<D, BT, AT, ST, true, true>), dim3((unsigned)(2 * plane)),
                               dim3(kChainThreads), 0, stream, a.cu_seqlens, a.seq_pos, a.num_seqs,
                               a.heads, static_cast<ST*>(a.pool), a.num_slots, a.slots, a.has_init,
                               static_cast<ST*>(a.ckpt), a.ckpt_capacity, a.ckpt_interval, a.scale,
                               static_cast<AT*>(a.out), a.out_stride, ws,
                               lay.xch_off, lay.chunks, lay.flag_off, status, spin, nrm);
    } else if (norm) {
        hipLaunchKernelGGL((chain_kernel<D, BT, AT, ST, true, false>), dim3((unsigned)(2 * plane)),
                           dim3(kChainThreads), 0, stream, a.cu_seqlens, a.seq_pos, a.num_seqs, a.heads,
                           static_cast<ST*>(a.pool), a.num_slots, a.slots, a.has_init,
                           static_cast<ST*>(a.ckpt), a.ckpt_capacity, a.ckpt_interval, a.scale,
                           static_cast<AT*>(a.out), a.out_stride, ws,
                           lay.xch_off, lay.chunks, lay.flag_off, status, spin, nrm);
    } else if (pack) {
        if constexpr (D == 128)
            hipLaunchKernelGGL((chain_kernel<D, BT, AT, ST, false, true>), dim3((unsigned)(2 * plane)),
                               dim3(kChainThreads), 0, stream, a.cu_seqlens, a.seq_pos, a.num_seqs,
                               a.heads, static_cast<ST*>(a.pool), a.num_slots, a.slots, a.has_init,
                               static_cast<ST*>(a.ckpt), a.ckpt_capacity, a.ckpt_interval, a.scale,
                               static_cast<AT*>(a.out), a.out_stride, ws,
                               lay.xch_off, lay.chunks, lay.flag_off, status, spin, nrm);
    } else {
        hipLaunchKernelGGL((chain_kernel<D, BT, AT, ST, false, false>), dim3((unsigned)(2 * plane)),
                           dim3(kChainThreads), 0, stream, a.cu_seqlens, a.seq_pos, a.num_seqs, a.heads,
                           static_cast<ST*>(a.pool), a.num_slots, a.slots, a.has_init,
                           static_cast<ST*>(a.ckpt), a.ckpt_capacity, a.ckpt_interval, a.scale,
                           static_cast<AT*>(a.out), a.out_stride, ws,
                           lay.xch_off, lay.chunks, lay.flag_off, status, spin, nrm);
    }
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

}  // namespace

size_t prefill_workspace_bytes(int32_t num_seqs, int64_t total_tokens, int32_t heads, int32_t dk,
                               int32_t dv, int32_t chunk, bool norm)
{
    if (dk != dv) return 0;
    auto by_chunk = [&](auto dtag) -> int64_t {
        constexpr int D = decltype(dtag)::value;
        switch (chunk) {
            case 16: return workspace_layout<D, 16>(num_seqs, total_tokens, heads, norm).bytes;
            case 32: return workspace_layout<D, 32>(num_seqs, total_tokens, heads, norm).bytes;
            case 64: return workspace_layout<D, 64>(num_seqs, total_tokens, heads, norm).bytes;
            default: return 0;
        }
    };
    switch (dk) {
        case 16: return (size_t)by_chunk(std::integral_constant<int, 16>{});
        case 32: return (size_t)by_chunk(std::integral_constant<int, 32>{});
        case 64: return (size_t)by_chunk(std::integral_constant<int, 64>{});
        case 128: return (size_t)by_chunk(std::integral_constant<int, 128>{});
        default: return 0;
    }
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
