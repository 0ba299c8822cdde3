// kda_api.hip -- the C ABI declared in include/kda.h: argument validation and
// dispatch to the kernel launchers.  Every check here runs on the host before
// any HIP call, so a rejected call enqueues nothing and touches no device.

#include <stdint.h>
#include <string.h>

#include <mutex>

#include "kda_internal.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned8(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }
bool dtype_ok(kda_dtype_t t) { return t == KDA_F32 || t == KDA_BF16; }
bool dim_ok(int32_t d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool chunk_ok(int32_t c) { return c == 16 || c == 32 || c == 64; }

kda_status_t launch_status(hipError_t e)
{
    return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int kda_abi_version(void) { return KDA_ABI_VERSION; }

const char* kda_status_string(kda_status_t status)
{
    switch (status) {
        case KDA_OK: return "ok";
        case KDA_ERR_INVALID_ARG: return "invalid argument";
        case KDA_ERR_UNSUPPORTED: return "unsupported shape, dtype, chunk size or interval";
        case KDA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
        case KDA_ERR_LAUNCH: return "kernel launch failed";
        case KDA_ERR_DEVICE: return "the device reported a failed call";
        case KDA_ERR_SCRATCH_LIMIT: return "the call needs more than the library's fixed scratch area";
        default: return "unknown status";
    }
}

size_t kda_chunk_prefill_workspace_size(int32_t num_seqs, int64_t total_tokens,
                                        int32_t num_heads, int32_t dk, int32_t dv,
                                        int32_t chunk_size)
{
    if (num_seqs < 0 || total_tokens < 0 || num_heads <= 0) return 0;
    if (!dim_ok(dk) || dk != dv || !chunk_ok(chunk_size)) return 0;
    return kda::prefill_workspace_bytes(num_seqs, total_tokens, num_heads, dk, dv, chunk_size);
}

size_t kda_chunk_prefill_norm_workspace_size(int32_t num_seqs, int64_t total_tokens,
                                             int32_t num_heads, int32_t dk, int32_t dv,
                                             int32_t chunk_size)
{
    if (num_seqs < 0 || total_tokens < 0 || num_heads <= 0) return 0;
    if (!dim_ok(dk) || dk != dv || !chunk_ok(chunk_size)) return 0;
    return kda::prefill_workspace_bytes(num_seqs, total_tokens, num_heads, dk, dv, chunk_size, true);
}

namespace {

// Checks and fills everything the two prefill entry points share.  q, k, v
// may be null when total_tokens is 0.
kda_status_t prefill_common(
    kda::PrefillArgs& a,
    const void* q, const void* k, const void* v, kda_dtype_t act_dtype,
    int64_t q_stride_t, int64_t k_stride_t, int64_t v_stride_t,
    const float* g, const float* beta,
    const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
    int32_t num_heads, int32_t dk, int32_t dv,
    void* state_pool, kda_dtype_t state_dtype, int64_t num_slots,
    const int32_t* state_indices, const uint8_t* has_initial_state,
    void* checkpoints, int64_t ckpt_capacity, int32_t ckpt_interval,
    float scale, int32_t chunk_size, uint32_t flags,
    void* out, int64_t out_stride_t,
    void* workspace, size_t workspace_bytes)
{
    if (num_seqs < 0 || total_tokens < 0 || num_heads <= 0 || num_slots < 0 ||
        ckpt_capacity < 0 || ckpt_interval < 0)
        return KDA_ERR_INVALID_ARG;
    if (!dtype_ok(act_dtype) || !dtype_ok(state_dtype)) return KDA_ERR_INVALID_ARG;
    if (flags & ~(KDA_FLAG_QK_L2NORM | KDA_FLAG_DIAG_GIVE_UP)) return KDA_ERR_INVALID_ARG;
    if (!dim_ok(dk) || dk != dv || !chunk_ok(chunk_size)) return KDA_ERR_UNSUPPORTED;
    if (ckpt_interval > 0 && ckpt_interval % chunk_size != 0) return KDA_ERR_UNSUPPORTED;
    if (num_seqs == 0) return KDA_OK;
    if (!cu_seqlens || !state_indices) return KDA_ERR_INVALID_ARG;
    if (total_tokens > 0 && (!q || !k || !v || !g || !beta || !out)) return KDA_ERR_INVALID_ARG;
    if (num_slots > 0 && !state_pool) return KDA_ERR_INVALID_ARG;
    if (ckpt_interval > 0 && ckpt_capacity > 0 && !checkpoints) return KDA_ERR_INVALID_ARG;
    const int64_t hk = (int64_t)num_heads * dk, hv = (int64_t)num_heads * dv;
    if (q_stride_t < hk || k_stride_t < hk || v_stride_t < hv || out_stride_t < hv)
        return KDA_ERR_INVALID_ARG;
    if ((q_stride_t | k_stride_t | v_stride_t | out_stride_t) & 7) return KDA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(g) || !aligned16(out) ||
        !aligned16(state_pool) || !aligned16(checkpoints))
        return KDA_ERR_INVALID_ARG;
    const size_t need = kda::prefill_workspace_bytes(num_seqs, total_tokens, num_heads, dk, dv,
                                                     chunk_size);
    if (workspace_bytes < need) return KDA_ERR_WORKSPACE_TOO_SMALL;
    if (need > 0 && (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u)))
        return KDA_ERR_INVALID_ARG;

    a.q = q; a.k = k; a.v = v;
    a.q_stride = q_stride_t; a.k_stride = k_stride_t; a.v_stride = v_stride_t;
    a.g = g; a.beta = beta;
    a.cu_seqlens = cu_seqlens; a.num_seqs = num_seqs; a.total_tokens = total_tokens;
    a.heads = num_heads; a.dk = dk; a.dv = dv;
    a.pool = state_pool; a.num_slots = num_slots;
    a.slots = state_indices; a.has_init = has_initial_state;
    a.ckpt = (ckpt_interval > 0) ? checkpoints : nullptr;
    a.ckpt_capacity = (ckpt_interval > 0 && checkpoints) ? ckpt_capacity : 0;
    a.ckpt_interval = ckpt_interval;
    a.scale = scale; a.chunk = chunk_size; a.flags = flags;
    a.out = out; a.out_stride = out_stride_t;
    a.workspace = workspace;
    a.act = act_dtype; a.state = state_dtype;
    a.seq_pos = nullptr;
    a.conv_w = a.conv_b = nullptr; a.conv_state = nullptr;
    a.conv_width = 0; a.conv_flags = 0;
    a.norm_gate = nullptr; a.norm_gate_stride = 0; a.norm_weight = nullptr;
    a.norm_eps = 0.0f; a.norm_y = nullptr; a.norm_y_stride = 0;
    return KDA_OK;
}

// Checks the fused norm's arguments and the larger workspace it needs, and
// fills them in (after prefill_common).
kda_status_t norm_common(kda::PrefillArgs& a, const void* norm_gate, int64_t norm_gate_stride_t,
                         const void* norm_weight, float norm_eps, void* norm_out,
                         int64_t norm_out_stride_t, size_t workspace_bytes)
{
    if (!(norm_eps >= 0.0f)) return KDA_ERR_INVALID_ARG;
    const int64_t hv = (int64_t)a.heads * a.dv;
    if (a.total_tokens > 0 && (!norm_gate || !norm_out)) return KDA_ERR_INVALID_ARG;
    if (norm_gate_stride_t < hv || norm_out_stride_t < hv) return KDA_ERR_INVALID_ARG;
    if ((norm_gate_stride_t | norm_out_stride_t) & 7) return KDA_ERR_INVALID_ARG;
    // out is read back through 32-bit byte offsets from a chunk's first row.
    const int64_t esz = a.act == KDA_BF16 ? 2 : 4;
    if ((int64_t)a.chunk * a.out_stride * esz >= ((int64_t)1 << 31)) return KDA_ERR_INVALID_ARG;
    if (!aligned16(norm_gate) || !aligned16(norm_weight) || !aligned16(norm_out))
        return KDA_ERR_INVALID_ARG;
    const size_t need = kda::prefill_workspace_bytes(a.num_seqs, a.total_tokens, a.heads, a.dk,
                                                     a.dv, a.chunk, true);
    if (workspace_bytes < need) return KDA_ERR_WORKSPACE_TOO_SMALL;
    a.norm_gate = norm_gate; a.norm_gate_stride = norm_gate_stride_t;
    a.norm_weight = norm_weight; a.norm_eps = norm_eps;
    a.norm_y = a.total_tokens > 0 ? norm_out : nullptr;
    a.norm_y_stride = norm_out_stride_t;
    return KDA_OK;
}

}  // namespace

kda_status_t kda_chunk_prefill(
    const void* q, const void* k, const void* v, kda_dtype_t act_dtype,
    int64_t q_stride_t, int64_t k_stride_t, int64_t v_stride_t,
    const float* g, const float* beta,
    const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
    int32_t num_heads, int32_t dk, int32_t dv,
    void* state_pool, kda_dtype_t state_dtype, int64_t num_slots,
    const int32_t* state_indices, const uint8_t* has_initial_state,
    void* checkpoints, int64_t ckpt_capacity, int32_t ckpt_interval,
    float scale, int32_t chunk_size, uint32_t flags,
    void* out, int64_t out_stride_t,
    void* workspace, size_t workspace_bytes, void* stream)
{
    kda::PrefillArgs a;
    const kda_status_t st = prefill_common(
        a, q, k, v, act_dtype, q_stride_t, k_stride_t, v_stride_t, g, beta, cu_seqlens, num_seqs,
        total_tokens, num_heads, dk, dv, state_pool, state_dtype, num_slots, state_indices,
        has_initial_state, checkpoints, ckpt_capacity, ckpt_interval, scale, chunk_size, flags, out,
        out_stride_t, workspace, workspace_bytes);
    if (st != KDA_OK || num_seqs == 0) return st;
    return launch_status(kda::launch_prefill(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// Scratch of kda_chunk_prefill_noalloc: a fixed array in device memory that
// every GPU the library runs on holds from module load to process end, sized
// for one 4096-token sequence with 16 heads of d = 128 at chunk 64 (that
// call's workspace is 130.3 MB).  Host code never passes the array's name to
// a kernel or a copy (on the host it names a stand-in, not device memory):
// it uses the device address that hipGetSymbolAddress returns, looked up
// once per device with that device current and kept in g_scratch.
constexpr size_t kStaticScratchBytes = size_t(128) << 20;
__device__ __align__(256) uint8_t scratch[kStaticScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch[kMaxDevices];

// The current device's copy of `scratch`.
hipError_t scratch_address(void** out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

kda_status_t kda_chunk_prefill_noalloc(
    const void* q, const void* k, const void* v, kda_dtype_t act_dtype,
    int64_t q_stride_t, int64_t k_stride_t, int64_t v_stride_t,
    const float* g, const float* beta,
    const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
    int32_t num_heads, int32_t dk, int32_t dv,
    void* state_pool, kda_dtype_t state_dtype, int64_t num_slots,
    const int32_t* state_indices, const uint8_t* has_initial_state,
    void* checkpoints, int64_t ckpt_capacity, int32_t ckpt_interval,
    float scale, int32_t chunk_size, uint32_t flags,
    void* out, int64_t out_stride_t, void* stream)
{
    // Validated against the fixed area's size with a stand-in address (the
    // checks only look at its alignment), so a rejected call still makes no
    // HIP call.
    void* const stand_in = reinterpret_cast<void*>(uintptr_t(256));
    kda::PrefillArgs a;
    const kda_status_t st = prefill_common(
        a, q, k, v, act_dtype, q_stride_t, k_stride_t, v_stride_t, g, beta, cu_seqlens, num_seqs,
        total_tokens, num_heads, dk, dv, state_pool, state_dtype, num_slots, state_indices,
        has_initial_state, checkpoints, ckpt_capacity, ckpt_interval, scale, chunk_size, flags, out,
        out_stride_t, stand_in, kStaticScratchBytes);
    if (st == KDA_ERR_WORKSPACE_TOO_SMALL) return KDA_ERR_SCRATCH_LIMIT;
    if (st != KDA_OK || num_seqs == 0) return st;
    void* ws = nullptr;
    if (scratch_address(&ws) != hipSuccess) return KDA_ERR_LAUNCH;
    a.workspace = ws;
    return launch_status(kda::launch_prefill(a, static_cast<hipStream_t>(stream)));
}

kda_status_t kda_chunk_prefill_check(const void* workspace, size_t workspace_bytes,
                                     uint32_t* device_flags, void* stream)
{
    if (!workspace || workspace_bytes < 4) return KDA_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint32_t word = 0;
    if (hipStreamSynchronize(s) != hipSuccess) return KDA_ERR_LAUNCH;
    if (hipMemcpy(&word, workspace, sizeof(word), hipMemcpyDeviceToHost) != hipSuccess)
        return KDA_ERR_LAUNCH;
    if (device_flags) *device_flags = word;
    return word == 0 ? KDA_OK : KDA_ERR_DEVICE;
}

kda_status_t kda_chunk_prefill_at(
    const void* q, const void* k, const void* v, kda_dtype_t act_dtype,
    int64_t q_stride_t, int64_t k_stride_t, int64_t v_stride_t,
    const float* g, const float* beta,
    const int32_t* cu_seqlens, const int64_t* seq_start_pos, int32_t num_seqs,
    int64_t total_tokens, int32_t num_heads, int32_t dk, int32_t dv,
    void* state_pool, kda_dtype_t state_dtype, int64_t num_slots,
    const int32_t* state_indices, const uint8_t* has_initial_state,
    void* checkpoints, int64_t ckpt_capacity, int32_t ckpt_interval,
    float scale, int32_t chunk_size, uint32_t flags,
    void* out, int64_t out_stride_t,
    void* workspace, size_t workspace_bytes, void* stream)
{
    kda::PrefillArgs a;
    const kda_status_t st = prefill_common(
        a, q, k, v, act_dtype, q_stride_t, k_stride_t, v_stride_t, g, beta, cu_seqlens, num_seqs,
        total_tokens, num_heads, dk, dv, state_pool, state_dtype, num_slots, state_indices,
        has_initial_state, checkpoints, ckpt_capacity, ckpt_interval, scale, chunk_size, flags, out,
        out_stride_t, workspace, workspace_bytes);
    if (st != KDA_OK || num_seqs == 0) return st;
    if (!aligned8(seq_start_pos)) return KDA_ERR_INVALID_ARG;
    a.seq_pos = seq_start_pos;
    return launch_status(kda::launch_prefill(a, static_cast<hipStream_t>(stream)));
}

kda_status_t kda_conv_chunk_prefill(
    const void* x, int64_t x_stride_t, kda_dtype_t act_dtype,
    const void* conv_weight, const void* conv_bias, int32_t conv_width, uint32_t conv_flags,
    void* conv_state_pool,
    const float* g, const float* beta,
    const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
    int32_t num_heads, int32_t dk, int32_t dv,
    void* state_pool, kda_dtype_t state_dtype, int64_t num_slots,
    const int32_t* state_indices, const uint8_t* has_initial_state,
    void* checkpoints, int64_t ckpt_capacity, int32_t ckpt_interval,
    float scale, int32_t chunk_size, uint32_t flags,
    void* out, int64_t out_stride_t,
    void* workspace, size_t workspace_bytes, void* stream)
{
    if (conv_width < 2 || conv_width > 8) return KDA_ERR_UNSUPPORTED;
    if (conv_flags & ~KDA_CONV_SILU) return KDA_ERR_INVALID_ARG;
    if (!dtype_ok(act_dtype)) return KDA_ERR_INVALID_ARG;
    const int64_t hd = (int64_t)num_heads * dk;
    if (num_heads > 0 && x_stride_t < 3 * hd) return KDA_ERR_INVALID_ARG;
    const size_t es = act_dtype == KDA_BF16 ? 2 : 4;
    const char* xb = static_cast<const char*>(x);
    const bool have_x = total_tokens > 0 && x;
    kda::PrefillArgs a;
    const kda_status_t st = prefill_common(
        a, x, have_x ? xb + hd * es : nullptr, have_x ? xb + 2 * hd * es : nullptr, act_dtype,
        x_stride_t, x_stride_t, x_stride_t, g, beta, cu_seqlens, num_seqs, total_tokens, num_heads,
        dk, dv, state_pool, state_dtype, num_slots, state_indices, has_initial_state, checkpoints,
        ckpt_capacity, ckpt_interval, scale, chunk_size, flags, out, out_stride_t, workspace,
        workspace_bytes);
    if (st != KDA_OK || num_seqs == 0) return st;
    if (total_tokens > 0 && !conv_weight) return KDA_ERR_INVALID_ARG;
    if (num_slots > 0 && !conv_state_pool) return KDA_ERR_INVALID_ARG;
    if (!aligned16(conv_weight) || !aligned16(conv_bias) || !aligned16(conv_state_pool))
        return KDA_ERR_INVALID_ARG;
    a.conv_w = conv_weight; a.conv_b = conv_bias; a.conv_state = conv_state_pool;
    a.conv_width = conv_width; a.conv_flags = conv_flags;
    return launch_status(kda::launch_prefill(a, static_cast<hipStream_t>(stream)));
}

kda_status_t kda_chunk_prefill_norm(
    const void* q, const void* k, const void* v, kda_dtype_t act_dtype,
    int64_t q_stride_t, int64_t k_stride_t, int64_t v_stride_t,
    const float* g, const float* beta,
    const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
    int32_t num_heads, int32_t dk, int32_t dv,
    void* state_pool, kda_dtype_t state_dtype, int64_t num_slots,
    const int32_t* state_indices, const uint8_t* has_initial_state,
    void* checkpoints, int64_t ckpt_capacity, int32_t ckpt_interval,
    float scale, int32_t chunk_size, uint32_t flags,
    void* out, int64_t out_stride_t,
    const void* norm_gate, int64_t norm_gate_stride_t, const void* norm_weight, float norm_eps,
    void* norm_out, int64_t norm_out_stride_t,
    void* workspace, size_t workspace_bytes, void* stream)
{
    kda::PrefillArgs a;
    kda_status_t st = prefill_common(
        a, q, k, v, act_dtype, q_stride_t, k_stride_t, v_stride_t, g, beta, cu_seqlens, num_seqs,
        total_tokens, num_heads, dk, dv, state_pool, state_dtype, num_slots, state_indices,
        has_initial_state, checkpoints, ckpt_capacity, ckpt_interval, scale, chunk_size, flags, out,
        out_stride_t, workspace, workspace_bytes);
    if (st != KDA_OK || num_seqs == 0) return st;
    st = norm_common(a, norm_gate, norm_gate_stride_t, norm_weight, norm_eps, norm_out,
                     norm_out_stride_t, workspace_bytes);
    if (st != KDA_OK) return st;
    return launch_status(kda::launch_prefill(a, static_cast<hipStream_t>(stream)));
}

kda_status_t kda_conv_chunk_prefill_norm(
    const void* x, int64_t x_stride_t, kda_dtype_t act_dtype,
    const void* conv_weight, const void* conv_bias, int32_t conv_width, uint32_t conv_flags,
    void* conv_state_pool,
    const float* g, const float* beta,
    const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
    int32_t num_heads, int32_t dk, int32_t dv,
    void* state_pool, kda_dtype_t state_dtype, int64_t num_slots,
    const int32_t* state_indices, const uint8_t* has_initial_state,
    void* checkpoints, int64_t ckpt_capacity, int32_t ckpt_interval,
    float scale, int32_t chunk_size, uint32_t flags,
    void* out, int64_t out_stride_t,
    const void* norm_gate, int64_t norm_gate_stride_t, const void* norm_weight, float norm_eps,
    void* norm_out, int64_t norm_out_stride_t,
    void* workspace, size_t workspace_bytes, void* stream)
{
    if (conv_width < 2 || conv_width > 8) return KDA_ERR_UNSUPPORTED;
    if (conv_flags & ~KDA_CONV_SILU) return KDA_ERR_INVALID_ARG;
    if (!dtype_ok(act_dtype)) return KDA_ERR_INVALID_ARG;
    const int64_t hd = (int64_t)num_heads * dk;
    if (num_heads > 0 && x_stride_t < 3 * hd) return KDA_ERR_INVALID_ARG;
    const size_t es = act_dtype == KDA_BF16 ? 2 : 4;
    const char* xb = static_cast<const char*>(x);
    const bool have_x = total_tokens > 0 && x;
    kda::PrefillArgs a;
    kda_status_t st = prefill_common(
        a, x, have_x ? xb + hd * es : nullptr, have_x ? xb + 2 * hd * es : nullptr, act_dtype,
        x_stride_t, x_stride_t, x_stride_t, g, beta, cu_seqlens, num_seqs, total_tokens, num_heads,
        dk, dv, state_pool, state_dtype, num_slots, state_indices, has_initial_state, checkpoints,
        ckpt_capacity, ckpt_interval, scale, chunk_size, flags, out, out_stride_t, workspace,
        workspace_bytes);
    if (st != KDA_OK || num_seqs == 0) return st;
    if (total_tokens > 0 && !conv_weight) return KDA_ERR_INVALID_ARG;
    if (num_slots > 0 && !conv_state_pool) return KDA_ERR_INVALID_ARG;
    if (!aligned16(conv_weight) || !aligned16(conv_bias) || !aligned16(conv_state_pool))
        return KDA_ERR_INVALID_ARG;
    st = norm_common(a, norm_gate, norm_gate_stride_t, norm_weight, norm_eps, norm_out,
                     norm_out_stride_t, workspace_bytes);
    if (st != KDA_OK) return st;
    a.conv_w = conv_weight; a.conv_b = conv_bias; a.conv_state = conv_state_pool;
    a.conv_width = conv_width; a.conv_flags = conv_flags;
    return launch_status(kda::launch_prefill(a, static_cast<hipStream_t>(stream)));
}

kda_status_t kda_recurrent_decode(
    const void* q, const void* k, const void* v, kda_dtype_t act_dtype,
    int64_t q_stride_b, int64_t k_stride_b, int64_t v_stride_b,
    const float* g, const float* beta,
    int32_t batch, int32_t num_heads, int32_t dk, int32_t dv,
    void* state_pool, kda_dtype_t state_dtype, int64_t num_slots,
    const int32_t* state_indices, float scale, uint32_t flags,
    void* out, int64_t out_stride_b, void* stream)
{
    if (batch < 0 || num_heads <= 0 || num_slots < 0) return KDA_ERR_INVALID_ARG;
    if (!dtype_ok(act_dtype) || !dtype_ok(state_dtype)) return KDA_ERR_INVALID_ARG;
    if (flags & ~KDA_FLAG_QK_L2NORM) return KDA_ERR_INVALID_ARG;
    if (!dim_ok(dk) || dk != dv) return KDA_ERR_UNSUPPORTED;
    if (batch == 0) return KDA_OK;
    if (!q || !k || !v || !g || !beta || !state_indices || !out) return KDA_ERR_INVALID_ARG;
    if (num_slots > 0 && !state_pool) return KDA_ERR_INVALID_ARG;
    const int64_t hk = (int64_t)num_heads * dk, hv = (int64_t)num_heads * dv;
    if (q_stride_b < hk || k_stride_b < hk || v_stride_b < hv || out_stride_b < hv)
        return KDA_ERR_INVALID_ARG;
    if ((q_stride_b | k_stride_b | v_stride_b | out_stride_b) & 7) return KDA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
        !aligned16(state_pool))
        return KDA_ERR_INVALID_ARG;
    if ((int64_t)batch * num_heads > INT32_MAX) return KDA_ERR_UNSUPPORTED;

    kda::DecodeArgs a;
    a.q = q; a.k = k; a.v = v;
    a.q_stride = q_stride_b; a.k_stride = k_stride_b; a.v_stride = v_stride_b;
    a.g = g; a.beta = beta;
    a.batch = batch; a.ntok = 1; a.heads = num_heads; a.dk = dk; a.dv = dv;
    a.pool = state_pool; a.num_slots = num_slots; a.slots = state_indices;
    a.token_states = nullptr;
    a.scale = scale; a.flags = flags;
    a.out = out; a.out_stride = out_stride_b;
    a.act = act_dtype; a.state = state_dtype;
    return launch_status(kda::launch_decode(a, static_cast<hipStream_t>(stream)));
}

kda_status_t kda_spec_decode(
    const void* q, const void* k, const void* v, kda_dtype_t act_dtype,
    int64_t q_stride_t, int64_t k_stride_t, int64_t v_stride_t,
    const float* g, const float* beta,
    int32_t batch, int32_t ntok, int32_t num_heads, int32_t dk, int32_t dv,
    const void* state_pool, kda_dtype_t state_dtype, int64_t num_slots,
    const int32_t* state_indices, void* token_states, float scale, uint32_t flags,
    void* out, int64_t out_stride_t, void* stream)
{
    if (batch < 0 || ntok <= 0 || num_heads <= 0 || num_slots < 0) return KDA_ERR_INVALID_ARG;
    if (!dtype_ok(act_dtype) || !dtype_ok(state_dtype)) return KDA_ERR_INVALID_ARG;
    if (flags & ~KDA_FLAG_QK_L2NORM) return KDA_ERR_INVALID_ARG;
    if (!dim_ok(dk) || dk != dv) return KDA_ERR_UNSUPPORTED;
    if (batch == 0) return KDA_OK;
    if (!q || !k || !v || !g || !beta || !state_indices || !out || !token_states)
        return KDA_ERR_INVALID_ARG;
    if (num_slots > 0 && !state_pool) return KDA_ERR_INVALID_ARG;
    const int64_t hk = (int64_t)num_heads * dk, hv = (int64_t)num_heads * dv;
    if (q_stride_t < hk || k_stride_t < hk || v_stride_t < hv || out_stride_t < hv)
        return KDA_ERR_INVALID_ARG;
    if ((q_stride_t | k_stride_t | v_stride_t | out_stride_t) & 7) return KDA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
        !aligned16(state_pool) || !aligned16(token_states))
        return KDA_ERR_INVALID_ARG;
    if ((int64_t)batch * num_heads > INT32_MAX || (int64_t)batch * ntok > INT32_MAX)
        return KDA_ERR_UNSUPPORTED;

    kda::DecodeArgs a;
    a.q = q; a.k = k; a.v = v;
    a.q_stride = q_stride_t; a.k_stride = k_stride_t; a.v_stride = v_stride_t;
    a.g = g; a.beta = beta;
    a.batch = batch; a.ntok = ntok; a.heads = num_heads; a.dk = dk; a.dv = dv;
    a.pool = const_cast<void*>(state_pool); a.num_slots = num_slots; a.slots = state_indices;
    a.token_states = token_states;
    a.scale = scale; a.flags = flags;
    a.out = out; a.out_stride = out_stride_t;
    a.act = act_dtype; a.state = state_dtype;
    return launch_status(kda::launch_decode(a, static_cast<hipStream_t>(stream)));
}

kda_status_t kda_spec_commit(
    const void* token_states, int32_t batch, int32_t ntok, int32_t num_heads,
    int32_t dk, int32_t dv, const int32_t* num_accepted,
    void* state_pool, kda_dtype_t state_dtype, int64_t num_slots,
    const int32_t* state_indices, void* stream)
{
    if (batch < 0 || ntok <= 0 || num_heads <= 0 || num_slots < 0) return KDA_ERR_INVALID_ARG;
    if (!dtype_ok(state_dtype)) return KDA_ERR_INVALID_ARG;
    if (!dim_ok(dk) || dk != dv) return KDA_ERR_UNSUPPORTED;
    if (batch == 0 || num_slots == 0) return KDA_OK;
    if (!token_states || !num_accepted || !state_pool || !state_indices) return KDA_ERR_INVALID_ARG;
    if (!aligned16(token_states) || !aligned16(state_pool)) return KDA_ERR_INVALID_ARG;
    if ((int64_t)batch * num_heads > INT32_MAX) return KDA_ERR_UNSUPPORTED;

    kda::SpecCommitArgs a;
    a.token_states = token_states;
    a.batch = batch; a.ntok = ntok; a.heads = num_heads; a.dk = dk; a.dv = dv;
    a.accepted = num_accepted;
    a.pool = state_pool; a.num_slots = num_slots; a.slots = state_indices;
    a.state = state_dtype;
    return launch_status(kda::launch_spec_commit(a, static_cast<hipStream_t>(stream)));
}

kda_status_t kda_gated_rmsnorm_ex(
    const void* x, int64_t x_stride_t, const void* gate, int64_t gate_stride_t,
    const void* residual, int64_t residual_stride_t, const void* weight, const void* bias,
    void* y, int64_t y_stride_t, void* residual_out, int64_t residual_out_stride_t,
    kda_dtype_t dtype, int64_t tokens, int32_t heads, int32_t dim, float eps, uint32_t flags,
    void* stream)
{
    if (tokens < 0 || heads <= 0 || !(eps >= 0.0f)) return KDA_ERR_INVALID_ARG;
    if (dtype != KDA_F32 && dtype != KDA_BF16 && dtype != KDA_F16) return KDA_ERR_INVALID_ARG;
    if (flags & ~(KDA_NORM_SIGMOID | KDA_NORM_RESIDUAL_F32)) return KDA_ERR_INVALID_ARG;
    if (dim <= 0 || dim > 1024 || dim % 8 != 0) return KDA_ERR_UNSUPPORTED;
    if (tokens == 0) return KDA_OK;
    if (!x || !gate || !y) return KDA_ERR_INVALID_ARG;
    const int64_t hd = (int64_t)heads * dim;
    if (x_stride_t < hd || gate_stride_t < hd || y_stride_t < hd) return KDA_ERR_INVALID_ARG;
    if (residual && residual_stride_t < hd) return KDA_ERR_INVALID_ARG;
    if (residual_out && residual_out_stride_t < hd) return KDA_ERR_INVALID_ARG;
    if ((x_stride_t | gate_stride_t | y_stride_t | (residual ? residual_stride_t : 0) |
         (residual_out ? residual_out_stride_t : 0)) & 7)
        return KDA_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(gate) || !aligned16(y) || !aligned16(weight) ||
        !aligned16(bias) || !aligned16(residual) || !aligned16(residual_out))
        return KDA_ERR_INVALID_ARG;

    kda::RmsNormArgs a;
    a.x = x; a.x_stride = x_stride_t;
    a.gate = gate; a.gate_stride = gate_stride_t;
    a.residual = residual; a.residual_stride = residual_stride_t;
    a.weight = weight; a.bias = bias;
    a.y = y; a.y_stride = y_stride_t;
    a.residual_out = residual_out; a.residual_out_stride = residual_out_stride_t;
    a.tokens = tokens; a.heads = heads; a.dim = dim;
    a.eps = eps; a.dtype = dtype;
    a.sigmoid = (flags & KDA_NORM_SIGMOID) != 0;
    a.residual_f32 = dtype == KDA_F32 || (flags & KDA_NORM_RESIDUAL_F32) != 0;
    return launch_status(kda::launch_gated_rmsnorm(a, static_cast<hipStream_t>(stream)));
}

kda_status_t kda_gated_rmsnorm(
    const void* x, int64_t x_stride_t, const void* gate, int64_t gate_stride_t,
    const void* weight, void* y, int64_t y_stride_t, kda_dtype_t dtype,
    int64_t tokens, int32_t heads, int32_t dim, float eps, void* stream)
{
    return kda_gated_rmsnorm_ex(x, x_stride_t, gate, gate_stride_t, nullptr, 0, weight, nullptr,
                                y, y_stride_t, nullptr, 0, dtype, tokens, heads, dim, eps, 0u,
                                stream);
}

kda_status_t kda_causal_conv1d(
    const void* x, int64_t x_stride_t, const void* weight, const void* bias,
    void* conv_state_pool, int64_t num_slots,
    const int32_t* cu_seqlens, const int32_t* state_indices,
    const uint8_t* has_initial_state, int32_t num_seqs, int64_t total_tokens,
    int32_t channels, int32_t width, kda_dtype_t dtype, uint32_t flags,
    void* y, int64_t y_stride_t, void* stream)
{
    if (num_seqs < 0 || total_tokens < 0 || num_slots < 0 || channels <= 0)
        return KDA_ERR_INVALID_ARG;
    if (!dtype_ok(dtype)) return KDA_ERR_INVALID_ARG;
    if (flags & ~KDA_CONV_SILU) return KDA_ERR_INVALID_ARG;
    if (width < 2 || width > 8 || channels % 8 != 0) return KDA_ERR_UNSUPPORTED;
    if (num_seqs == 0) return KDA_OK;
    if (!cu_seqlens || !state_indices || !weight) return KDA_ERR_INVALID_ARG;
    if (total_tokens > 0 && (!x || !y)) return KDA_ERR_INVALID_ARG;
    if (num_slots > 0 && !conv_state_pool) return KDA_ERR_INVALID_ARG;
    if (x_stride_t < channels || y_stride_t < channels) return KDA_ERR_INVALID_ARG;
    if ((x_stride_t | y_stride_t) & 7) return KDA_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(y) || !aligned16(conv_state_pool) || !aligned16(weight) ||
        !aligned16(bias))
        return KDA_ERR_INVALID_ARG;

    kda::ConvArgs a;
    a.x = x; a.x_stride = x_stride_t;
    a.weight = weight; a.bias = bias;
    a.state = conv_state_pool; a.num_slots = num_slots;
    a.cu_seqlens = cu_seqlens; a.slots = state_indices; a.has_init = has_initial_state;
    a.num_seqs = num_seqs; a.total_tokens = total_tokens;
    a.channels = channels; a.width = width; a.flags = flags;
    a.y = y; a.y_stride = y_stride_t;
    a.dtype = dtype;
    return launch_status(kda::launch_causal_conv1d(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
