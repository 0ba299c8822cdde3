// kda_internal.h -- launcher interfaces between the C-ABI layer (kda_api.hip)
// and the kernel translation units.  Host code only; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kda.h"

namespace kda {

// Decode (ntok = 1, token_states null: the pool slot is updated in place)
// and speculative decode (ntok >= 1 tokens per row, the state after each
// token written to token_states; the pool is only read).
struct DecodeArgs {
    const void* q; const void* k; const void* v;
    int64_t q_stride, k_stride, v_stride;       // elements between token rows
    const float* g; const float* beta;
    int32_t batch, ntok, heads, dk, dv;
    void* pool; int64_t num_slots;
    const int32_t* slots;
    void* token_states;
    float scale; uint32_t flags;
    void* out; int64_t out_stride;
    kda_dtype_t act, state;
};
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

struct SpecCommitArgs {
    const void* token_states;
    int32_t batch, ntok, heads, dk, dv;
    const int32_t* accepted;
    void* pool; int64_t num_slots;
    const int32_t* slots;
    kda_dtype_t state;
};
hipError_t launch_spec_commit(const SpecCommitArgs& a, hipStream_t stream);

struct PrefillArgs {
    const void* q; const void* k; const void* v;
    int64_t q_stride, k_stride, v_stride;        // elements between tokens
    const float* g; const float* beta;
    const int32_t* cu_seqlens; int32_t num_seqs; int64_t total_tokens;
    int32_t heads, dk, dv;
    void* pool; int64_t num_slots;
    const int32_t* slots; const uint8_t* has_init;
    void* ckpt; int64_t ckpt_capacity; int32_t ckpt_interval;
    float scale; int32_t chunk; uint32_t flags;
    void* out; int64_t out_stride;
    void* workspace;
    kda_dtype_t act, state;
    // Absolute position of each sequence's first token ([num_seqs], device)
    // or null (all 0): chunk boundaries and checkpoints follow absolute
    // positions.
    const int64_t* seq_pos;
    // Fused front end (conv_width > 0): q, k, v point into the packed
    // projection x and are taken through the causal conv1d first; its state
    // pool is indexed like the state pool (same slots, has_init, num_slots).
    const void* conv_w; const void* conv_b; void* conv_state;
    int32_t conv_width; uint32_t conv_flags;
    // Gated RMSNorm fused into the output (norm_y non-null): y = o *
    // rsqrt(mean(o^2) + eps) * w * SiLU(gate) per (token, head) row of o as
    // stored, [total_tokens, heads, dv] of act, token strides in elements.
    const void* norm_gate; int64_t norm_gate_stride;
    const void* norm_weight;                     // [dv] or null (= 1)
    float norm_eps;
    void* norm_y; int64_t norm_y_stride;
};
// Workspace bytes for a call (with the fused norm: norm); 0 if the shape is
// unsupported.
size_t prefill_workspace_bytes(int32_t num_seqs, int64_t total_tokens, int32_t heads,
                               int32_t dk, int32_t dv, int32_t chunk, bool norm = false);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);

struct RmsNormArgs {
    const void* x; int64_t x_stride;
    const void* gate; int64_t gate_stride;
    const void* residual; int64_t residual_stride;      // null: no residual
    const void* weight; const void* bias;               // null: 1 / 0
    void* y; int64_t y_stride;
    void* residual_out; int64_t residual_out_stride;    // null: not written
    int64_t tokens; int32_t heads, dim;
    float eps;
    kda_dtype_t dtype;
    bool sigmoid;                                       // gate activation sigmoid (else SiLU)
    bool residual_f32;                                  // residual and residual_out in fp32
};
hipError_t launch_gated_rmsnorm(const RmsNormArgs& a, hipStream_t stream);

struct ConvArgs {
    const void* x; int64_t x_stride;
    const void* weight; const void* bias;
    void* state; int64_t num_slots;
    const int32_t* cu_seqlens; const int32_t* slots; const uint8_t* has_init;
    int32_t num_seqs; int64_t total_tokens;
    int32_t channels, width;
    uint32_t flags;
    void* y; int64_t y_stride;
    kda_dtype_t dtype;
};
hipError_t launch_causal_conv1d(const ConvArgs& a, hipStream_t stream);

}  // namespace kda
