/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention library, libkda.so.
 *
 * Kimi Delta Attention (KDA) is the gated delta rule with a per-key-channel
 * decay.  For each head the state S is a d_k x d_v matrix and each token does
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(exp(g_t)) S_{t-1} + beta_t k_t v_t^T
 *     o_t = scale * S_t^T q_t
 *
 * The pages name this operator and split it into a chunk prefill and a
 * recurrent decode (page "[Feature][KDA] Add Kimi K3 KDA execution", What this
 * PR does and KDA execution steps 3-4).  Around the two sit the causal
 * convolution that feeds them (step 2) and the gated RMSNorm applied to their
 * output (What this PR does).
 *
 * Conventions for every entry point
 *   - Every pointer argument is DEVICE memory owned by the caller, except
 *     where a comment says otherwise.  The library allocates nothing and
 *     keeps no state between calls.  Apart from kda_chunk_prefill_check (a
 *     diagnostic that waits for its stream) no call synchronises: each only
 *     enqueues kernels on `stream` (a hipStream_t; NULL = the null stream),
 *     so it can be captured into a HIP graph.  Outputs are valid once the
 *     stream has reached that point.
 *   - Layouts are row-major.  Activations are [tokens, heads, dim] with the
 *     head blocks of one token contiguous and a caller-given token stride (in
 *     elements), so packed projections can be read in place.  Recurrent
 *     states are [slots, heads, d_k, d_v] with d_v contiguous.
 *   - Inputs are read-only.  Outputs must not alias inputs.
 *   - Only errors the host can see are reported: a bad argument returns a
 *     status without enqueuing anything; a failed launch returns
 *     KDA_ERR_LAUNCH.  Device-side data (cu_seqlens, slot indices) are a
 *     caller contract: cu_seqlens must be non-decreasing with
 *     cu_seqlens[0] = 0 and cu_seqlens[num_seqs] <= total_tokens, slot
 *     indices must be < num_slots and distinct within a call (< 0 marks a
 *     padding row).  The kernels clamp what they can so that a violation
 *     corrupts results rather than memory, but results are then undefined.
 *   - Results are deterministic: the same call on the same inputs gives
 *     bitwise identical outputs and states (no floating-point atomics), and
 *     which pool slot a sequence uses does not change any value.
 *   - The prefill entry points read the current device's CU count
 *     (hipDeviceGetAttribute, no stream work) to choose how densely the
 *     state-passing kernel is packed on the chip; every choice computes the
 *     same bits, so a sequence's results do not depend on the batch it is in.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 1

/* The library is built with hidden symbol visibility: exactly the entry
 * points declared here are exported. */
#define KDA_API __attribute__((visibility("default")))

/* Status codes. */
typedef int32_t kda_status_t;
#define KDA_OK 0
#define KDA_ERR_INVALID_ARG 1          /* null pointer, negative size, bad stride     */
#define KDA_ERR_UNSUPPORTED 2          /* dims / chunk size / dtype / interval not built */
#define KDA_ERR_WORKSPACE_TOO_SMALL 3  /* workspace_bytes below the query's result     */
#define KDA_ERR_LAUNCH 4               /* hipGetLastError() after the launch            */
#define KDA_ERR_DEVICE 5               /* kda_chunk_prefill_check: the device reported a failure */
#define KDA_ERR_SCRATCH_LIMIT 6        /* kda_chunk_prefill_noalloc: call exceeds the fixed scratch */

/* Element types. */
typedef int32_t kda_dtype_t;
#define KDA_F32 0
#define KDA_BF16 1
#define KDA_F16 2      /* IEEE half: the gated RMSNorm entry points only */

/* Flags. */
#define KDA_FLAG_QK_L2NORM 1u   /* q, k <- x / sqrt(sum x^2 + 1e-6) per (token, head) in-kernel */
/* Prefill diagnostic, for testing the failure report only: the chain
 * kernel's output workgroups give up their bounded waits at once, as if the
 * producing workgroup never published.  The call still completes normally,
 * its output rows are NaN and its status word (kda_chunk_prefill_check)
 * reports a wait that ran out; states and checkpoints are computed as usual. */
#define KDA_FLAG_DIAG_GIVE_UP 0x80000000u
#define KDA_CONV_SILU 1u        /* apply SiLU after the convolution                        */
#define KDA_NORM_SIGMOID 1u      /* gated norm: gate activation sigmoid(z), not z*sigmoid(z) */
#define KDA_NORM_RESIDUAL_F32 2u /* gated norm: residual and residual_out are fp32            */

/* Supported shapes: d_k = d_v in {16, 32, 64, 128}; chunk_size in {16, 32, 64}. */

/* KDA_ABI_VERSION of the loaded library. */
KDA_API int kda_abi_version(void);

/* Static, NUL-terminated description of a status code (never NULL). */
KDA_API const char* kda_status_string(kda_status_t status);

/*
 * Bytes of caller-owned scratch that kda_chunk_prefill needs for a call with
 * these sizes (page "[KK] Prepare B12X Kimi KDA prefill ...", Behavior:
 * reusable caller-owned scratch).  Depends only on host-known sizes, so one
 * buffer sized for the largest batch serves every later call.  Returns 0 for
 * unsupported shapes.
 */
KDA_API size_t kda_chunk_prefill_workspace_size(int32_t num_seqs, int64_t total_tokens,
                                        int32_t num_heads, int32_t dk, int32_t dv,
                                        int32_t chunk_size);

/*
 * Chunk prefill over a varlen token batch (page "Add Kimi K3 KDA execution",
 * KDA execution step 3: build the cumulative gate, then run the chunked
 * prefill).
 *
 *   q, k        [total_tokens, H, dk] of act_dtype, token strides q_stride_t,
 *               k_stride_t (elements, >= H*dk)
 *   v           [total_tokens, H, dv] of act_dtype, token stride v_stride_t
 *   g           [total_tokens, H, dk] fp32, contiguous: per-token log-decay
 *               (alpha = exp(g), g <= 0 expected).  The kernels factor the
 *               decay per 16-token sub-chunk; per channel the decay summed
 *               over any 16 consecutive tokens must stay above -80.
 *   beta        [total_tokens, H] fp32, contiguous
 *   cu_seqlens  [num_seqs + 1] int32: sequence i is tokens
 *               cu_seqlens[i] .. cu_seqlens[i+1]-1.  Empty sequences are
 *               no-ops (same page, Metadata construction: empty segments).
 *   state_pool  [num_slots, H, dk, dv] of state_dtype (fp32 or bf16), read
 *               and written IN PLACE at state_pool[state_indices[i]] -- no
 *               gather or scatter around the kernels (page "[KK] Prepare B12X
 *               Kimi KDA prefill ...", Behavior).
 *   state_indices [num_seqs] int32; < 0 marks a graph-padding sequence: its
 *               output rows are written as zeros and no state is touched
 *               (page "Add Kimi K3 KDA execution", KDA execution step 5).
 *   has_initial_state [num_seqs] uint8 or NULL (= all 1): 0 starts the
 *               sequence from a zero state, a genuine prompt without state
 *               (same page, Metadata construction).
 *   checkpoints [ckpt_capacity, H, dk, dv] of state_dtype or NULL; written
 *               when ckpt_interval > 0 (page "FlashKDA kernel upgrade supports
 *               bf16 checkpoint state": checkpoint states stored in the state
 *               dtype).  Checkpoint j of sequence i is the state after token
 *               (j+1)*ckpt_interval of this call, stored at row
 *               sum_{m<i} floor(L_m / ckpt_interval) + j (padding sequences
 *               keep their rows, unwritten).  Rows >= ckpt_capacity are
 *               skipped; floor(total_tokens / ckpt_interval) rows always
 *               suffice.  ckpt_interval must be a multiple of chunk_size.
 *   scale       output scale (1.0 gives o_t = S_t^T q_t)
 *   flags       KDA_FLAG_QK_L2NORM, KDA_FLAG_DIAG_GIVE_UP (testing only)
 *   out         [total_tokens, H, dv] of act_dtype, token stride out_stride_t;
 *               rows of padding sequences are zeroed, rows outside every
 *               sequence are left alone.
 *   workspace   at least kda_chunk_prefill_workspace_size(...) bytes, 256-byte
 *               aligned.  Its contents are scratch: any call may overwrite it,
 *               so concurrent calls need separate workspaces.  Its first 4
 *               bytes are a status word that kda_chunk_prefill_check reads.
 *               It also carries the per-chunk exchange between the two
 *               workgroups that share each 16-column tile of the state;
 *               should the GPU ever place such a pair on different XCDs, that
 *               tile's output rows come out NaN (never stale values) and the
 *               status word says so.
 * States are computed in fp32 between chunks; a bf16 state is rounded to
 * nearest-even when stored (final state and checkpoints).  The MFMA products
 * take their operands in bf16 whatever act_dtype and state_dtype are: q, k, v
 * (fp32 activations are rounded once on load), the chunk's decay-weighted
 * keys and queries, and the state where it multiplies them; accumulation,
 * the decay factors, beta and the carried state stay fp32.
 * The call enqueues two kernels: the intra-chunk kernel (every chunk in
 * parallel; it also clears the status word and the exchange flags) and the
 * chain kernel (the chunk-to-chunk state recurrence); a call without tokens
 * runs a one-workgroup clearing kernel instead of the first.  A call with
 * more than 2^24 (chunk slot, head) pairs -- chunk slots being
 * ceil(total_tokens / chunk_size) + 2 * num_seqs -- does not fit the
 * one-dimensional grid of the intra-chunk kernel and returns KDA_ERR_LAUNCH
 * without enqueuing anything.
 */
KDA_API kda_status_t kda_chunk_prefill(
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
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * kda_chunk_prefill without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, layouts, results and
 * errors as kda_chunk_prefill, whose kernels it runs, except that the scratch
 * is a fixed 128 MiB area of device memory inside the library: one per GPU,
 * held from the library's load to the end of the process.  That is enough for
 * one 4096-token sequence with 16 heads of dk = dv = 128 at chunk 64; a call
 * whose kda_chunk_prefill_workspace_size exceeds 128 MiB (134,217,728 bytes)
 * returns KDA_ERR_SCRATCH_LIMIT without enqueuing anything.  The call uses the
 * area of the current device (stream must belong to it) and allocates
 * nothing: on its first call on a device it looks up that device's copy of
 * the area, after which it only enqueues kernels, like kda_chunk_prefill.
 * Every call on one GPU shares that GPU's area and leaves its contents
 * there (the kernels clear what must start at zero): two calls that overlap
 * on one GPU -- on different streams, or from different threads without
 * ordering -- race and give wrong results.
 */
KDA_API kda_status_t kda_chunk_prefill_noalloc(
    const void* q, const void* k, const void* v, kda_dtype_t act_dtype,
    int64_t q_stride_t, int64_t k_stride_t, int64_t v_stride_t,
    const float* g, const float* beta,
    const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
    int32_t num_heads, int32_t dk, int32_t dv,
    void* state_pool, kda_dtype_t state_dtype, int64_t num_slots,
    const int32_t* state_indices, const uint8_t* has_initial_state,
    void* checkpoints, int64_t ckpt_capacity, int32_t ckpt_interval,
    float scale, int32_t chunk_size, uint32_t flags,
    void* out, int64_t out_stride_t, void* stream);

/*
 * Diagnostic for the prefill calls (kda_chunk_prefill, kda_chunk_prefill_at,
 * kda_conv_chunk_prefill): waits for `stream`, then reads the status word that
 * the last such call on `workspace` left (a call with num_seqs == 0 launches
 * nothing and leaves it as it was).  The prefill's waves and workgroups wait
 * for one another with bounded waits; if one ever ran out (so that call's
 * outputs and states are not valid: the affected rows are NaN), the word is
 * nonzero.  *device_flags (may be NULL) receives the word: bit 0 a wait ran
 * out, bit 1 the two workgroups of a state tile ran on different XCDs.
 * Returns KDA_OK when the word is 0, KDA_ERR_DEVICE otherwise,
 * KDA_ERR_INVALID_ARG for a null or too small workspace (< 4 bytes) and
 * KDA_ERR_LAUNCH if the stream or the copy fails.  Unlike every other entry
 * point this one synchronises; it is not meant for the hot path.
 */
KDA_API kda_status_t kda_chunk_prefill_check(const void* workspace, size_t workspace_bytes,
                                     uint32_t* device_flags, void* stream);

/*
 * Recurrent decode: one token per row, every non-padding row has a state
 * (page "Add Kimi K3 KDA execution", KDA execution step 4 and Metadata
 * construction: a one-token request with an existing state is decode).
 * Each head's state is streamed once through registers and written back in
 * place.
 *
 *   q, k   [batch, H, dk] of act_dtype, row strides q_stride_b, k_stride_b
 *   v      [batch, H, dv] of act_dtype, row stride v_stride_b
 *   g      [batch, H, dk] fp32 contiguous;  beta [batch, H] fp32 contiguous
 *   state_pool [num_slots, H, dk, dv] of state_dtype, in place
 *   state_indices [batch] int32; < 0 = padding row (zero output, no state I/O)
 *   flags  KDA_FLAG_QK_L2NORM
 *   out    [batch, H, dv] of act_dtype, row stride out_stride_b
 */
KDA_API kda_status_t kda_recurrent_decode(
    const void* q, const void* k, const void* v, kda_dtype_t act_dtype,
    int64_t q_stride_b, int64_t k_stride_b, int64_t v_stride_b,
    const float* g, const float* beta,
    int32_t batch, int32_t num_heads, int32_t dk, int32_t dv,
    void* state_pool, kda_dtype_t state_dtype, int64_t num_slots,
    const int32_t* state_indices, float scale, uint32_t flags,
    void* out, int64_t out_stride_b, void* stream);

/*
 * Gated RMSNorm, norm before gate, on [tokens, heads, dim] rows (page "Add
 * Kimi K3 KDA execution", What this PR does: output normalisation and gating
 * with the result in a separate allocation so the input is preserved):
 *
 *     y = x / sqrt(mean(x^2) + eps) * weight * silu(gate),  silu(z) = z*sigmoid(z)
 *
 * statistics over the `dim` elements of one (token, head).  x, gate, y have
 * per-token strides (elements) so packed gates can be read in place; heads
 * of one token are contiguous blocks of `dim`.  weight is [dim] of `dtype` or
 * NULL (no affine).  dtype KDA_F32, KDA_BF16 or KDA_F16.  Math in fp32; y may
 * not alias x or gate.
 */
KDA_API kda_status_t kda_gated_rmsnorm(
    const void* x, int64_t x_stride_t, const void* gate, int64_t gate_stride_t,
    const void* weight, void* y, int64_t y_stride_t, kda_dtype_t dtype,
    int64_t tokens, int32_t heads, int32_t dim, float eps, void* stream);

/*
 * Gated RMSNorm variants (page "Add Kimi K3 KDA execution", How was this
 * patch tested: the norm-gate cases cover fp16 and bf16 data, sigmoid and SiLU
 * gates, packed gate strides, the affine path, the residual / prenorm path,
 * and preserving the input):
 *
 *     h = x + residual                       (residual NULL: h = x)
 *     residual_out = h                       (residual_out NULL: not written)
 *     y = (h / sqrt(mean(h^2) + eps) * weight + bias) * act(gate)
 *     act(z) = z*sigmoid(z), or sigmoid(z) with KDA_NORM_SIGMOID
 *
 * The sum h is formed in fp32; the norm uses that unrounded sum, and
 * residual_out stores it rounded to its type.  x, gate, y, weight [dim] and
 * bias [dim] (either may be NULL) are of `dtype` (KDA_F32, KDA_BF16 or
 * KDA_F16); residual and residual_out are of `dtype` too, or fp32 with
 * KDA_NORM_RESIDUAL_F32 (always fp32 when dtype is KDA_F32).  Strides are per
 * token, in elements, multiples of 8; every pointer 16-byte aligned.  No
 * output may alias an input.  kda_gated_rmsnorm is this call with no
 * residual, no bias and the SiLU gate.
 */
KDA_API kda_status_t kda_gated_rmsnorm_ex(
    const void* x, int64_t x_stride_t, const void* gate, int64_t gate_stride_t,
    const void* residual, int64_t residual_stride_t, const void* weight, const void* bias,
    void* y, int64_t y_stride_t, void* residual_out, int64_t residual_out_stride_t,
    kda_dtype_t dtype, int64_t tokens, int32_t heads, int32_t dim, float eps, uint32_t flags,
    void* stream);

/*
 * Causal depthwise conv1d over a varlen token batch with a rolling per-slot
 * conv state (page "Add Kimi K3 KDA execution", KDA execution step 2: run the
 * causal convolution and update its cache; What this PR does: causal-
 * convolution state packing).
 *
 *     y_t[c] = act( bias[c] + sum_{j<width} weight[c, j] * x_{t-width+1+j}[c] )
 *
 * weight[c, width-1] multiplies the current token; inputs before the start of
 * a sequence come from its conv state (zeros without an initial state).
 *   x        [total_tokens, channels] of dtype, token stride x_stride_t
 *   weight   [channels, width] of dtype;  bias [channels] of dtype or NULL
 *   conv_state_pool [num_slots, width-1, channels] of dtype: row width-2 is
 *            the most recent input.  After the call it holds the last
 *            width-1 inputs seen by the sequence (pre-activation).
 *   state_indices [num_seqs]; < 0 = padding (zero output, no state I/O)
 *   has_initial_state [num_seqs] uint8 or NULL (= all 1)
 *   flags    KDA_CONV_SILU
 *   y        [total_tokens, channels] of dtype, token stride y_stride_t; may
 *            not alias x.
 * Supported: width in [2, 8], channels a multiple of 8, dtype bf16 or fp32.
 */
KDA_API kda_status_t kda_causal_conv1d(
    const void* x, int64_t x_stride_t, const void* weight, const void* bias,
    void* conv_state_pool, int64_t num_slots,
    const int32_t* cu_seqlens, const int32_t* state_indices,
    const uint8_t* has_initial_state, int32_t num_seqs, int64_t total_tokens,
    int32_t channels, int32_t width, kda_dtype_t dtype, uint32_t flags,
    void* y, int64_t y_stride_t, void* stream);

/*
 * Chunk prefill of sequences that start at absolute positions (page
 * "FlashKDA kernel upgrade supports bf16 checkpoint state", function and
 * motivation: checkpoint states are the breakpoints that join the recurrent
 * state across segments, so they belong to absolute positions of a
 * sequence, e.g. aligned with a cached prefix).
 *   seq_start_pos [num_seqs] int64, device, or NULL (all 0): tokens of each
 *            sequence processed before this call; negative values count as 0.
 * Chunk boundaries fall on absolute multiples of chunk_size (a sequence's
 * first chunk holds chunk_size - start % chunk_size tokens), and checkpoint
 * rows hold the state after every token whose absolute count
 * start + (tokens of this call so far) is a multiple of ckpt_interval: the
 * multiples of the interval in (start, start + L] for a sequence of L tokens,
 * rows laid out sequence by sequence.  Everything else is kda_chunk_prefill
 * (same workspace query); with all positions 0 the results are identical.
 */
KDA_API kda_status_t kda_chunk_prefill_at(
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
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Fused front end + chunk prefill: kda_causal_conv1d over the packed
 * projection x = [q | k | v] followed by kda_chunk_prefill on its three parts,
 * with the convolution evaluated where the prefill loads its activations, so
 * the conv output never goes to memory (page "Add Kimi K3 KDA execution", KDA
 * execution steps 2-3: run the causal convolution and update its cache, then
 * the chunked prefill; What this PR does: causal-convolution state packing).
 *   x        [total_tokens, 3 H d] of act_dtype, token stride x_stride_t:
 *            channels [0, Hd) are q, [Hd, 2Hd) k, [2Hd, 3Hd) v (head-major d)
 *   conv_weight [3 H d, conv_width] of act_dtype; conv_bias [3 H d] or NULL
 *   conv_width  2 .. 8;  conv_flags  KDA_CONV_SILU
 *   conv_state_pool [num_slots, conv_width - 1, 3 H d] of act_dtype, indexed
 *            like state_pool (state_indices, has_initial_state, num_slots);
 *            after the call it holds each sequence's last conv_width - 1 rows
 *            of x, exactly as kda_causal_conv1d leaves it.
 * All other arguments, the workspace and the results are those of
 * kda_chunk_prefill (flags KDA_FLAG_QK_L2NORM normalises the conv outputs
 * q, k).  The result equals, bit for bit, kda_causal_conv1d into a buffer y
 * followed by kda_chunk_prefill reading q, k, v from y.
 */
KDA_API kda_status_t kda_conv_chunk_prefill(
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
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Prefill with the gated RMSNorm fused into its output (page "[Feature][KDA]
 * Add Kimi K3 KDA execution", What this PR does: the KDA output goes through
 * a fused normalisation-and-gating step whose result is allocated
 * separately, so the KDA output itself is kept).  Besides everything
 * kda_chunk_prefill (or kda_conv_chunk_prefill) computes and writes, including
 * `out`, these write
 *   norm_out[t, h, :] = out[t, h, :] * rsqrt(mean(out[t, h, :]^2) + norm_eps)
 *                       * norm_weight * SiLU(norm_gate[t, h, :])
 * for every token row, out taken as stored (act_dtype); norm_out equals, bit
 * for bit, kda_gated_rmsnorm(out, norm_gate, norm_weight, norm_eps) after the
 * plain call.  Padding sequences (state index < 0) get the norm of their zero
 * rows, as that call would give them.
 *   norm_gate  [total_tokens, H, dv] of act_dtype, token stride
 *              norm_gate_stride_t (elements, >= H*dv, a multiple of 8)
 *   norm_weight [dv] of act_dtype or NULL (= 1);  norm_eps >= 0
 *   norm_out   [total_tokens, H, dv] of act_dtype, token stride
 *              norm_out_stride_t (same rules); must not overlap out
 *   workspace  at least kda_chunk_prefill_norm_workspace_size(...) bytes (the
 *              plain size plus a second flag per (sequence, head, 16-column
 *              tile)), 256-byte aligned
 * The output workgroups of a (sequence, head) tell one another through those
 * flags which chunks of `out` are stored, and each then normalises a share of
 * the chunk's rows; the same device-side status word reports a bounded wait
 * that ran out (kda_chunk_prefill_check).  Returns as kda_chunk_prefill, and
 * KDA_ERR_INVALID_ARG for a missing norm_gate / norm_out with tokens, a bad
 * stride (including an out_stride_t with chunk_size * out_stride_t *
 * element size at or above 2^31 bytes), a misaligned pointer or a negative
 * (or NaN) norm_eps.
 * Cost: the call saves a launch and the second read of `out`, but the norm's
 * loads and stores join the prefill's serial chunk steps; at 4096 tokens x 16
 * heads of dv = 128 it is slower than the plain call followed by
 * kda_gated_rmsnorm.
 */
KDA_API size_t kda_chunk_prefill_norm_workspace_size(int32_t num_seqs, int64_t total_tokens,
                                                     int32_t num_heads, int32_t dk, int32_t dv,
                                                     int32_t chunk_size);
KDA_API kda_status_t kda_chunk_prefill_norm(
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
    void* workspace, size_t workspace_bytes, void* stream);
KDA_API kda_status_t kda_conv_chunk_prefill_norm(
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
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Speculative multi-token decode (page "[Feature][KDA] Add Kimi K3 KDA
 * execution", Metadata construction: speculative decode is a path of its own
 * next to chunk prefill and recurrent decode; page "FlashKDA kernel upgrade
 * supports bf16 checkpoint state", risks: restoring checkpoint states in the
 * speculative decode chain).
 *
 * Row b carries ntok draft tokens, token rows b*ntok + t (t = 0 .. ntok-1) in
 * order.  Starting from state_pool[state_indices[b]], the tokens are applied
 * with the recurrence at the top of this header; out[b*ntok + t] is the output
 * of token t, and the state after token t is written to token_states[b, t].
 * The pool is read and never written, so a verifier can accept any prefix
 * afterwards with kda_spec_commit.
 *   q, k     [batch*ntok, heads, dk] of act_dtype, token strides in elements
 *   v, out   [batch*ntok, heads, dv] of act_dtype
 *   g        [batch*ntok, heads, dk] fp32;  beta [batch*ntok, heads] fp32
 *   state_pool [num_slots, heads, dk, dv] of state_dtype (read only)
 *   state_indices [batch]; < 0 = padding row: zero outputs, its token states
 *            are not written
 *   token_states [batch, ntok, heads, dk, dv] of state_dtype (written)
 *   flags    KDA_FLAG_QK_L2NORM
 * Supported: dk = dv in {16, 32, 64, 128}, ntok >= 1.
 */
KDA_API kda_status_t kda_spec_decode(
    const void* q, const void* k, const void* v, kda_dtype_t act_dtype,
    int64_t q_stride_t, int64_t k_stride_t, int64_t v_stride_t,
    const float* g, const float* beta,
    int32_t batch, int32_t ntok, int32_t num_heads, int32_t dk, int32_t dv,
    const void* state_pool, kda_dtype_t state_dtype, int64_t num_slots,
    const int32_t* state_indices, void* token_states, float scale, uint32_t flags,
    void* out, int64_t out_stride_t, void* stream);

/*
 * Commit a verified speculative step (same passages): for every row b with
 * state_indices[b] >= 0 and 0 < num_accepted[b] <= ntok,
 * state_pool[state_indices[b]] = token_states[b, num_accepted[b] - 1], in
 * place; rows with num_accepted[b] == 0 keep their state.  num_accepted is a
 * device array of int32 [batch]; a value outside [0, ntok] is a caller
 * contract violation and leaves that slot unchanged.  token_states and the
 * pool must not overlap.
 */
KDA_API kda_status_t kda_spec_commit(
    const void* token_states, int32_t batch, int32_t ntok, int32_t num_heads,
    int32_t dk, int32_t dv, const int32_t* num_accepted,
    void* state_pool, kda_dtype_t state_dtype, int64_t num_slots,
    const int32_t* state_indices, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
