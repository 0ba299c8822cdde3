/*
 * kda_oracle.c -- plain, slow, fp64 CPU reference for Kimi Delta Attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or
 * calls this file: only the tests, the smoke check and the benchmark's CPU
 * baseline leg do.  It shares no code, header, table or helper with the HIP
 * library, and it never sees a value the HIP library produced.
 *
 * What it computes (state S is d_k x d_v per head, row-major, d_v contiguous):
 *
 *   Kimi Delta Attention (KDA) is the gated delta rule with a per-channel
 *   decay.  The pages name the operator and its two execution forms -- chunk
 *   prefill and recurrent decode (page "[Feature][KDA] Add Kimi K3 KDA
 *   execution", "What this PR does" and "KDA execution") -- but do not write
 *   the recurrence out.  Its definition, taken as given:
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = scale * S_t^T q_t              (read after the update)
 *     alpha_t = exp(g_t), g_t the per-key-channel log-decay of token t.
 *
 *   The oracle takes those steps token by token, in that order, in fp64:
 *   decay the rows of S, project with (I - beta k k^T), add the rank-one
 *   write, then read the output.  No blocking, no chunking, no reordering.
 *
 * Serving semantics around the recurrence, from the pages:
 *   - states are read and written in place at pool[slot] with no gather or
 *     scatter (page "[KK] Prepare B12X Kimi KDA prefill ...", Behavior);
 *   - a sequence without an existing state starts from zero; a one-token
 *     request with state is a decode step (page "Add Kimi K3 KDA execution",
 *     Metadata construction);
 *   - empty segments do nothing; graph-padding rows (slot < 0) produce zero
 *     output and touch no state (same page, Metadata construction and KDA
 *     execution step 5);
 *   - checkpoint states at segment boundaries, stored like the state
 *     (page "FlashKDA kernel upgrade supports bf16 checkpoint state",
 *     function and motivation).  Reading taken: checkpoint j of a sequence is
 *     the state after token (j+1)*interval of that call; sequence i's
 *     checkpoints start at row sum_{m<i} floor(L_m / interval).
 *
 * Causal depthwise conv1d and the gated RMSNorm are the pre- and post-KDA
 * operators of the same execution path (page "Add Kimi K3 KDA execution",
 * What this PR does and KDA execution steps 2 and 5).
 *
 * Parallelism: OpenMP over independent (sequence, head) or (row, head)
 * units only; each unit runs the plain serial loop.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_EINVAL 1
#define ORACLE_ENOMEM 2

int kda_oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* x / sqrt(sum x^2 + eps): per-head L2 normalisation of a query or key. */
static void l2_normalise(const double* x, int64_t n, double eps, double* y)
{
    double ss = 0.0;
    for (int64_t i = 0; i < n; ++i) ss += x[i] * x[i];
    double r = 1.0 / sqrt(ss + eps);
    for (int64_t i = 0; i < n; ++i) y[i] = x[i] * r;
}

/*
 * One token of the recurrence, in place on S.  `work` holds d_v doubles.
 */
static void kda_token(double* S, int64_t dk, int64_t dv,
                      const double* q, const double* k, const double* v,
                      const double* g, double beta, double scale,
                      double* o, double* work)
{
    /* S <- Diag(alpha) S: alpha_i = exp(g_i) multiplies row i. */
    for (int64_t i = 0; i < dk; ++i) {
        double a = exp(g[i]);
        for (int64_t j = 0; j < dv; ++j) S[i * dv + j] *= a;
    }
    /* S <- (I - beta k k^T) S = S - beta k (k^T S). */
    for (int64_t j = 0; j < dv; ++j) {
        double s = 0.0;
        for (int64_t i = 0; i < dk; ++i) s += k[i] * S[i * dv + j];
        work[j] = s;
    }
    for (int64_t i = 0; i < dk; ++i)
        for (int64_t j = 0; j < dv; ++j)
            S[i * dv + j] -= beta * k[i] * work[j];
    /* S <- S + beta k v^T. */
    for (int64_t i = 0; i < dk; ++i)
        for (int64_t j = 0; j < dv; ++j)
            S[i * dv + j] += beta * k[i] * v[j];
    /* o = scale * S^T q. */
    for (int64_t j = 0; j < dv; ++j) {
        double s = 0.0;
        for (int64_t i = 0; i < dk; ++i) s += S[i * dv + j] * q[i];
        o[j] = scale * s;
    }
}

/*
 * Chunk prefill over a varlen token batch (the result the chunked method must
 * reach; here it is the plain token loop).
 *
 *   q, k, g : [T, H, dk]      v, o : [T, H, dv]      beta : [T, H]
 *   cu_seqlens : [n_seqs + 1], non-decreasing, cu_seqlens[0] = 0
 *   pool : [n_slots, H, dk, dv], read and written in place
 *   slots : [n_seqs]; < 0 marks a graph-padding sequence
 *   has_init : [n_seqs] or NULL (all sequences have a state)
 *   ckpt : [ckpt_capacity, H, dk, dv] or NULL; ckpt_interval 0 = none
 *   start_pos : [n_seqs] or NULL (all 0): absolute position of each
 *          sequence's first token of this call (tokens processed before it,
 *          e.g. a cached prefix).  A checkpoint is the state after every
 *          token whose absolute count of processed tokens, start_pos + r + 1,
 *          is a multiple of ckpt_interval; rows are laid out sequence by
 *          sequence.
 *   l2norm_qk : normalise q and k per (token, head) before use
 */
int kda_oracle_prefill_at(const double* q, const double* k, const double* v,
                          const double* g, const double* beta,
                          const int64_t* cu_seqlens, int64_t n_seqs,
                          int64_t H, int64_t dk, int64_t dv,
                          double* pool, int64_t n_slots, const int64_t* slots,
                          const uint8_t* has_init, const int64_t* start_pos,
                          double* ckpt, int64_t ckpt_capacity, int64_t ckpt_interval,
                          double scale, int l2norm_qk, double l2_eps, double* o)
{
    if (n_seqs < 0 || H <= 0 || dk <= 0 || dv <= 0 || ckpt_interval < 0)
        return ORACLE_EINVAL;
    for (int64_t i = 0; i < n_seqs; ++i) {
        if (cu_seqlens[i + 1] < cu_seqlens[i]) return ORACLE_EINVAL;
        if (slots[i] >= n_slots) return ORACLE_EINVAL;
        if (start_pos && start_pos[i] < 0) return ORACLE_EINVAL;
    }
    /* Checkpoint row where each sequence starts: the multiples of the
     * interval in (start, start + L]. */
    int64_t* ckpt_base = (int64_t*)calloc((size_t)n_seqs + 1, sizeof(int64_t));
    if (!ckpt_base) return ORACLE_ENOMEM;
    for (int64_t i = 0; i < n_seqs; ++i) {
        int64_t L = cu_seqlens[i + 1] - cu_seqlens[i];
        int64_t p0 = start_pos ? start_pos[i] : 0;
        ckpt_base[i + 1] = ckpt_base[i] +
                           (ckpt_interval > 0 ? (p0 + L) / ckpt_interval - p0 / ckpt_interval : 0);
    }
    const int64_t state_sz = dk * dv;
    int status = ORACLE_OK;

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t unit = 0; unit < n_seqs * H; ++unit) {
        const int64_t i = unit / H, h = unit % H;
        const int64_t t0 = cu_seqlens[i], L = cu_seqlens[i + 1] - cu_seqlens[i];
        const int64_t p0 = start_pos ? start_pos[i] : 0;
        const int64_t slot = slots[i];
        if (slot < 0) {                                   /* padding: zero rows */
            for (int64_t t = t0; t < t0 + L; ++t)
                memset(o + (t * H + h) * dv, 0, (size_t)dv * sizeof(double));
            continue;
        }
        if (L == 0) continue;                             /* empty segment */
        double* S = (double*)calloc((size_t)state_sz, sizeof(double));
        double* work = (double*)malloc((size_t)dv * sizeof(double));
        double* qn = (double*)malloc((size_t)dk * sizeof(double));
        double* kn = (double*)malloc((size_t)dk * sizeof(double));
        if (!S || !work || !qn || !kn) {
            free(S); free(work); free(qn); free(kn);
#pragma omp atomic write
            status = ORACLE_ENOMEM;
            continue;
        }
        double* home = pool + (slot * H + h) * state_sz;
        if (!has_init || has_init[i]) memcpy(S, home, (size_t)state_sz * sizeof(double));
        for (int64_t r = 0; r < L; ++r) {
            const int64_t t = t0 + r;
            const double* qt = q + (t * H + h) * dk;
            const double* kt = k + (t * H + h) * dk;
            if (l2norm_qk) {
                l2_normalise(qt, dk, l2_eps, qn);
                l2_normalise(kt, dk, l2_eps, kn);
                qt = qn;
                kt = kn;
            }
            kda_token(S, dk, dv, qt, kt, v + (t * H + h) * dv, g + (t * H + h) * dk,
                      beta[t * H + h], scale, o + (t * H + h) * dv, work);
            const int64_t pos = p0 + r + 1;            /* tokens processed so far */
            if (ckpt && ckpt_interval > 0 && pos % ckpt_interval == 0) {
                int64_t row = ckpt_base[i] + pos / ckpt_interval - p0 / ckpt_interval - 1;
                if (row >= 0 && row < ckpt_capacity)
                    memcpy(ckpt + (row * H + h) * state_sz, S, (size_t)state_sz * sizeof(double));
            }
        }
        memcpy(home, S, (size_t)state_sz * sizeof(double));
        free(S); free(work); free(qn); free(kn);
    }
    free(ckpt_base);
    return status;
}

/* kda_oracle_prefill_at with every sequence starting at position 0. */
int kda_oracle_prefill(const double* q, const double* k, const double* v,
                       const double* g, const double* beta,
                       const int64_t* cu_seqlens, int64_t n_seqs,
                       int64_t H, int64_t dk, int64_t dv,
                       double* pool, int64_t n_slots, const int64_t* slots,
                       const uint8_t* has_init,
                       double* ckpt, int64_t ckpt_capacity, int64_t ckpt_interval,
                       double scale, int l2norm_qk, double l2_eps, double* o)
{
    return kda_oracle_prefill_at(q, k, v, g, beta, cu_seqlens, n_seqs, H, dk, dv, pool, n_slots,
                                 slots, has_init, NULL, ckpt, ckpt_capacity, ckpt_interval, scale,
                                 l2norm_qk, l2_eps, o);
}

/*
 * Recurrent decode: one token per row, every row has a state (page "Add Kimi
 * K3 KDA execution", Metadata construction: a one-token request with an
 * existing state is decode).
 *
 *   q, k, g : [B, H, dk]    v, o : [B, H, dv]    beta : [B, H]
 *   slots : [B]; < 0 marks a padding row (zero output, no state I/O)
 */
int kda_oracle_decode(const double* q, const double* k, const double* v,
                      const double* g, const double* beta, int64_t B,
                      int64_t H, int64_t dk, int64_t dv,
                      double* pool, int64_t n_slots, const int64_t* slots,
                      double scale, int l2norm_qk, double l2_eps, double* o)
{
    if (B < 0 || H <= 0 || dk <= 0 || dv <= 0) return ORACLE_EINVAL;
    for (int64_t b = 0; b < B; ++b)
        if (slots[b] >= n_slots) return ORACLE_EINVAL;
    int status = ORACLE_OK;
#pragma omp parallel for schedule(static)
    for (int64_t unit = 0; unit < B * H; ++unit) {
        const int64_t b = unit / H, h = unit % H;
        double* ob = o + (b * H + h) * dv;
        if (slots[b] < 0) {
            memset(ob, 0, (size_t)dv * sizeof(double));
            continue;
        }
        double* work = (double*)malloc((size_t)dv * sizeof(double));
        double* qn = (double*)malloc((size_t)dk * sizeof(double));
        double* kn = (double*)malloc((size_t)dk * sizeof(double));
        if (!work || !qn || !kn) {
            free(work); free(qn); free(kn);
#pragma omp atomic write
            status = ORACLE_ENOMEM;
            continue;
        }
        const double* qb = q + (b * H + h) * dk;
        const double* kb = k + (b * H + h) * dk;
        if (l2norm_qk) {
            l2_normalise(qb, dk, l2_eps, qn);
            l2_normalise(kb, dk, l2_eps, kn);
            qb = qn;
            kb = kn;
        }
        double* S = pool + (slots[b] * H + h) * dk * dv;
        kda_token(S, dk, dv, qb, kb, v + (b * H + h) * dv, g + (b * H + h) * dk,
                  beta[b * H + h], scale, ob, work);
        free(work); free(qn); free(kn);
    }
    return status;
}

/*
 * Speculative multi-token decode (page "[Feature][KDA] Add Kimi K3 KDA
 * execution", Metadata construction: speculative decode is a path of its own
 * next to prefill and decode; page "FlashKDA kernel upgrade supports bf16
 * checkpoint state", risks: restoring checkpoint states in the speculative
 * decode chain).
 *
 * Reading taken: row b carries ntok draft tokens, rows b*ntok + t (t in
 * order) of the token arrays.  Starting from pool[slots[b]] the tokens are
 * applied one by one with the recurrence above; the output of token t is
 * o[b*ntok + t] and the state after token t is stored in
 * token_states[b, t] ([B, ntok, H, dk, dv]).  The pool is not modified, so
 * the verifier can later accept any prefix (kda_oracle_spec_commit).
 * slots[b] < 0: zero outputs, token states untouched.
 */
int kda_oracle_spec_decode(const double* q, const double* k, const double* v,
                           const double* g, const double* beta, int64_t B, int64_t ntok,
                           int64_t H, int64_t dk, int64_t dv,
                           const double* pool, int64_t n_slots, const int64_t* slots,
                           double* token_states, double scale, int l2norm_qk, double l2_eps,
                           double* o)
{
    if (B < 0 || ntok < 0 || H <= 0 || dk <= 0 || dv <= 0) return ORACLE_EINVAL;
    for (int64_t b = 0; b < B; ++b)
        if (slots[b] >= n_slots) return ORACLE_EINVAL;
    int status = ORACLE_OK;
#pragma omp parallel for schedule(static)
    for (int64_t unit = 0; unit < B * H; ++unit) {
        const int64_t b = unit / H, h = unit % H;
        if (slots[b] < 0) {
            for (int64_t t = 0; t < ntok; ++t)
                memset(o + ((b * ntok + t) * H + h) * dv, 0, (size_t)dv * sizeof(double));
            continue;
        }
        double* S = (double*)malloc((size_t)(dk * dv) * sizeof(double));
        double* work = (double*)malloc((size_t)dv * sizeof(double));
        double* qn = (double*)malloc((size_t)dk * sizeof(double));
        double* kn = (double*)malloc((size_t)dk * sizeof(double));
        if (!S || !work || !qn || !kn) {
            free(S); free(work); free(qn); free(kn);
#pragma omp atomic write
            status = ORACLE_ENOMEM;
            continue;
        }
        memcpy(S, pool + (slots[b] * H + h) * dk * dv, (size_t)(dk * dv) * sizeof(double));
        for (int64_t t = 0; t < ntok; ++t) {
            const int64_t row = b * ntok + t;
            const double* qt = q + (row * H + h) * dk;
            const double* kt = k + (row * H + h) * dk;
            if (l2norm_qk) {
                l2_normalise(qt, dk, l2_eps, qn);
                l2_normalise(kt, dk, l2_eps, kn);
                qt = qn;
                kt = kn;
            }
            kda_token(S, dk, dv, qt, kt, v + (row * H + h) * dv, g + (row * H + h) * dk,
                      beta[row * H + h], scale, o + (row * H + h) * dv, work);
            memcpy(token_states + ((b * ntok + t) * H + h) * dk * dv, S,
                   (size_t)(dk * dv) * sizeof(double));
        }
        free(S); free(work); free(qn); free(kn);
    }
    return status;
}

/*
 * Commit the verifier's decision (same passages): for each row b with
 * accepted[b] > 0, pool[slots[b]] = token_states[b, accepted[b] - 1]; rows
 * with accepted[b] == 0 or slots[b] < 0 leave the pool alone.
 */
int kda_oracle_spec_commit(const double* token_states, int64_t B, int64_t ntok, int64_t H,
                           int64_t dk, int64_t dv, const int64_t* accepted,
                           double* pool, int64_t n_slots, const int64_t* slots)
{
    if (B < 0 || ntok < 0 || H <= 0 || dk <= 0 || dv <= 0) return ORACLE_EINVAL;
    for (int64_t b = 0; b < B; ++b)
        if (slots[b] >= n_slots || accepted[b] < 0 || accepted[b] > ntok) return ORACLE_EINVAL;
    for (int64_t b = 0; b < B; ++b) {
        if (slots[b] < 0 || accepted[b] == 0) continue;
        for (int64_t h = 0; h < H; ++h)
            memcpy(pool + (slots[b] * H + h) * dk * dv,
                   token_states + ((b * ntok + accepted[b] - 1) * H + h) * dk * dv,
                   (size_t)(dk * dv) * sizeof(double));
    }
    return ORACLE_OK;
}

/*
 * Causal depthwise conv1d with a rolling per-sequence conv state (page "Add
 * Kimi K3 KDA execution", KDA execution step 2: run the causal convolution and
 * update its cache).  Reading taken: PyTorch cross-correlation tap order, so
 * w[c, W-1] multiplies the current token; the state holds the last W-1
 * pre-activation inputs; optional SiLU after the optional bias.
 *
 *   x, y : [T, Cch]   w : [Cch, W]   bias : [Cch] or NULL
 *   conv_pool : [n_slots, W-1, Cch], row W-2 is the most recent input
 *   slots : [n_seqs]; < 0 marks padding (zero output, no state I/O)
 */
int kda_oracle_conv1d(const double* x, const double* w, const double* bias,
                      double* conv_pool, int64_t n_slots,
                      const int64_t* cu_seqlens, const int64_t* slots,
                      const uint8_t* has_init, int64_t n_seqs,
                      int64_t Cch, int64_t W, int silu, double* y)
{
    if (W < 1 || Cch <= 0 || n_seqs < 0) return ORACLE_EINVAL;
    for (int64_t i = 0; i < n_seqs; ++i)
        if (slots[i] >= n_slots || cu_seqlens[i + 1] < cu_seqlens[i]) return ORACLE_EINVAL;
    const int64_t hist = W - 1;
    int status = ORACLE_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < n_seqs; ++i) {
        const int64_t t0 = cu_seqlens[i], L = cu_seqlens[i + 1] - cu_seqlens[i];
        if (slots[i] < 0) {
            memset(y + t0 * Cch, 0, (size_t)(L * Cch) * sizeof(double));
            continue;
        }
        if (L == 0) continue;
        double* st = conv_pool + slots[i] * hist * Cch;
        /* Sequence seen by the filter: W-1 history rows, then the L inputs. */
        double* ext = (double*)calloc((size_t)((hist + L) * Cch), sizeof(double));
        if (!ext) {
#pragma omp atomic write
            status = ORACLE_ENOMEM;
            continue;
        }
        if (!has_init || has_init[i]) memcpy(ext, st, (size_t)(hist * Cch) * sizeof(double));
        memcpy(ext + hist * Cch, x + t0 * Cch, (size_t)(L * Cch) * sizeof(double));
        for (int64_t r = 0; r < L; ++r) {
            for (int64_t c = 0; c < Cch; ++c) {
                double acc = bias ? bias[c] : 0.0;
                for (int64_t j = 0; j < W; ++j) acc += w[c * W + j] * ext[(r + j) * Cch + c];
                if (silu) acc = acc / (1.0 + exp(-acc));
                y[(t0 + r) * Cch + c] = acc;
            }
        }
        /* New state: the last W-1 rows of the extended sequence. */
        memcpy(st, ext + L * Cch, (size_t)(hist * Cch) * sizeof(double));
        free(ext);
    }
    return status;
}

/*
 * Gated RMSNorm, norm before gate (page "Add Kimi K3 KDA execution", What this
 * PR does: output normalisation and gating, result in a separate buffer so
 * the input is preserved; How was this patch tested: sigmoid and SiLU gates,
 * the affine path and the residual / prenorm path).  Per row of `dim`:
 *   h = x + residual                     (residual NULL: h = x)
 *   h_out = h                            (h_out NULL: not written)
 *   y = (h / sqrt(mean(h^2) + eps) * w + b) * act(gate)
 *   act(z) = z / (1 + e^-z)  (SiLU),  or  1 / (1 + e^-z) when `sigmoid`
 * w and b are [dim] or NULL (weight 1, bias 0).
 */
int kda_oracle_gated_rmsnorm_ex(const double* x, const double* gate, const double* residual,
                                const double* w, const double* b, int64_t rows, int64_t dim,
                                double eps, int sigmoid, double* y, double* h_out)
{
    if (rows < 0 || dim <= 0) return ORACLE_EINVAL;
    int status = ORACLE_OK;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double* h = (double*)malloc((size_t)dim * sizeof(double));
        if (!h) {
#pragma omp atomic write
            status = ORACLE_ENOMEM;
            continue;
        }
        const double* gr = gate + r * dim;
        for (int64_t c = 0; c < dim; ++c)
            h[c] = x[r * dim + c] + (residual ? residual[r * dim + c] : 0.0);
        if (h_out) memcpy(h_out + r * dim, h, (size_t)dim * sizeof(double));
        double ss = 0.0;
        for (int64_t c = 0; c < dim; ++c) ss += h[c] * h[c];
        double inv = 1.0 / sqrt(ss / (double)dim + eps);
        for (int64_t c = 0; c < dim; ++c) {
            double z = gr[c];
            double act = sigmoid ? 1.0 / (1.0 + exp(-z)) : z / (1.0 + exp(-z));
            y[r * dim + c] = (h[c] * inv * (w ? w[c] : 1.0) + (b ? b[c] : 0.0)) * act;
        }
        free(h);
    }
    return status;
}

/* The plain gated RMSNorm: no residual, no bias, SiLU gate. */
int kda_oracle_gated_rmsnorm(const double* x, const double* gate, const double* w,
                             int64_t rows, int64_t dim, double eps, double* y)
{
    return kda_oracle_gated_rmsnorm_ex(x, gate, NULL, w, NULL, rows, dim, eps, 0, y, NULL);
}
