/*
 * libisd -- Introspective Strided Decoding (ISD) verify-and-propose step on
 * AMD Instinct MI355X (gfx950).
 *
 * The step follows "Introspective Diffusion Language Models | Summary"
 * (greeksharifa.github.io):
 *   - section 2 (Background and Motivation) defines the introspective
 *     acceptance rate alpha: the mean over the L proposed positions of
 *     min(1, p_k(x_k) / q_k(x_k)), with q_k the law that generated x_k and
 *     p_k the causal anchor that scores it;
 *   - section 3.2 (Introspective Strided Decoding) keeps each proposal with
 *     probability min(1, p_k(x_k)/q_k(x_k)), replaces the first rejected one by
 *     a draw from normalize(max(0, p_k - q_k)), drops every later proposal, and
 *     takes the next proposals from the mask positions of the same forward;
 *   - section 3.3 (I-DLM Serving Stack) proposes by argmax and verifies
 *     strictly (ISD_MODE_GREEDY).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layout.  Logits rows are V contiguous elements; row (c, k) starts at
 *   element c*ldc + k*ld of its buffer, with ld >= V and ldc either 0 (which
 *   means L*ld, a dense [C, L, V] tensor) or >= L*ld.  A [C, 2L, V] extend
 *   output whose first L rows per sequence are anchors and last L are mask
 *   rows is passed as p = base, qnext = base + L*ld, ld = V, ldc = 2L*V.
 *   Token and uniform arrays are dense [C, L] (row-major).
 *   p_logits[c, k] is the anchor row that scores proposal x[c, k] (the
 *   next-token logit shift is applied by the caller); q_logits[c, k] is the
 *   proposal row that generated x[c, k]; qnext_logits[c, k] is the mask row
 *   whose draw becomes the next proposal at position k.
 * Memory.  Every pointer argument except `s` is device memory owned by the
 *   caller; the library never allocates, frees or keeps a pointer.  `s` is a
 *   host pointer read synchronously.
 * Workspace.  Size it with isd_workspace_bytes() for the same shape.  It must
 *   be zero-filled before its first use; every call leaves it zero-filled
 *   again once its kernels have finished (it holds work counters and
 *   per-row partial results).  So the workspace carries state from one call
 *   to the next: its zero state.  A decision published inside a launch is
 *   tagged with that launch's epoch (a library-wide counter), so a record
 *   left behind by a launch that flagged the device error word can never be
 *   taken for a later launch's; the workspace must still be zero-filled again
 *   after isd_check_device_error() returns ISD_ERR_DEVICE.  One workspace
 *   serves one call at a time: calls that share a workspace must be ordered
 *   on one stream; calls that overlap on one workspace race.
 * Asynchrony.  Every call validates its arguments on the host, enqueues its
 *   kernels on `stream` (a hipStream_t; NULL is the null stream) and returns;
 *   outputs are valid once the stream has reached that point.
 * Draws.  Randomness is passed in: one uniform in [0, 1) per decision.  A
 *   proposal is kept iff u_accept < min(1, P(x)/Q(x)).  The residual and the
 *   proposals are inverse-CDF draws over ascending vocab index: the token is
 *   the smallest i whose running weight sum exceeds u * (total weight).
 * Precision.  Streaming sums are fp32 per 32-element lane block, accumulated
 *   in fp64; decisions use fp64 ratios.  Residual weights are formed as
 *   a_i - rho*b_i with the ratio of the two rows' denominators carried as a
 *   pair of fp32 numbers, so no row-wide rounding enters the difference.
 *   Probabilities match an exact fp64 evaluation to ~1e-7 relative; a
 *   residual draw's cumulative weights agree to ~1e-7 * P_max / Z (P_max the
 *   anchor row's largest probability, Z the residual mass), so only draws
 *   within ~1e-6 of a boundary come out differently unless Z is below ~0.01.
 * Errors.  On a non-OK status nothing has been enqueued and no output or
 *   workspace byte is touched; isd_last_error() then describes the problem.
 *     ISD_ERR_ARG          bad shape (C < 1, L not in [1, 64], V < 1, ld < V,
 *                          0 < ldc < L*ld),
 *                          a required NULL pointer, a base not aligned to its
 *                          element size, T <= 0 / non-finite in sample mode,
 *                          relax < 0, q_onehot or sampler out of range,
 *                          top_k < 0, top_p < 0 or NaN
 *     ISD_ERR_UNSUPPORTED  unknown dtype or mode, top_k > 64, top_p < 1
 *                          without top_k
 *     ISD_ERR_WORKSPACE    ws_bytes smaller than isd_workspace_bytes()
 *     ISD_ERR_DEVICE       a HIP call failed (text in isd_last_error())
 *   Out-of-range proposal ids and NaN/+inf logits are undefined input; the
 *   kernels never read out of bounds because of them, and record them in a
 *   device error word that isd_check_device_error() reports.
 */
#ifndef ISD_H
#define ISD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ISD_OK = 0,
    ISD_ERR_ARG = 1,
    ISD_ERR_UNSUPPORTED = 2,
    ISD_ERR_WORKSPACE = 3,
    ISD_ERR_DEVICE = 4
} isd_status_t;

typedef enum { ISD_DTYPE_BF16 = 0, ISD_DTYPE_F32 = 1 } isd_dtype_t;

/* ISD_MODE_SAMPLE: probabilistic acceptance with residual correction
 * (section 3.2).  ISD_MODE_GREEDY: argmax proposals verified strictly
 * (section 3.3): x_k is kept iff it equals argmax p_k (ties to the lowest
 * index, raw logits, temperature ignored), the correction is that argmax,
 * alpha is the match fraction, proposals are argmax of the mask rows, and
 * q_logits and all uniforms are ignored (may be NULL). */
typedef enum { ISD_MODE_SAMPLE = 0, ISD_MODE_GREEDY = 1 } isd_mode_t;

/* How the correction token is drawn from the residual max(0, P - Q) (P if
 * that is empty) after a rejection (sample mode; section 3.2).
 * ISD_SAMPLER_CDF: inverse CDF in vocabulary order at the uniform
 *   u_resid[c, j].
 * ISD_SAMPLER_GUMBEL: Gumbel-max, the correction of the pages' fused
 *   verification kernel (section 3.3): argmax_i ln w_i + G_i with standard
 *   Gumbel noise G_i = -ln(-ln U_i), ties to the lowest index.  U_i comes from
 *   Philox4x32-10 (Salmon et al., SC 2011) with key (bits of the fp32
 *   u_resid[c, j], c) and counter (i / 4, j, 0x15D, 0), word i % 4 of the
 *   block w giving U_i = (2 * (w >> 9) + 1) / 2^24; c is the sequence's index
 *   in the call.  Same law as the inverse CDF, different samples. */
typedef enum { ISD_SAMPLER_CDF = 0, ISD_SAMPLER_GUMBEL = 1 } isd_sampler_t;

/* Truncated laws (sample mode, top_k >= 1).  The pages' quality runs sample
 * with top-k 50 and top-p 0.95 (section 4.1), and verification must use the
 * law of the proposal mechanism actually used (section 3.3).  So with
 * truncation P, Q and the law of the next proposals are all the truncated
 * laws of their rows: rank the entries of a row by logit, larger first, ties
 * to the lower index (-0 ranks as +0); keep the first top_k ranks; then, if
 * top_p is on, keep a rank while the probability mass of the ranks before it
 * (in the top-k renormalised law at temperature T) is below top_p; the
 * survivors are renormalised.  Proposals and the correction draw over the
 * survivors in increasing vocabulary index, exactly as without truncation.
 * Greedy mode ignores truncation: it never changes an argmax.  top_p without
 * top_k is ISD_ERR_UNSUPPORTED. */

typedef struct {
    int32_t C;           /* concurrent sequences, >= 1 */
    int32_t L;           /* strided positions per step, 1..64 */
    int32_t V;           /* vocabulary size, >= 1 */
    int64_t ld;          /* elements between consecutive logits rows, >= V */
    int32_t dtype;       /* isd_dtype_t of every logits tensor */
    int32_t mode;        /* isd_mode_t */
    float temperature;   /* softmax temperature T > 0 (sample mode) */
    int64_t ldc;         /* elements between sequences c and c+1 (0: L*ld) */
    float relax;         /* tau >= 0 (sample mode): accept with min(1, (1 + tau) P(x)/Q(x)),
                            the relaxed acceptance of the pages' ablation (section 4); 0 is
                            the exact rule.  alpha and the correction are unchanged. */
    int32_t q_onehot;    /* 1 (sample mode): the proposals were argmax picks, so their law
                            is one-hot at x (section 3.3 with a sampled anchor): q_logits
                            is not read (may be NULL), the ratio is P(x), and the
                            correction draws from P with x removed.  0: q_logits as given */
    int32_t sampler;     /* isd_sampler_t of the correction draw (sample mode) */
    int32_t top_k;       /* sample mode: 0 = no truncation; 1..64 = keep the top_k
                            highest-ranked entries of every row (ranked by logit, ties to
                            the lower index) */
    float top_p;         /* sample mode, with top_k >= 1: nucleus mass in (0, 1); 0 (the
                            zero-initialised value) or >= 1 turns it off.  See the
                            truncated laws below. */
} isd_shape_t;

/* Workspace bytes needed by any call on shape `s`; 0 if `s` is invalid. */
size_t isd_workspace_bytes(const isd_shape_t *s);

/* Verification of the previous step's proposals (section 3.2; strict
 * variant section 3.3).
 *   p_logits, q_logits  [C, L, V] logits (q ignored in greedy mode)
 *   proposals           [C, L] int32 proposal ids x, in [0, V)
 *   u_accept, u_resid   [C, L] fp32 uniforms; the residual draw uses
 *                       u_resid[c, j] at the first rejected position j
 * outputs (device):
 *   accept_len [C]      j = number of leading proposals kept (L if none fails)
 *   out_tokens [C, L]   x[c, 0..j-1], then the correction at j when j < L,
 *                       then -1
 *   n_emitted  [C]      j + (j < L); no bonus token is drawn after a full accept
 *   p_x, q_x   [C, L]   P_k(x_k), Q_k(x_k) (greedy: 1 if x_k matches else 0,
 *                       and 1); may be NULL
 *   alpha      [C]      per-sequence alpha over all L positions; may be NULL */
isd_status_t isd_verify_step(const isd_shape_t *s,
                             const void *p_logits, const void *q_logits,
                             const int32_t *proposals,
                             const float *u_accept, const float *u_resid,
                             int32_t *accept_len, int32_t *out_tokens, int32_t *n_emitted,
                             float *p_x, float *q_x, float *alpha,
                             void *workspace, size_t ws_bytes, void *stream);

/* Next proposals from the mask-position logits (section 3.2, Algorithm 1's
 * mask positions; greedy: argmax, section 3.3).  All C*L draws are made; a
 * caller whose step rejected (accept_len < L) discards them.
 *   qnext_logits [C, L, V]; u_propose [C, L] fp32 (ignored in greedy mode)
 *   next_tokens  [C, L] int32 out; qnext_x [C, L] fp32 out: the proposal's
 *   probability under softmax(qnext/T) (greedy: 1); may be NULL */
isd_status_t isd_propose(const isd_shape_t *s,
                         const void *qnext_logits, const float *u_propose,
                         int32_t *next_tokens, float *qnext_x,
                         void *workspace, size_t ws_bytes, void *stream);

/* The introspective acceptance rate alone (section 2): alpha[c] is the mean
 * over k of min(1, P_k(x_k)/Q_k(x_k)) (greedy: the match fraction);
 * alpha_mean [1] is the mean over sequences (may be NULL). */
isd_status_t isd_alpha(const isd_shape_t *s,
                       const void *p_logits, const void *q_logits,
                       const int32_t *proposals,
                       float *alpha, float *alpha_mean,
                       void *workspace, size_t ws_bytes, void *stream);

/* One fused ISD step: isd_verify_step and isd_propose in one launch, as the
 * single forward of section 3.2 yields both the anchor rows that verify the
 * previous proposals and the mask rows that propose the next ones.  Arguments
 * and outputs are those of the two calls; results are identical to calling
 * isd_verify_step then isd_propose. */
isd_status_t isd_step(const isd_shape_t *s,
                      const void *p_logits, const void *q_logits,
                      const int32_t *proposals,
                      const float *u_accept, const float *u_resid,
                      const void *qnext_logits, const float *u_propose,
                      int32_t *accept_len, int32_t *out_tokens, int32_t *n_emitted,
                      float *p_x, float *q_x, float *alpha,
                      int32_t *next_tokens, float *qnext_x,
                      void *workspace, size_t ws_bytes, void *stream);

/* ---- The multi-step decoding loop (section 3.2) ----------------------------
 * After every proposal passes, one more token is drawn from the final causal
 * anchor (the bonus); after a rejection the next step only proposes (a
 * recovery step that draws one token from the anchor of the last clean
 * position).  A sequence is in state 0 (recovery) or 1 (verify).  One loop
 * step for a batch with rows p [C, L+1, V] (rows 0..L-1 verify, row L is the
 * bonus anchor, row 0 is the anchor of a recovering sequence), q, qn [C, L, V]:
 *   1. isd_step_masked with verify_mask = state (recovering sequences verify
 *      nothing) and propose_mask NULL;
 *   2. isd_decode_masks: bonus_mask = state == 1 && accept_len == L,
 *      anchor_mask = state == 0;
 *   3. isd_propose_masked on rows p[:, L] (shape L = 1) with bonus_mask, and
 *      on rows p[:, 0] with anchor_mask;
 *   4. isd_decode_commit: appends the emitted tokens, counts tokens and
 *      forwards, and moves each sequence to its next state. */

/* isd_step with per-sequence masks (int32 [C], nonzero = active; NULL = all).
 * A sequence outside verify_mask reads no p, q or x row and gets
 * accept_len -1, n_emitted 0, out_tokens -1, p_x = q_x = alpha = 0.  A
 * sequence outside propose_mask reads no qn row and gets next_tokens -1 and
 * qnext_x 0.  Other sequences get exactly what isd_step gives them. */
isd_status_t isd_step_masked(const isd_shape_t *s,
                             const void *p_logits, const void *q_logits,
                             const int32_t *proposals,
                             const float *u_accept, const float *u_resid,
                             const void *qnext_logits, const float *u_propose,
                             const int32_t *verify_mask, const int32_t *propose_mask,
                             int32_t *accept_len, int32_t *out_tokens, int32_t *n_emitted,
                             float *p_x, float *q_x, float *alpha,
                             int32_t *next_tokens, float *qnext_x,
                             void *workspace, size_t ws_bytes, void *stream);

/* isd_propose with a per-sequence mask (int32 [C], nonzero = draw; NULL =
 * all); masked-out sequences read no row and get next_tokens -1. */
isd_status_t isd_propose_masked(const isd_shape_t *s,
                                const void *qnext_logits, const float *u_propose,
                                const int32_t *mask,
                                int32_t *next_tokens, float *qnext_x,
                                void *workspace, size_t ws_bytes, void *stream);

/* Draw masks of one loop step from the state before it and the step's
 * accept_len (all int32 [C]). */
isd_status_t isd_decode_masks(int32_t C, int32_t L, const int32_t *state,
                              const int32_t *accept_len, int32_t *bonus_mask,
                              int32_t *anchor_mask, void *stream);

/* Closes one loop step.  A verifying sequence emits out_tokens[c, 0..j]
 * (j + 1 tokens) when it rejected at j < L and moves to recovery, or
 * out_tokens[c, 0..L-1] and bonus[c] (L + 1 tokens) and stays verifying; a
 * recovering sequence emits anchor[c] and moves to verify.  The tokens are
 * appended to history [C, hist_cap] (int32; those past hist_cap are dropped;
 * history may be NULL when hist_cap is 0), tokens [C] (int64) counts every
 * emitted token, forwards [C] (int64) the steps; state [C] is updated in
 * place. */
isd_status_t isd_decode_commit(int32_t C, int32_t L, int32_t *state, const int32_t *accept_len,
                               const int32_t *out_tokens, const int32_t *bonus,
                               const int32_t *anchor, int32_t *history, int64_t hist_cap,
                               int64_t *tokens, int64_t *forwards, void *stream);

/* Logits projection ahead of the step (the LM head that produces every p and
 * mask row of the extend forward, section 3.3): logits[M, N] = h[M, K] @
 * w[K, N], bf16 inputs, fp32 accumulation on the matrix cores, rounded to
 * bf16 (nearest-even).  All three matrices are dense row-major; requires
 * K % 64 == 0; M, N >= 1.  No workspace is used (pass NULL, 0). */
isd_status_t isd_lm_head(const void *h, const void *w, int32_t M, int32_t K, int32_t N,
                         void *logits, void *workspace, size_t ws_bytes, void *stream);

/* The LM head on a pre-packed head: logits[M, N] = h[M, K] @ wt[N, K]^T,
 * where wt = w^T is k-contiguous per vocabulary row (isd_lm_head_pack).  Same
 * arithmetic and rounding as isd_lm_head; K % 64 == 0; h and wt 16-byte
 * aligned.  The workspace is optional (NULL, 0: none): given at least
 * isd_gemm_workspace_bytes(M, K, N) bytes, 256-byte aligned and zero-filled
 * before its first use, the output tiles of a last partial round over the
 * CUs are computed as two halves along K that meet in it (each call leaves
 * its counters zero again; calls that share one workspace must not overlap).
 * Those tiles then sum two fp32 partial products, so they can differ from the
 * unsplit result by the fp32 rounding of that sum; the split is deterministic. */
isd_status_t isd_lm_head_packed(const void *h, const void *wt, int32_t M, int32_t K, int32_t N,
                                void *logits, void *workspace, size_t ws_bytes, void *stream);

/* Bytes of the optional workspace of isd_lm_head_packed and isd_lora_gemm
 * for an output of M x N and a (first) K segment of K; 0 when the K split
 * does not apply to the shape (the workspace is then not used). */
size_t isd_gemm_workspace_bytes(int32_t M, int32_t K, int32_t N);

/* One-time packing of a head w[K, N] (bf16, row-major) into wt[N, K]
 * (caller-allocated, 16-byte aligned): a bit-exact transpose. */
isd_status_t isd_lm_head_pack(const void *w, int32_t K, int32_t N, void *wt, void *stream);

/* Waits for `stream`, then reads and clears the device error word of
 * `workspace`.  Returns ISD_OK if no kernel flagged undefined input or an
 * expired internal wait since the last check, else ISD_ERR_DEVICE with the
 * flags described by isd_last_error().  After ISD_ERR_DEVICE the workspace
 * must be zero-filled again before reuse. */
isd_status_t isd_check_device_error(void *workspace, size_t ws_bytes, void *stream);

/* isd_step for callers that cannot allocate or pass memory for a workspace
 * (code under stream capture into a graph, tight serving loops, harnesses
 * that forbid allocation).  Same arguments, outputs and conventions as
 * isd_step without workspace and ws_bytes; the kernels keep their counters
 * and partial results in a fixed 16 MiB device array of the library instead,
 * one per device, held until the process ends.  The first call on a device
 * zero-fills that array (one kernel on the null stream, waited for); every
 * call leaves it zero again.  No call allocates or frees memory.
 *   device_error  NULL, or device memory for one uint32: after the step, a
 *                 small kernel on `stream` moves the device error word there
 *                 (the bits isd_check_device_error describes: 1 proposal id
 *                 out of range, 2 row without a finite logit, 4 expired
 *                 wait) and clears it; 0 means none.
 * Every call on one device shares that device's array: calls that overlap
 * on one device (other streams or threads) race and must be ordered by the
 * caller.  Shapes whose isd_workspace_bytes() exceeds 16 MiB are rejected
 * with ISD_ERR_WORKSPACE before anything is enqueued (the serving step needs
 * about 1 MiB, C=256, L=16 about 7.4 MiB). */
isd_status_t isd_step_noalloc(const isd_shape_t *s, const void *p_logits, const void *q_logits,
                              const int32_t *proposals, const float *u_accept,
                              const float *u_resid, const void *qnext_logits,
                              const float *u_propose, int32_t *accept_len, int32_t *out_tokens,
                              int32_t *n_emitted, float *p_x, float *q_x, float *alpha,
                              int32_t *next_tokens, float *qnext_x, uint32_t *device_error,
                              void *stream);

/* Measurement: a streaming-read probe.  Reads the `bytes` bytes at `buf`
 * (device memory, 16-byte aligned; bytes a multiple of 4096 and at most
 * 2^31 elements of 2 bytes) once, with the step kernel's own tile loader:
 * each workgroup streams `tiles_per_group` consecutive 4 KiB tiles (the
 * step's verify segments are 38).  Nothing is written except, with
 * negligible probability, one word at `sink` (device memory).  Its time over
 * `bytes` is the read rate the step's loop can reach on the device, the
 * practical ceiling beside the HBM peak ("Introspective Diffusion Language
 * Models | Summary", section 2: decoding speed is bound by memory
 * bandwidth).  ISD_ERR_ARG for bad sizes or pointers, ISD_ERR_DEVICE if the
 * launch fails. */
isd_status_t isd_read_probe(const void *buf, size_t bytes, int32_t tiles_per_group,
                            uint32_t *sink, void *stream);

/* Tuning knobs, process-wide (they apply to every later call of every
 * thread; the calls themselves stay reentrant); 0 restores the automatic
 * choice.
 *   segments          workgroups sharing one verify row (1..32)
 *   propose_segments  workgroups sharing one mask row (1..32)
 *   resid_segments    workgroups sharing one residual row pair (1..64)
 *   spin_limit        bound on the polls of an internal cross-workgroup wait
 *                     before it gives up and flags the device error word */
isd_status_t isd_set_tuning(int32_t segments, int32_t propose_segments, int32_t resid_segments,
                            int64_t spin_limit);

/* The LM head with softmax statistics (fused epilogue).  Like
 * isd_lm_head_packed (logits [M, N] = h [M, K] wt[N, K]^T, bf16, K a multiple
 * of 64), and in the same launch, for every output row and 128-column tile t:
 *   stats[(row * ceil(N / 128) + t) * 2 + 0] = e = ceil(max_i x_i * k2)
 *   stats[(row * ceil(N / 128) + t) * 2 + 1] = sum_i 2^(x_i * k2 - e)
 * over the bf16 logits x it writes, k2 = log2(e) / temperature; e is an
 * integer (fp32), -inf for a tile past N.  stats: fp32, 8-byte aligned,
 * M * ceil(N / 128) * 2 values.  An extend forward's rows (per sequence L
 * anchor rows then L mask rows) give both the p and the qn statistics of a
 * step; the q statistics are the previous step's qn statistics.  workspace,
 * ws_bytes: optional, as for isd_lm_head_packed (the same K split, so the
 * logits equal isd_lm_head_packed's given a workspace too). */
isd_status_t isd_lm_head_stats(const void *h, const void *wt, int32_t M, int32_t K, int32_t N,
                               float temperature, void *logits, float *stats, void *workspace,
                               size_t ws_bytes, void *stream);

/* isd_step fed by those statistics (sample mode, no top-k): the softmax
 * denominators and the proposal draws come from the tile partials, and the
 * logits are read only at the proposals x, along the residual rows p_j, q_j
 * of rejecting sequences and in the one 128-column tile where each proposal
 * draw lands.  Same outputs, conventions and workspace as isd_step; the
 * statistics must be those of the same logits at the same temperature.
 *   p_stats, q_stats, qn_stats  tile partials of rows (c, k) of p, q, qn at
 *     stats + 2 * (c * stats_ldc + k * stats_ld); stats_ld >= ceil(V / 128),
 *     stats_ldc = 0 means L * stats_ld.  q_stats may be NULL with q_onehot.
 * Two launches on `stream` (decisions and proposals, then the residual
 * draws) when C + ceil(C * L / 8) <= 256, else three.  Errors as isd_step,
 * and ISD_ERR_UNSUPPORTED in greedy mode or with top_k. */
isd_status_t isd_step_fused(const isd_shape_t *s, const void *p_logits, const void *q_logits,
                            const int32_t *proposals, const float *u_accept, const float *u_resid,
                            const void *qnext_logits, const float *u_propose,
                            const float *p_stats, const float *q_stats, const float *qn_stats,
                            int64_t stats_ld, int64_t stats_ldc, int32_t *accept_len,
                            int32_t *out_tokens, int32_t *n_emitted, float *p_x, float *q_x,
                            float *alpha, int32_t *next_tokens, float *qnext_x, void *workspace,
                            size_t ws_bytes, void *stream);

/* Segment-gated LoRA projection of the residual ISD variant (appendix G;
 * section 3.2): h_j = W x_j + [mask_j != 0] B A x_j.  The adapter acts only at
 * mask positions, so clean and introspection rows keep the base weights and
 * the causal anchor stays the base model's.  Everything is bf16 bit patterns,
 * row-major, output features first (the torch Linear layout):
 *   x     [M, K]       inputs, 16-byte aligned
 *   a     [r, K]       adapter down-projection A, 16-byte aligned
 *   wcat  [N, K + r]   (W | B) from isd_lora_pack, 16-byte aligned
 *   mask  [M] int32    nonzero at mask positions; NULL: every row
 *   t     [M, r]       written: the gated adapter activations gate * A x
 *                      (bf16, zero on clean rows); caller-owned scratch,
 *                      16-byte aligned
 *   out   [M, N]       written: h, fp32 accumulation rounded to bf16; must
 *                      not overlap the other buffers.  When it is 16-byte
 *                      aligned, r is a multiple of 128 and it can hold
 *                      ceil(K / 256) * M * r floats, it first holds the
 *                      shrink's partial sums (split over K)
 *   workspace, ws_bytes  optional, as for isd_lm_head_packed: with at least
 *                      isd_gemm_workspace_bytes(M, K, N) bytes the GEMM
 *                      halves the tiles of its last partial round along K
 *                      (the halves split at the same K step as the base
 *                      projection's, so clean rows still equal it bit for
 *                      bit when both are given a workspace)
 * K and r must be multiples of 64.  Two or three launches on `stream` (the
 * shrink, in one kernel or as partial sums and their sum, then one GEMM over
 * the concatenated K); no host synchronisation, no allocation, so the call
 * can be captured in a graph.  Errors: ISD_ERR_ARG
 * for bad sizes or pointers, ISD_ERR_DEVICE if a launch fails. */
isd_status_t isd_lora_gemm(const void *x, const void *a, const void *wcat, const int32_t *mask,
                           int32_t M, int32_t K, int32_t N, int32_t r, void *t, void *out,
                           void *workspace, size_t ws_bytes, void *stream);

/* wcat [N, K + r] = (W [N, K] | B [N, r]), row by row (two 2-D device copies on
 * `stream`, done once per adapter).  All bf16, 2-byte aligned. */
isd_status_t isd_lora_pack(const void *w, const void *b, int32_t N, int32_t K, int32_t r,
                           void *wcat, void *stream);

/* Tuning knob of the truncated (top-k) path, process-wide: workgroups sharing
 * one row (1..8); 0 restores the automatic choice. */
isd_status_t isd_set_trunc_tuning(int32_t segments);

/* Thread-local description of the last non-OK status of this thread. */
const char *isd_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ISD_H */
