/*
 * specverify.h -- C ABI of an MI355X (gfx950) library for batched
 * speculative-decoding verification over full-vocabulary logits.
 *
 * The method comes from three pages:
 *   [SD]  "Speculative Decoding: как черновая модель ускоряет генерацию LLM
 *          без потери качества" (zer0kernel forum post): the draft/verify loop
 *          and the lossless accept/resample rule, sections "Основная идея:
 *          черновик и верификация" and "Математика верификации".
 *   [FLy] "Training-Free Loosely Speculative Decoding: Accepting Semantically
 *          Correct Drafts Beyond Exact Match" (gist.science summary): the
 *          entropy gate and deferral window, section "2. Metodologia",
 *          part "A. Mecanismo de Verificacao de Dois Niveis".
 *   [AV]  "Verificacion Adaptativa sin una cabeza de confianza" (spke.com):
 *          the online acceptance estimator sigmoid(omega*logit(q_max)+beta_i),
 *          sections "Solucion", "Puntuar la Distribucion", "Ajuste de los
 *          Coeficientes" and footnote 1 ("Notas al pie").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers named as device pointers must point to HIP device memory (or
 *    memory the device can read).  The library allocates nothing: every
 *    buffer, including scratch ("workspace"), belongs to the caller.
 *  - Apart from the workspaces, whose sizes are arguments, the library cannot
 *    see a device buffer's size: each must hold the elements its description
 *    gives, or a kernel reads or writes past its end.
 *  - Logits are rows of `vocab` values, row r of a tensor starting at
 *    base + r*row_stride elements.  dtype SPEC_DTYPE_F32 (float) or
 *    SPEC_DTYPE_BF16 (bfloat16 bit patterns).  The base pointer must be
 *    16-byte aligned and row_stride*sizeof(element) a multiple of 16.
 *    Logits must be -inf (a masked vocabulary entry) or finite and greater
 *    than -1e30 (the passes treat values at or below -1e30 as "no maximum
 *    yet"); +inf and NaN are not supported.  At least one entry per row must
 *    be finite.
 *  - Every statistic is of the temperature-scaled distribution softmax(l/T).
 *  - All work is enqueued asynchronously on `stream` (a hipStream_t; NULL is
 *    the null stream).  Arguments are validated on the host before anything
 *    is enqueued: on any status other than SPEC_OK nothing was enqueued,
 *    except SPEC_ERR_HIP, which reports a failed launch.
 *  - Results are a pure function of the inputs, the seed and the parameters:
 *    reductions run in a fixed order and no floating-point atomics are used.
 *  - Calls on different streams may overlap if they share no output or
 *    workspace memory.
 *
 * Randomness: Philox4x32-10 (Salmon et al., SC'11) keyed by the 64-bit seed,
 * counter (x>>2, position, sequence, stream tag), output word x&3; a draw r
 * becomes u = (2*(r>>9)+1) * 2^-24.  The accept test at position j uses
 * x = 0 and tag 1.  The sampling race gives vocabulary id x the 32-bit word
 * whose high 16 bits are half x&1 (the low half for even x) of word
 * (x>>1)&3 of the block at counter (x>>3, position, sequence, 3), and whose
 * low 16 bits are the high half of the tag-2 draw for x; u is formed from
 * that word the same way.
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum spec_status {
    SPEC_OK = 0,
    SPEC_ERR_ARG = -1,         /* invalid argument (null, range, alignment)   */
    SPEC_ERR_UNSUPPORTED = -2, /* valid but outside what this build handles   */
    SPEC_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required  */
    SPEC_ERR_HIP = -4          /* a HIP launch reported an error              */
} spec_status;

enum { SPEC_DTYPE_F32 = 0, SPEC_DTYPE_BF16 = 1 };
enum { SPEC_MODE_LOSSLESS = 0, SPEC_MODE_FLY = 1 };

/* Problem description.  B sequences, each with K draft tokens, K draft rows
 * and K+1 target rows (row K follows the last draft token). */
typedef struct spec_params {
    int32_t batch;      /* B >= 0                                            */
    int32_t num_draft;  /* K, 1 <= K <= 64                                   */
    int32_t vocab;      /* V >= 2; a row of V elements must be < 2 GiB      */
                        /* (SPEC_ERR_UNSUPPORTED otherwise)                  */
    int32_t dtype;      /* SPEC_DTYPE_F32 or SPEC_DTYPE_BF16                 */
    int64_t row_stride; /* elements between consecutive rows, >= V           */
    float temperature;  /* T, 1e-4 <= T <= 1e4                               */
    float fly_theta;    /* FLy entropy gate theta on h = H(p)/log V          */
    int32_t fly_window; /* FLy deferral window W, 0 <= W <= 2^20             */
    int32_t reserved;   /* must be 0                                         */
} spec_params;

/* Boundary-case bits of spec_verify_out.boundary.  Each marks a near-tie
 * where the float32 arithmetic of the row pass may legitimately decide the
 * other way than exact arithmetic would; outside them accepted_len and the
 * tokens equal those of an exact evaluation of the rule.
 *   SPEC_NEAR_ACCEPT     an accept test the sequence evaluated (positions
 *                        0..accepted_len, the rejected one included) had
 *                        |u_j - p(x_j)/q(x_j)| < 1e-5 ([SD] section
 *                        "Математика верификации").
 *   SPEC_NEAR_RACE       the two largest keys w(x)/E_x of the sequence's
 *                        sampling race were within 1e-6 relative.
 *   SPEC_RESIDUAL_EMPTY  after a rejection max(0, p - q) rounded to zero at
 *                        every id; the token was drawn from p at that row.
 *   SPEC_NEAR_GATE       (FLy) a gate the scan evaluated had
 *                        |h_j - theta| < 1e-5 ([FLy] part A). */
enum {
    SPEC_NEAR_ACCEPT = 1,
    SPEC_NEAR_RACE = 2,
    SPEC_RESIDUAL_EMPTY = 4,
    SPEC_NEAR_GATE = 8
};

/* Outputs of spec_verify.  accepted_len and tokens are required; every
 * statistics pointer may be NULL.  Rows that a call does not read (target
 * rows past kept_len, draft rows at or past kept_len) are reported as NaN
 * and -1. */
typedef struct spec_verify_out {
    int32_t *accepted_len;   /* [B] draft tokens accepted, 0..kept_len          */
    int32_t *tokens;         /* [B][K+1] emitted tokens: the accepted drafts,
                                then one replacement or bonus token, then -1   */
    float *target_lse;       /* [B][K+1] log-sum-exp of l/T                      */
    float *target_entropy;   /* [B][K+1] normalised entropy h = H/log V          */
    int32_t *target_argmax;  /* [B][K+1] top token, lowest id on ties            */
    float *draft_lse;        /* [B][K] (only when spec_verify reads draft rows)  */
    float *draft_qmax;       /* [B][K] probability of the draft's top token      */
    float *draft_feat;       /* [B][K] logit(q_max), clamped to <= 126 log 2     */
    void *draft_stats_out;   /* device or NULL (16-byte aligned): when the call
                                reads the draft rows itself (lossless mode,
                                draft_stats NULL), their statistics are written
                                here as well, in the layout of
                                spec_draft_stats_bytes, for spec_av_score_stats
                                and spec_av_update                              */
    uint32_t *boundary;      /* [B] or NULL: the sequence's boundary-case bits
                                (SPEC_NEAR_*, SPEC_RESIDUAL_EMPTY), 0 for none */
} spec_verify_out;

/* Bytes of device workspace spec_verify needs for `params` (0 if invalid). */
size_t spec_workspace_bytes(const spec_params *params);

/* Bytes of the draft-statistics buffer that spec_av_score fills and
 * spec_verify / spec_av_update read, for B sequences of K drafts.  Layout
 * (n = B*K, entry b*K+j): double lse2[n] (log2-sum of 2^(l*c), c = log2(e)/T),
 * double logq2[n] (log2 q(x_j)), float qmax[n], float feat[n]. */
size_t spec_draft_stats_bytes(int32_t batch, int32_t num_draft);

/*
 * spec_verify -- verify K draft tokens per sequence against the target.
 *
 * target       device, [B][K+1] rows of logits.
 * draft        device, [B][K] rows of draft logits.  Required in lossless
 *              mode (a rejected position re-reads its draft row even when
 *              draft_stats is given); ignored in FLy mode.
 * draft_tokens device, int32 [B][K].  A token outside [0, V) has p = q = 0:
 *              it is rejected in lossless mode and counts as a deviation in
 *              FLy mode.
 * kept_len     device, int32 [B] or NULL (= K).  Number of leading drafts
 *              that go to verification after adaptive-verification trimming;
 *              values outside [0, K] are clamped.  Only target rows 0..L and
 *              draft rows 0..L-1 are read.
 * draft_stats  device or NULL: the buffer filled by spec_av_score for the
 *              same drafts and temperature; then draft rows are not read.
 * seed         key of every random draw.
 * mode         SPEC_MODE_LOSSLESS: position by position accept x_j when
 *              u_j < p(x_j)/q(x_j) (probability min(1, p/q), [SD] section
 *              "Математика верификации"); at the first rejection emit a token
 *              drawn from norm(max(0, p - q)); if all L verified drafts are
 *              accepted emit a token drawn from p at row L (the bonus token
 *              when L = K, the target's own sample at the trim point when
 *              L < K, [AV] footnote 1).  Draws use the exponential race
 *              argmax_x w(x)/E_x with E_x = -ln u_x.
 *              SPEC_MODE_FLY: greedy exact match relaxed by FLy's entropy gate
 *              and deferral window ([FLy] part A): a deviation (draft token !=
 *              target top token) with h < theta is rejected; one with
 *              h >= theta is accepted when the next W drafts all match and lie
 *              inside the draft, else rejected.  The replacement / bonus token
 *              is the target's top token at that row.  Deterministic.
 * params       problem description (host pointer).
 * out          output pointers (host struct of device pointers).
 * workspace    device scratch of at least spec_workspace_bytes(params) bytes,
 *              owned by the caller; its contents on entry do not matter.
 * stream       hipStream_t to enqueue on.
 */
spec_status spec_verify(const void *target, const void *draft, const int32_t *draft_tokens,
                        const int32_t *kept_len, const void *draft_stats, uint64_t seed,
                        int32_t mode, const spec_params *params, const spec_verify_out *out,
                        void *workspace, size_t workspace_bytes, void *stream);

/*
 * spec_verify_noalloc -- spec_verify without a workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Arguments, outputs,
 * results and errors are those of spec_verify; the scratch spec_verify takes
 * from the caller's workspace lives instead in a fixed device array of
 * SPEC_NOALLOC_SCRATCH_BYTES (16 MiB) that each GPU the library runs on holds
 * until the process ends.  A problem whose spec_workspace_bytes exceeds it
 * returns SPEC_ERR_UNSUPPORTED before anything is enqueued (at K = 8 and
 * V = 128256 that is about 17800 sequences).  No hipMalloc, hipFree or other
 * allocating call is made.  The array belongs to the current device, which
 * must be the stream's device; every call on one GPU shares it, so calls that
 * overlap on one GPU (other streams, other host threads) race and must be
 * serialised by the caller.  Nothing in it needs clearing between calls.
 */
#define SPEC_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
spec_status spec_verify_noalloc(const void *target, const void *draft,
                                const int32_t *draft_tokens, const int32_t *kept_len,
                                const void *draft_stats, uint64_t seed, int32_t mode,
                                const spec_params *params, const spec_verify_out *out,
                                void *stream);

/*
 * spec_av_score -- adaptive-verification confidence and trimming ([AV]
 * sections "Solucion" and "Puntuar la Distribucion"; survival as the running
 * product over positions from section "Otras Caracteristicas Consideradas").
 *
 * Reads every draft row once and, per sequence b and position i < K:
 *   c_i = sigmoid(omega * logit(q_max,i) + beta_i)   -> conf[b][i]
 *   P_i = c_0 * ... * c_i;  keep while P_i >= tau     -> keep_mask, kept_len
 * tau <= 0 keeps every position.  omega_beta: device float[K+1] =
 * (omega, beta_0..beta_{K-1}).  conf (float [B][K]), keep_mask (uint8
 * [B][K]) and kept_len (int32 [B]) may each be NULL.  draft_stats (device,
 * spec_draft_stats_bytes) is required and receives the draft-row statistics
 * for spec_verify and spec_av_update.  draft_tokens (device int32 [B][K]) is
 * required.  params->fly_* are ignored.
 */
spec_status spec_av_score(const void *draft, const int32_t *draft_tokens,
                          const spec_params *params, const float *omega_beta, float tau,
                          float *conf, uint8_t *keep_mask, int32_t *kept_len, void *draft_stats,
                          void *stream);

/*
 * spec_av_score_prefix -- spec_av_score for a step that uses the kept drafts
 * only (verification, labels, refits): each sequence's draft rows are read in
 * order and reading stops after the first trimmed position, whose row
 * decides the trim ([AV] footnote 1: a trimmed position is not verified, the
 * target samples there).  kept_len, keep_mask, and conf and draft_stats for
 * positions 0..min(kept_len, K-1) equal spec_av_score's bit for bit;
 * positions after the first trimmed one are not read: conf and their draft
 * statistics are NaN, keep_mask 0.  With tau <= 0 nothing is trimmed and
 * every row is read.  One workgroup per sequence, so it pays off when B is
 * large (hundreds of sequences or more) and most sequences trim early.
 * Arguments and errors as spec_av_score.
 */
spec_status spec_av_score_prefix(const void *draft, const int32_t *draft_tokens,
                                 const spec_params *params, const float *omega_beta, float tau,
                                 float *conf, uint8_t *keep_mask, int32_t *kept_len,
                                 void *draft_stats, void *stream);

/*
 * spec_av_score_stats -- the scoring and trimming of spec_av_score from
 * draft statistics that are already computed (by spec_av_score, or by
 * spec_verify through draft_stats_out), without reading any draft row:
 * conf, keep_mask and kept_len as in spec_av_score (each nullable).  With
 * tau <= 0 nothing is trimmed, so a step can verify first (one row pass over
 * target and draft rows, exporting the draft statistics) and score after.
 * draft_stats: device, spec_draft_stats_bytes(batch, num_draft), 16-byte
 * aligned; omega_beta: device float[K+1].
 */
spec_status spec_av_score_stats(const void *draft_stats, int32_t batch, int32_t num_draft,
                                const float *omega_beta, float tau, float *conf,
                                uint8_t *keep_mask, int32_t *kept_len, void *stream);

/*
 * spec_av_update -- one online SGD step of the estimator ([AV] section
 * "Ajuste de los Coeficientes" for the labels: drafts up to and including the
 * first rejection; accepted = 1, the first rejected = 0, nothing else
 * labelled).  With N labels over the batch and s_n the pre-step prediction:
 *   omega  -= lr * (1/N) sum_n (s_n - y_n) feat_n
 *   beta_i -= lr * (1/N) sum_{n at position i} (s_n - y_n)
 * N = 0 leaves the parameters unchanged.  draft_stats: filled by
 * spec_av_score; accepted_len: from spec_verify; kept_len: device int32 [B]
 * or NULL (= K); omega_beta: device float[K+1], updated in place.  Single
 * workgroup (a wave per position), fixed-order double-precision sums.
 */
spec_status spec_av_update(const void *draft_stats, const int32_t *accepted_len,
                           const int32_t *kept_len, int32_t batch, int32_t num_draft, float lr,
                           float *omega_beta, void *stream);

/*
 * spec_av_score_update -- for a step with nothing trimmed (tau <= 0), scored
 * after its verification: spec_av_score_stats with tau <= 0 (every draft
 * kept; conf, keep_mask and kept_len each nullable) at the coefficients
 * before the update, then spec_av_update with kept_len NULL, in one launch.
 * The results equal those two calls in that order, bit for bit.
 * draft_stats: device, spec_draft_stats_bytes(batch, num_draft), 16-byte
 * aligned (from spec_verify's draft_stats_out, or spec_av_score);
 * accepted_len: device int32 [B] from spec_verify; omega_beta: device
 * float[K+1], updated in place.  Errors as spec_av_update.
 */
spec_status spec_av_score_update(const void *draft_stats, const int32_t *accepted_len,
                                 int32_t batch, int32_t num_draft, float lr, float *omega_beta,
                                 float *conf, uint8_t *keep_mask, int32_t *kept_len,
                                 void *stream);

/*
 * spec_verify_update -- one adaptive-verification step's verification and
 * update in one call ([SD] section "Математика верификации" for the lossless
 * rule, [AV] section "Ajuste de los Coeficientes" for the update): the
 * results of spec_verify in lossless mode with these arguments followed by
 *   - spec_av_update(draft statistics, accepted_len, kept_len, lr), or
 *   - when any of conf, keep_mask, kept_len_out is non-NULL (an untrimmed
 *     step: kept_len and draft_stats must then be NULL, else SPEC_ERR_ARG),
 *     spec_av_score_update(draft statistics, accepted_len, lr, conf,
 *     keep_mask, kept_len_out),
 * bit for bit.  The draft statistics are draft_stats when given, else those
 * the verify pass computes from the draft rows (written to
 * out->draft_stats_out as well when that is set).  The update's labels need
 * only the accepted lengths, which the race already holds, so the update runs
 * in the same launch as the choice of each sequence's token, beside it.
 * omega_beta: device float [K+1], updated in place; lr finite.  Other
 * arguments, workspace and errors as spec_verify.
 */
spec_status spec_verify_update(const void *target, const void *draft, const int32_t *draft_tokens,
                               const int32_t *kept_len, const void *draft_stats, uint64_t seed,
                               const spec_params *params, const spec_verify_out *out, float lr,
                               float *omega_beta, float *conf, uint8_t *keep_mask,
                               int32_t *kept_len_out, void *workspace, size_t workspace_bytes,
                               void *stream);

/*
 * Newton (IRLS) refit of the estimator ([AV] section "Ajuste de los
 * Coeficientes").  The pages refit omega and the beta_i after every round of
 * N decoding steps: each step adds its labelled drafts (the same labels as
 * spec_av_update) to the gradient g and Hessian H of the summed log-loss at
 * the current coefficients; the last step of the round solves H dtheta = -g
 * and moves each coefficient by dtheta scaled by n / (n + c_damp), n being
 * the labels behind it (all labels for omega, the labels at position i for
 * beta_i).
 *
 * With one shared slope, H has nonzeros only at H[0][0], H[0][1+i] and the
 * diagonal, so the state is 4K+3 doubles (spec_irls_state_bytes): device
 * memory, 8-byte aligned, owned by the caller, zero at the start of a round
 * (spec_irls_reset zeroes it; spec_irls_solve leaves it zeroed).
 *
 * spec_irls_accumulate: draft_stats from spec_av_score, accepted_len from
 *   spec_verify, kept_len device int32 [B] or NULL (= K), omega_beta device
 *   float [K+1] (read only).  One workgroup; fixed-order sums (deterministic).
 * spec_irls_solve: solves over the coefficients that have labels; when the
 *   slope has no curvature of its own left (Schur complement
 *   <= 1e-12 x the largest diagonal entry, e.g. every feature equal) the
 *   slope is held and each intercept takes its own Newton step.  omega_beta
 *   (device float [K+1]) is updated in place; flags (device int32, nullable)
 *   receives bit 0 = updated, bit 1 = slope held.  c_damp >= 0.
 */
size_t spec_irls_state_bytes(int32_t num_draft);
spec_status spec_irls_reset(void *state, int32_t num_draft, void *stream);
spec_status spec_irls_accumulate(const void *draft_stats, const int32_t *accepted_len,
                                 const int32_t *kept_len, int32_t batch, int32_t num_draft,
                                 const float *omega_beta, void *state, void *stream);
spec_status spec_irls_solve(void *state, int32_t num_draft, double c_damp, float *omega_beta,
                            int32_t *flags, void *stream);

/*
 * spec_av_diagnostics -- the estimator's quality over one batch's labels
 * ([AV] section "Otras Caracteristicas Consideradas": AUC, log-loss, ECE).
 * With z = omega*feat + beta_i (double; feat from draft_stats) and
 * s = sigmoid(z) over the labelled drafts:
 *   out[0] AUC: over every (accepted, rejected) pair, the share where the
 *          accepted draft's z is larger, ties counting one half (NaN without
 *          both classes);
 *   out[1] mean log-loss; out[2] ECE over nbins equal-width bins of s;
 *   out[3] the number of labels.
 * out: device double[4].  workspace: device, spec_av_diagnostics_workspace_bytes,
 * 16-byte aligned.  Log-loss and bin sums are accumulated in fixed point
 * (2^-32 and 2^-40 per label), so the result does not depend on the order of
 * the additions.  B*K <= 65536, nbins <= 64, else SPEC_ERR_UNSUPPORTED.
 */
size_t spec_av_diagnostics_workspace_bytes(int32_t batch, int32_t num_draft, int32_t nbins);
spec_status spec_av_diagnostics(const void *draft_stats, const int32_t *accepted_len,
                                const int32_t *kept_len, int32_t batch, int32_t num_draft,
                                const float *omega_beta, int32_t nbins, double *out,
                                void *workspace, size_t workspace_bytes, void *stream);

/*
 * spec_av_budget -- budgeted trimming ([AV] section "Otras Caracteristicas
 * Consideradas", the survival / top-k and draft-budget snippets).
 *   survival(b, i) = conf(b,0) * ... * conf(b,i), formed in float;
 *   the B*K survivals in decreasing order (ties: lower flat index b*K+i
 *   first) are s_(1) >= s_(2) >= ...;
 *   est(k) = n_requests + s_(1) + ... + s_(k),  k = 0..B*K;
 *   budget = the first k maximising est(k) / cost[k];
 *   the first `budget` drafts of that order are kept (a prefix of each
 *   sequence, as survival never grows along a sequence).
 * conf: device float [B][K] (spec_av_score's conf); cost: device double
 * [B*K+1], 8-byte aligned (the measured cost of verifying k drafts).
 * Outputs: kept_len device int32 [B]; keep_mask device uint8 [B][K] or NULL;
 * budget device int64 (8-byte aligned); best_ratio device double or NULL.
 * workspace: device, spec_av_budget_workspace_bytes, 16-byte aligned.  The
 * order is found by counting, for every draft, the keys below its own over
 * the whole GPU (O((B*K)^2) comparisons): B*K <= 65536, else
 * SPEC_ERR_UNSUPPORTED.
 */
size_t spec_av_budget_workspace_bytes(int32_t batch, int32_t num_draft);
spec_status spec_av_budget(const float *conf, int32_t batch, int32_t num_draft, const double *cost,
                           double n_requests, int32_t *kept_len, uint8_t *keep_mask,
                           int64_t *budget, double *best_ratio, void *workspace,
                           size_t workspace_bytes, void *stream);

/*
 * spec_ngram_propose -- prompt-lookup drafting ([SD] section "N-gram (prompt
 * lookup)"; [FLy] section "B. Aceleracao Multinivel"): for each sequence,
 * the longest suffix n-gram of its context (n from n_max down to n_min) that
 * also occurs earlier; of its earlier occurrences the latest; the draft is
 * the up to num_draft tokens that followed it.
 * context: device int32 [B][stride]; lengths: device int32 [B] (clamped to
 * [0, stride]).  Outputs (device int32): draft [B][num_draft] (-1 after
 * draft_len), draft_len [B], match_pos [B] (start of the matched occurrence,
 * -1 when none; nullable), match_n [B] (its length, 0 when none; nullable).
 * 1 <= n_min <= n_max <= 32, num_draft <= 64.
 */
spec_status spec_ngram_propose(const int32_t *context, const int32_t *lengths, int32_t batch,
                               int64_t stride, int32_t n_min, int32_t n_max, int32_t num_draft,
                               int32_t *draft, int32_t *draft_len, int32_t *match_pos,
                               int32_t *match_n, void *stream);

/*
 * spec_row_stats -- the streaming row pass on its own: per row of V logits,
 * log-sum-exp of l/T (lse), normalised entropy (entropy), top token (argmax,
 * lowest id on ties), top-token probability (qmax) and its log-odds (feat,
 * clamped to <= 126 log 2).  `rows` rows starting at `logits`; every output
 * is a device array of `rows` entries and may be NULL.
 */
spec_status spec_row_stats(const void *logits, int64_t rows, int32_t vocab, int64_t row_stride,
                           int32_t dtype, float temperature, float *lse, float *entropy,
                           int32_t *argmax, float *qmax, float *feat, void *stream);

/*
 * spec_read_probe -- a measurement aid, not part of verification: streams
 * `rows` rows of `row_bytes` bytes each (consecutive rows `row_stride_bytes`
 * apart) with the same loads, workgroup shape and one-workgroup-per-row grid
 * as the row pass on bfloat16 rows, but with almost no arithmetic, and stores
 * the XOR of each row's 32-bit words in sink[row].  Its bandwidth is the
 * ceiling the row pass can reach on the same rows.  logits: device, 16-byte
 * aligned; row_bytes and row_stride_bytes: multiples of 16, row_bytes <=
 * row_stride_bytes (row_bytes beyond 2^31 - 1: SPEC_ERR_UNSUPPORTED); sink:
 * device uint32 [rows].  Asynchronous on `stream`.
 */
spec_status spec_read_probe(const void *logits, int64_t rows, int64_t row_bytes,
                            int64_t row_stride_bytes, uint32_t *sink, void *stream);

/* Static description of a status code. */
const char *spec_status_string(int32_t status);

#ifdef __cplusplus
}
#endif
#endif
