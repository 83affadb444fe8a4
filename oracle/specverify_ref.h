/*
 * specverify_ref.h -- CPU oracle for speculative-decoding verification over
 * full-vocabulary logits.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the plain, slow, obviously-correct
 * reference that the HIP library is checked against.  Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load it.  It shares
 * no code, header, table or helper with the HIP library; the only thing both
 * sides have in common is the published definition of Philox4x32-10
 * (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3",
 * SC'11), which each side implements on its own.
 *
 * All arithmetic is IEEE double.  Inputs are logits rows stored as float32
 * (dtype 0) or bfloat16 bit patterns (dtype 1); a bfloat16 value is widened
 * exactly to float and then to double.
 *
 * Sources (the three pages the method is described on):
 *   [AV]  "Verificacion Adaptativa sin una cabeza de confianza" (spke.com)
 *   [FLy] "Training-Free Loosely Speculative Decoding: Accepting Semantically
 *          Correct Drafts Beyond Exact Match" (gist.science summary)
 *   [SD]  "Speculative Decoding: как черновая модель ускоряет генерацию LLM
 *          без потери качества" (zer0kernel forum post)
 */
#ifndef SPECVERIFY_REF_H
#define SPECVERIFY_REF_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Philox stream tags: the fourth counter word, keeping draws disjoint. */
#define REF_TAG_ACCEPT 1u /* uniform u_j of the accept test at position j   */
#define REF_TAG_RACE 2u   /* per-vocab-id uniforms of the sampling race      */
#define REF_TAG_SCREEN 3u /* high half of each race word (see ref_race_u32) */

/* Boundary-case bits reported per sequence (near-ties where an fp32 device
 * computation may legitimately decide the other way). */
#define REF_NEAR_ACCEPT 1u   /* |u_j - p/q| < 1e-5 at an evaluated position     */
#define REF_NEAR_RACE 2u     /* top two race keys within 1e-6 relative          */
#define REF_RESIDUAL_EMPTY 4u/* residual max(0,p-q) vanished: raced over p      */
#define REF_NEAR_GATE 8u     /* |h_j - theta| < 1e-5 at an evaluated deviation  */
#define REF_NEAR_TRIM 16u    /* |P_i - tau| <= 1e-5 tau for some position       */

#define REF_MODE_LOSSLESS 0
#define REF_MODE_FLY 1

/* Philox4x32-10 block function: 4-word counter, 2-word key -> 4 words. */
void ref_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);

/* One 32-bit draw: key = (seed low, seed high), counter = (x>>2, pos, b, tag),
 * output word x&3. */
uint32_t ref_draw_u32(uint64_t seed, uint32_t x, uint32_t pos, uint32_t b, uint32_t tag);

/* Uniform on the odd 2^-24 lattice: u = (2*(r>>9)+1) * 2^-24, in (0,1). */
double ref_uniform(uint64_t seed, uint32_t x, uint32_t pos, uint32_t b, uint32_t tag);

/* The sampling race's 32-bit word for vocabulary id x at (pos, b): high 16
 * bits = half (x&1) of word (x>>1)&3 of the block at counter
 * (x>>3, pos, b, REF_TAG_SCREEN); low 16 bits = the high half of
 * ref_draw_u32(seed, x, pos, b, REF_TAG_RACE). */
uint32_t ref_race_u32(uint64_t seed, uint32_t x, uint32_t pos, uint32_t b);

/* The race's uniform: ref_race_u32 on the same 2^-24 lattice. */
double ref_race_uniform(uint64_t seed, uint32_t x, uint32_t pos, uint32_t b);

/* Row statistics of nrows rows of V logits (row r starts at base + r*stride
 * elements).  Every output pointer may be NULL.  Per row, with z = l/T:
 *   m = max z, lse = log sum exp z, H = -sum p log p, h = H/log V,
 *   argmax = smallest id attaining m, qmax = max p,
 *   feat = logit(qmax) = -log(sum_{x != argmax} exp(z_x - m)),
 *          clamped to at most 126 log 2.
 * Returns 0, or -1 on bad arguments. */
int ref_rows_stats(const void *base, int64_t nrows, int64_t V, int64_t stride, int dtype,
                   double temperature, double *m, double *lse, double *H, double *h,
                   int64_t *argmax, double *qmax, double *feat, int nthreads);

/* Probability vector of one row at temperature T (V doubles). */
int ref_row_probs(const void *row, int64_t V, int dtype, double temperature, double *p);

/* Exponential race: argmax_x w[x]/E_x, E_x = -log u(seed, x, pos, b, RACE),
 * over entries with w[x] > 0, lowest id on ties.  Returns -1 when no entry is
 * positive.  *rel_gap (nullable) receives (k1-k2)/k1 for the two largest keys. */
int64_t ref_race(const double *w, int64_t V, uint64_t seed, uint32_t pos, uint32_t b,
                 double *rel_gap);

/* Residual weights w = max(0, p - q) (unnormalised; the race normalises). */
void ref_residual(const double *p, const double *q, int64_t V, double *w);

/* FLy two-level resolver over a draft of length L: dev[j] != 0 marks a
 * deviation from the target's top prediction, h[j] the target's normalised
 * entropy.  Returns the number of accepted draft tokens; *gate_gap (nullable)
 * receives the smallest |h_j - theta| over the gates the scan evaluated
 * (+inf when none); the gate is a boundary case when that is below 1e-5. */
int ref_fly_resolve(int L, int W, double theta, const int32_t *dev, const double *h,
                    double *gate_gap);

/* Full verification of B sequences (see specverify_ref.c for the steps).
 * target: [B][K+1] rows, draft: [B][K] rows (may be NULL in FLy mode), both
 * with the same V, stride and dtype.  tokens: [B][K] draft tokens.
 * kept_len: [B] or NULL (= K).  Outputs: accepted_len [B], out_tokens
 * [B][K+1] (-1 after the last emitted token), optional per-row statistics
 * (NaN / -1 for rows that were not evaluated), boundary bits [B], the race
 * gap [B] ((k1 - k2)/k1 of the two largest race keys; NaN when no race ran),
 * and the distances behind the other two near-tie bits, each nullable:
 * accept_gap [B], the smallest |u_j - p/q| over the evaluated accept tests,
 * and gate_gap [B], the smallest |h_j - theta| over the evaluated FLy gates
 * (+inf when there were none).  Returns 0, or -1 on bad arguments. */
int ref_verify(const void *target, const void *draft, const int32_t *tokens,
               const int32_t *kept_len, int32_t B, int32_t K, int64_t V, int64_t stride,
               int32_t dtype, double temperature, uint64_t seed, int32_t mode, double theta,
               int32_t W, int32_t *accepted_len, int32_t *out_tokens, double *t_lse,
               double *t_h, int64_t *t_argmax, double *d_lse, double *d_qmax,
               double *d_feat, uint32_t *boundary, double *race_gap, double *accept_gap,
               double *gate_gap, int nthreads);

/* AV scorer and trimming: c = sigmoid(omega*feat + beta_i), P_i = prod c,
 * keep while P_i >= tau (tau <= 0 keeps everything).  feat: [B][K];
 * omega_beta: [K+1] = (omega, beta_0..beta_{K-1}).  near: [B] (nullable). */
void ref_av_score(const double *feat, int32_t B, int32_t K, const double *omega_beta,
                  double tau, double *conf, uint8_t *mask, int32_t *kept_len, uint32_t *near);

/* Mean log-loss of the scorer over the labelled drafts (NaN when none). */
double ref_av_loss(const double *feat, const int32_t *accepted_len, const int32_t *kept_len,
                   int32_t B, int32_t K, const double *omega_beta, int64_t *n_labels);

/* One SGD step on the mean log-loss; omega_beta updated in place. */
void ref_av_update(const double *feat, const int32_t *accepted_len, const int32_t *kept_len,
                   int32_t B, int32_t K, double lr, double *omega_beta);

/* IRLS refit ([AV] "Ajuste de los Coeficientes").  Accumulate one step's
 * labels into g [K+1], H [(K+1)*(K+1)] (dense, row-major) and cnt [K+1] at
 * the current coefficients; solve at the round's end: H dtheta = -g over the
 * coefficients with labels (Cholesky; a pivot <= 1e-12 x the largest
 * diagonal entry holds omega and solves the intercepts alone), damped by
 * cnt/(cnt + c_damp) per coefficient.  The solve zeroes g, H and cnt.
 * Returns bit 0 = coefficients updated, bit 1 = slope held. */
void ref_irls_accumulate(const double *feat, const int32_t *accepted_len, const int32_t *kept_len,
                         int32_t B, int32_t K, const double *omega_beta, double *g, double *H,
                         int64_t *cnt);
int ref_irls_solve(int32_t K, double c_damp, double *g, double *H, int64_t *cnt,
                   double *omega_beta);

/* Scorer diagnostics over one batch's labels: out = {AUC, mean log-loss,
 * ECE over nbins equal-width bins of s, number of labels}. */
void ref_av_diagnostics(const double *feat, const int32_t *accepted_len, const int32_t *kept_len,
                        int32_t B, int32_t K, const double *omega_beta, int32_t nbins,
                        double *out, int32_t *near);

/* Budgeted trimming: returns the budget (number of kept drafts) and fills
 * kept_len [B] and mask [B*K] (nullable).  conf: float [B][K]; cost: [B*K+1]
 * (cost of verifying a budget of k drafts). */
int64_t ref_av_budget(const float *conf, int32_t B, int32_t K, const double *cost,
                      double n_requests, int32_t *kept_len, uint8_t *mask, double *best_ratio,
                      int32_t *near);

/* Prompt-lookup drafting over contexts ctx [B][stride] of lengths len [B]. */
void ref_ngram_propose(const int32_t *ctx, const int32_t *len, int32_t B, int64_t stride,
                       int32_t n_min, int32_t n_max, int32_t K, int32_t *draft,
                       int32_t *draft_len, int32_t *match_pos, int32_t *match_n);

#ifdef __cplusplus
}
#endif
#endif
