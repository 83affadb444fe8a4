/*
 * specverify_ref.c -- CPU oracle (TEST INFRASTRUCTURE ONLY; see the header).
 *
 * Plain C99, IEEE double, no blocking or fusion beyond what the definitions
 * state.  Each function names the passage it follows:
 *   [AV]  page "Verificacion Adaptativa sin una cabeza de confianza"
 *   [FLy] page "Training-Free Loosely Speculative Decoding: Accepting
 *         Semantically Correct Drafts Beyond Exact Match"
 *   [SD]  page "Speculative Decoding: как черновая модель ускоряет генерацию
 *         LLM без потери качества"
 * Where the pages leave a step open the reading taken is stated at the step.
 */
#include "specverify_ref.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Philox4x32-10, written from Salmon et al., SC'11, section 3 ("Philox"):   */
/* each round multiplies counter words 0 and 2 by two fixed odd constants,   */
/* forms the new words from the high halves xor-ed with the other counter    */
/* words and the round key, and bumps the key by the two Weyl increments     */
/* (golden ratio and sqrt(3)-1 in 32-bit fixed point) between rounds.        */
/* ------------------------------------------------------------------------ */
static const uint32_t PHILOX_M0 = 0xD2511F53u;
static const uint32_t PHILOX_M1 = 0xCD9E8D57u;
static const uint32_t PHILOX_W0 = 0x9E3779B9u;
static const uint32_t PHILOX_W1 = 0xBB67AE85u;

void ref_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
    uint32_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += PHILOX_W0;
            k1 += PHILOX_W1;
        }
        uint64_t p0 = (uint64_t)PHILOX_M0 * (uint64_t)x0;
        uint64_t p1 = (uint64_t)PHILOX_M1 * (uint64_t)x2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t y0 = hi1 ^ x1 ^ k0;
        uint32_t y1 = lo1;
        uint32_t y2 = hi0 ^ x3 ^ k1;
        uint32_t y3 = lo0;
        x0 = y0;
        x1 = y1;
        x2 = y2;
        x3 = y3;
    }
    out[0] = x0;
    out[1] = x1;
    out[2] = x2;
    out[3] = x3;
}

/* Counter layout: one Philox block serves four consecutive vocabulary ids of
 * one (sequence b, position pos, stream tag); the key is the 64-bit seed. */
uint32_t ref_draw_u32(uint64_t seed, uint32_t x, uint32_t pos, uint32_t b, uint32_t tag) {
    uint32_t ctr[4] = {x >> 2, pos, b, tag};
    uint32_t key[2] = {(uint32_t)(seed & 0xffffffffu), (uint32_t)(seed >> 32)};
    uint32_t out[4];
    ref_philox4x32_10(ctr, key, out);
    return out[x & 3u];
}

/* Top 23 bits of the draw, placed on the odd points of the 2^-24 grid so the
 * value is exact in float and double and never 0 or 1. */
double ref_uniform(uint64_t seed, uint32_t x, uint32_t pos, uint32_t b, uint32_t tag) {
    uint32_t r = ref_draw_u32(seed, x, pos, b, tag);
    double k = (double)(r >> 9);
    return (2.0 * k + 1.0) / 16777216.0;
}

/* The race's word for id x: two independent draws give its two halves.  The
 * high half is 16 bits of the screening stream, one Philox block per eight
 * consecutive ids (half x&1 of word (x>>1)&3 of the block at counter
 * (x>>3, pos, b, REF_TAG_SCREEN)); the low half is the high half of the race
 * stream's draw for x.  Independent uniform halves make a uniform word. */
uint32_t ref_race_u32(uint64_t seed, uint32_t x, uint32_t pos, uint32_t b) {
    uint32_t ctr[4] = {x >> 3, pos, b, REF_TAG_SCREEN};
    uint32_t key[2] = {(uint32_t)(seed & 0xffffffffu), (uint32_t)(seed >> 32)};
    uint32_t out[4];
    ref_philox4x32_10(ctr, key, out);
    uint32_t hi = (out[(x >> 1) & 3u] >> (16u * (x & 1u))) & 0xffffu;
    uint32_t lo = ref_draw_u32(seed, x, pos, b, REF_TAG_RACE) >> 16;
    return (hi << 16) | lo;
}

double ref_race_uniform(uint64_t seed, uint32_t x, uint32_t pos, uint32_t b) {
    uint32_t r = ref_race_u32(seed, x, pos, b);
    double k = (double)(r >> 9);
    return (2.0 * k + 1.0) / 16777216.0;
}

/* ------------------------------------------------------------------------ */
/* Inputs                                                                    */
/* ------------------------------------------------------------------------ */
static double load_logit(const void *row, int dtype, int64_t x) {
    if (dtype == 0) return (double)((const float *)row)[x];
    uint32_t bits = (uint32_t)((const uint16_t *)row)[x] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static const void *row_ptr(const void *base, int dtype, int64_t row, int64_t stride) {
    size_t esz = dtype == 0 ? 4 : 2;
    return (const void *)((const char *)base + (size_t)row * (size_t)stride * esz);
}

/* ------------------------------------------------------------------------ */
/* Row statistics.  The normalised target entropy h_j = H(p)/log V is the     */
/* quantity [FLy] section "A. Mecanismo de Verificacao de Dois Niveis" gates   */
/* on; logit(q_max), the log-odds of the draft's most likely token, is the     */
/* feature of [AV] section "Puntuar la Distribucion".  Everything is written   */
/* straight from the definitions of softmax, entropy and log-odds.            */
/* ------------------------------------------------------------------------ */
typedef struct {
    double m, lse, H, h, qmax, feat;
    int64_t argmax;
} row_stat;

static const double FEAT_CLAMP_R = 1.1754943508222875e-38; /* 2^-126 */

static void row_stats_one(const void *row, int dtype, int64_t V, double T, row_stat *st) {
    /* z_x = l_x / T; m = max z, argmax = first id attaining it */
    double m = -INFINITY;
    int64_t am = -1;
    for (int64_t x = 0; x < V; ++x) {
        double z = load_logit(row, dtype, x) / T;
        if (z > m) {
            m = z;
            am = x;
        }
    }
    /* r = sum over the ids other than the argmax of exp(z_x - m); the argmax
     * itself contributes exp(0) = 1, so sum_x exp(z_x - m) = 1 + r exactly.
     * lse = m + log(1 + r), evaluated as m + log1p(r). */
    double r = 0.0;
    for (int64_t x = 0; x < V; ++x)
        if (x != am) r += exp(load_logit(row, dtype, x) / T - m);
    const double l1p = log1p(r);
    double lse = m + l1p;
    /* H = -sum_x p_x log p_x with log p_x = z_x - lse, formed as
     * (z_x - m) - log(1 + r) so that the argmax's log p = -log1p(r) keeps
     * its precision when q_max is close to 1; p_x = 0 adds nothing. */
    double H = 0.0;
    for (int64_t x = 0; x < V; ++x) {
        double lp = (load_logit(row, dtype, x) / T - m) - l1p;
        double p = exp(lp);
        if (p > 0.0) H -= p * lp;
    }
    /* q_max = exp(m - lse) = 1/(1 + r); logit(q_max) = log q_max - log(1 - q_max)
     * = -log r, an exact rewrite that avoids forming 1 - q_max. */
    st->m = m;
    st->lse = lse;
    st->H = H;
    st->h = H / log((double)V);
    st->argmax = am;
    st->qmax = 1.0 / (1.0 + r);
    st->feat = -log(r > FEAT_CLAMP_R ? r : FEAT_CLAMP_R);
}

int ref_row_probs(const void *row, int64_t V, int dtype, double T, double *p) {
    if (!row || !p || V < 1 || !(T > 0.0) || (dtype != 0 && dtype != 1)) return -1;
    row_stat st;
    row_stats_one(row, dtype, V, T, &st);
    for (int64_t x = 0; x < V; ++x) p[x] = exp(load_logit(row, dtype, x) / T - st.lse);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Simple static row/sequence partition over POSIX threads.                   */
/* ------------------------------------------------------------------------ */
typedef void (*range_fn)(void *ctx, int64_t lo, int64_t hi, int tid);
typedef struct {
    range_fn fn;
    void *ctx;
    int64_t lo, hi;
    int tid;
} range_job;

static void *range_thunk(void *arg) {
    range_job *j = (range_job *)arg;
    j->fn(j->ctx, j->lo, j->hi, j->tid);
    return NULL;
}

static void parallel_ranges(range_fn fn, void *ctx, int64_t n, int nthreads) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((int64_t)nthreads > n) nthreads = n > 0 ? (int)n : 1;
    if (nthreads == 1) {
        fn(ctx, 0, n, 0);
        return;
    }
    pthread_t th[256];
    range_job jobs[256];
    for (int t = 0; t < nthreads; ++t) {
        jobs[t].fn = fn;
        jobs[t].ctx = ctx;
        jobs[t].lo = n * t / nthreads;
        jobs[t].hi = n * (t + 1) / nthreads;
        jobs[t].tid = t;
        pthread_create(&th[t], NULL, range_thunk, &jobs[t]);
    }
    for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
}

typedef struct {
    const void *base;
    int64_t V, stride;
    int dtype;
    double T;
    double *m, *lse, *H, *h, *qmax, *feat;
    int64_t *argmax;
} rows_ctx;

static void rows_range(void *vctx, int64_t lo, int64_t hi, int tid) {
    (void)tid;
    rows_ctx *c = (rows_ctx *)vctx;
    for (int64_t r = lo; r < hi; ++r) {
        row_stat st;
        row_stats_one(row_ptr(c->base, c->dtype, r, c->stride), c->dtype, c->V, c->T, &st);
        if (c->m) c->m[r] = st.m;
        if (c->lse) c->lse[r] = st.lse;
        if (c->H) c->H[r] = st.H;
        if (c->h) c->h[r] = st.h;
        if (c->argmax) c->argmax[r] = st.argmax;
        if (c->qmax) c->qmax[r] = st.qmax;
        if (c->feat) c->feat[r] = st.feat;
    }
}

int ref_rows_stats(const void *base, int64_t nrows, int64_t V, int64_t stride, int dtype,
                   double T, double *m, double *lse, double *H, double *h, int64_t *argmax,
                   double *qmax, double *feat, int nthreads) {
    if (nrows < 0 || V < 2 || stride < V || !(T > 0.0) || (dtype != 0 && dtype != 1)) return -1;
    if (nrows > 0 && !base) return -1;
    rows_ctx c = {base, V, stride, dtype, T, m, lse, H, h, qmax, feat, argmax};
    parallel_ranges(rows_range, &c, nrows, nthreads);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Sampling by exponential race: with independent E_x ~ Exp(1), the index    */
/* maximising w_x / E_x is distributed as w / sum(w).  Used for the residual  */
/* resample and for sampling the target's own distribution.                   */
/* ------------------------------------------------------------------------ */
int64_t ref_race(const double *w, int64_t V, uint64_t seed, uint32_t pos, uint32_t b,
                 double *rel_gap) {
    int64_t best = -1;
    double k1 = 0.0, k2 = 0.0;
    for (int64_t x = 0; x < V; ++x) {
        if (!(w[x] > 0.0)) continue;
        double u = ref_race_uniform(seed, (uint32_t)x, pos, b);
        double E = -log(u);
        double key = w[x] / E;
        if (key > k1) {
            k2 = k1;
            k1 = key;
            best = x;
        } else if (key > k2) {
            k2 = key;
        }
    }
    if (rel_gap) *rel_gap = best >= 0 ? (k1 - k2) / k1 : NAN;
    return best;
}

/* Residual of [SD] section "Математика верификации": after a rejection the
 * replacement token comes from norm(max(0, p - q)); the race needs no norm. */
void ref_residual(const double *p, const double *q, int64_t V, double *w) {
    for (int64_t x = 0; x < V; ++x) {
        double d = p[x] - q[x];
        w[x] = d > 0.0 ? d : 0.0;
    }
}

/* ------------------------------------------------------------------------ */
/* [FLy] section "A. Mecanismo de Verificacao de Dois Niveis".               */
/* Scan the draft in order.  A position whose token equals the target's top  */
/* prediction is accepted.  At a deviation the entropy gate decides: a        */
/* confident target (h < theta) rejects it at once; an uncertain one defers   */
/* the decision over the next W positions.  A deferred deviation whose window */
/* would run past the last draft position is rejected (boundary rule); one    */
/* followed by another deviation inside the window is rejected               */
/* retroactively; otherwise it and the W window positions (all matches) are   */
/* accepted and the scan resumes after the window.                            */
/* ------------------------------------------------------------------------ */
int ref_fly_resolve(int L, int W, double theta, const int32_t *dev, const double *h,
                    double *gate_gap) {
    int j = 0;
    if (gate_gap) *gate_gap = INFINITY;
    while (j < L) {
        if (!dev[j]) {
            ++j;
            continue;
        }
        /* distance of this evaluated gate from its threshold */
        if (gate_gap && fabs(h[j] - theta) < *gate_gap) *gate_gap = fabs(h[j] - theta);
        if (h[j] < theta) return j; /* low entropy: treat as a real error */
        if (j + W > L - 1) return j; /* window cannot be filled */
        for (int k = j + 1; k <= j + W; ++k)
            if (dev[k]) return j; /* target diverged again: retroactive */
        j += W + 1;
    }
    return L;
}

/* ------------------------------------------------------------------------ */
/* Full verification.                                                         */
/* Lossless ([SD] sections "Основная идея: черновик и верификация" and        */
/* "Математика верификации"): position by position, accept draft x_j with    */
/* probability min(1, p(x_j)/q(x_j)) -- realised as u_j < p/q with u_j from   */
/* Philox -- and at the first rejection emit a token drawn from               */
/* norm(max(0, p - q)).  When every verified draft is accepted one more token */
/* is drawn from the target's own distribution at the next row: the bonus    */
/* row K, or the trim point L < K under adaptive verification, where the     */
/* target samples its own p ([AV] section "Notas al pie", footnote 1).        */
/* FLy: the resolver above; the replacement / bonus token is the target's    */
/* top prediction at that row.                                                */
/* ------------------------------------------------------------------------ */
typedef struct {
    const void *target, *draft;
    const int32_t *tokens, *kept_len;
    int32_t B, K;
    int64_t V, stride;
    int32_t dtype;
    double T;
    uint64_t seed;
    int32_t mode;
    double theta;
    int32_t W;
    int32_t *accepted_len, *out_tokens;
    double *t_lse, *t_h, *d_lse, *d_qmax, *d_feat, *race_gap, *accept_gap, *gate_gap;
    int64_t *t_argmax;
    uint32_t *boundary;
    double **scratch; /* per thread: 3*V doubles */
} verify_ctx;

static void verify_one(verify_ctx *c, int64_t b, double *p, double *q, double *w) {
    const int32_t K = c->K;
    const int64_t V = c->V;
    int32_t L = c->kept_len ? c->kept_len[b] : K;
    const int32_t *tok = c->tokens + b * K;
    uint32_t near = 0;
    row_stat ts[K + 1], ds[K > 0 ? K : 1];
    const void *trow[K + 1];
    const void *drow[K > 0 ? K : 1];
    for (int32_t j = 0; j <= K; ++j) {
        trow[j] = row_ptr(c->target, c->dtype, b * (K + 1) + j, c->stride);
        ts[j].lse = ts[j].h = NAN;
        ts[j].argmax = -1;
        if (j <= L) row_stats_one(trow[j], c->dtype, V, c->T, &ts[j]);
    }
    for (int32_t j = 0; j < K; ++j) {
        drow[j] = NULL;
        ds[j].lse = ds[j].qmax = ds[j].feat = NAN;
        if (c->mode == REF_MODE_LOSSLESS && j < L) {
            drow[j] = row_ptr(c->draft, c->dtype, b * K + j, c->stride);
            row_stats_one(drow[j], c->dtype, V, c->T, &ds[j]);
        }
    }

    int32_t jstar = L;
    int64_t y = -1;
    double gap = NAN;
    double agap = INFINITY, ggap = INFINITY; /* nearest evaluated accept test / gate */
    if (c->mode == REF_MODE_LOSSLESS) {
        for (int32_t j = 0; j < L; ++j) {
            int32_t x = tok[j];
            double logp = -INFINITY, logq = -INFINITY;
            if (x >= 0 && x < V) {
                logp = load_logit(trow[j], c->dtype, x) / c->T - ts[j].lse;
                logq = load_logit(drow[j], c->dtype, x) / c->T - ds[j].lse;
            }
            double ratio = exp(logp - logq); /* p(x_j)/q(x_j); NaN for a token outside V */
            double u = ref_uniform(c->seed, 0u, (uint32_t)j, (uint32_t)b, REF_TAG_ACCEPT);
            if (fabs(u - ratio) < agap) agap = fabs(u - ratio); /* NaN ratio: skipped */
            if (fabs(u - ratio) < 1e-5) near |= REF_NEAR_ACCEPT;
            if (!(u < ratio)) {
                jstar = j;
                break;
            }
        }
        if (jstar < L) {
            for (int64_t x = 0; x < V; ++x) {
                p[x] = exp(load_logit(trow[jstar], c->dtype, x) / c->T - ts[jstar].lse);
                q[x] = exp(load_logit(drow[jstar], c->dtype, x) / c->T - ds[jstar].lse);
            }
            ref_residual(p, q, V, w);
            y = ref_race(w, V, c->seed, (uint32_t)jstar, (uint32_t)b, &gap);
            if (y < 0) { /* cannot happen in exact arithmetic after a rejection */
                near |= REF_RESIDUAL_EMPTY;
                y = ref_race(p, V, c->seed, (uint32_t)jstar, (uint32_t)b, &gap);
            }
        } else {
            for (int64_t x = 0; x < V; ++x)
                p[x] = exp(load_logit(trow[L], c->dtype, x) / c->T - ts[L].lse);
            y = ref_race(p, V, c->seed, (uint32_t)L, (uint32_t)b, &gap);
        }
        if (!(gap > 1e-6)) near |= REF_NEAR_RACE;
    } else {
        int32_t dev[K > 0 ? K : 1];
        double hh[K > 0 ? K : 1];
        for (int32_t j = 0; j < L; ++j) {
            dev[j] = tok[j] != ts[j].argmax;
            hh[j] = ts[j].h;
        }
        jstar = ref_fly_resolve(L, c->W, c->theta, dev, hh, &ggap);
        if (ggap < 1e-5) near |= REF_NEAR_GATE;
        y = ts[jstar].argmax;
    }

    c->accepted_len[b] = jstar;
    int32_t *ot = c->out_tokens + b * (K + 1);
    for (int32_t j = 0; j <= K; ++j) ot[j] = -1;
    for (int32_t j = 0; j < jstar; ++j) ot[j] = tok[j];
    ot[jstar] = (int32_t)y;
    for (int32_t j = 0; j <= K; ++j) {
        int64_t r = b * (K + 1) + j;
        if (c->t_lse) c->t_lse[r] = ts[j].lse;
        if (c->t_h) c->t_h[r] = ts[j].h;
        if (c->t_argmax) c->t_argmax[r] = ts[j].argmax;
    }
    for (int32_t j = 0; j < K; ++j) {
        int64_t r = b * K + j;
        if (c->d_lse) c->d_lse[r] = ds[j].lse;
        if (c->d_qmax) c->d_qmax[r] = ds[j].qmax;
        if (c->d_feat) c->d_feat[r] = ds[j].feat;
    }
    if (c->boundary) c->boundary[b] = near;
    if (c->race_gap) c->race_gap[b] = gap;
    if (c->accept_gap) c->accept_gap[b] = agap;
    if (c->gate_gap) c->gate_gap[b] = ggap;
}

static void verify_range(void *vctx, int64_t lo, int64_t hi, int tid) {
    verify_ctx *c = (verify_ctx *)vctx;
    double *buf = c->scratch[tid];
    for (int64_t b = lo; b < hi; ++b) verify_one(c, b, buf, buf + c->V, buf + 2 * c->V);
}

int ref_verify(const void *target, const void *draft, const int32_t *tokens,
               const int32_t *kept_len, int32_t B, int32_t K, int64_t V, int64_t stride,
               int32_t dtype, double temperature, uint64_t seed, int32_t mode, double theta,
               int32_t W, int32_t *accepted_len, int32_t *out_tokens, double *t_lse,
               double *t_h, int64_t *t_argmax, double *d_lse, double *d_qmax, double *d_feat,
               uint32_t *boundary, double *race_gap, double *accept_gap, double *gate_gap,
               int nthreads) {
    if (B < 0 || K < 1 || V < 2 || stride < V || !(temperature > 0.0)) return -1;
    if (dtype != 0 && dtype != 1) return -1;
    if (mode != REF_MODE_LOSSLESS && mode != REF_MODE_FLY) return -1;
    if (mode == REF_MODE_FLY && (W < 0 || isnan(theta))) return -1;
    if (B == 0) return 0;
    if (!target || !tokens || !accepted_len || !out_tokens) return -1;
    if (mode == REF_MODE_LOSSLESS && !draft) return -1;
    if (kept_len)
        for (int32_t b = 0; b < B; ++b)
            if (kept_len[b] < 0 || kept_len[b] > K) return -1;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > B) nthreads = B;
    if (nthreads > 256) nthreads = 256;
    double *scratch[256];
    for (int t = 0; t < nthreads; ++t) {
        scratch[t] = (double *)malloc(sizeof(double) * 3 * (size_t)V);
        if (!scratch[t]) {
            for (int u = 0; u < t; ++u) free(scratch[u]);
            return -1;
        }
    }
    verify_ctx c = {target, draft, tokens, kept_len, B, K, V, stride, dtype, temperature,
                    seed, mode, theta, W, accepted_len, out_tokens, t_lse, t_h, d_lse,
                    d_qmax, d_feat, race_gap, accept_gap, gate_gap, t_argmax, boundary,
                    scratch};
    parallel_ranges(verify_range, &c, B, nthreads);
    for (int t = 0; t < nthreads; ++t) free(scratch[t]);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Adaptive verification scorer, [AV] sections "Solucion: Estimador de        */
/* aceptacion ajustado en linea" and "Puntuar la Distribucion": one logistic  */
/* regression with a slope omega shared by all draft positions and one        */
/* intercept beta_i per position (K+1 parameters), on the single feature      */
/* logit(q_max).  Survival is the running product of the per-position        */
/* confidences ([AV] section "Otras Caracteristicas Consideradas", the        */
/* cumprod over positions); a position is kept while that product stays at    */
/* or above the threshold tau, so the kept set is a prefix.                   */
/* ------------------------------------------------------------------------ */
static double sigmoid(double a) { return 1.0 / (1.0 + exp(-a)); }

/* log(1 + e^a) without overflow or cancellation; -log sigmoid(a) = softplus(-a)
 * and -log(1 - sigmoid(a)) = softplus(a). */
static double softplus(double a) { return a > 0.0 ? a + log1p(exp(-a)) : log1p(exp(a)); }

void ref_av_score(const double *feat, int32_t B, int32_t K, const double *omega_beta,
                  double tau, double *conf, uint8_t *mask, int32_t *kept_len, uint32_t *near) {
    const double omega = omega_beta[0];
    for (int32_t b = 0; b < B; ++b) {
        double P = 1.0;
        int32_t L = 0;
        int open = 1;
        uint32_t nb = 0;
        for (int32_t i = 0; i < K; ++i) {
            double c = sigmoid(omega * feat[b * K + i] + omega_beta[1 + i]);
            conf[b * K + i] = c;
            P *= c;
            if (tau > 0.0 && fabs(P - tau) <= 1e-5 * tau) nb |= REF_NEAR_TRIM;
            int keep = open && (tau <= 0.0 || P >= tau);
            mask[b * K + i] = (uint8_t)keep;
            if (keep)
                ++L;
            else
                open = 0;
        }
        kept_len[b] = L;
        if (near) near[b] = nb;
    }
}

/* [AV] section "Ajuste de los Coeficientes": only drafts up to and including
 * the first rejection carry a label (accepted = 1, the first rejected = 0);
 * drafts that were trimmed or came after the rejection carry none. */
static int32_t n_labels_of(const int32_t *accepted_len, const int32_t *kept_len, int32_t K,
                           int32_t b) {
    int32_t L = kept_len ? kept_len[b] : K;
    int32_t a = accepted_len[b];
    return a + 1 < L ? a + 1 : L;
}

double ref_av_loss(const double *feat, const int32_t *accepted_len, const int32_t *kept_len,
                   int32_t B, int32_t K, const double *omega_beta, int64_t *n_labels) {
    double sum = 0.0;
    int64_t N = 0;
    for (int32_t b = 0; b < B; ++b) {
        int32_t n = n_labels_of(accepted_len, kept_len, K, b);
        for (int32_t i = 0; i < n; ++i) {
            double a = omega_beta[0] * feat[b * K + i] + omega_beta[1 + i];
            sum += i < accepted_len[b] ? softplus(-a) : softplus(a);
            ++N;
        }
    }
    if (n_labels) *n_labels = N;
    return N > 0 ? sum / (double)N : NAN;
}

/* The pages refit by Newton steps over rounds; the scope here is one plain
 * gradient step per call on the mean log-loss of the call's labels, all
 * parameters updated together from their pre-step values. */
void ref_av_update(const double *feat, const int32_t *accepted_len, const int32_t *kept_len,
                   int32_t B, int32_t K, double lr, double *omega_beta) {
    double g_omega = 0.0;
    double *g_beta = (double *)calloc((size_t)(K > 0 ? K : 1), sizeof(double));
    int64_t N = 0;
    for (int32_t b = 0; b < B; ++b) {
        int32_t n = n_labels_of(accepted_len, kept_len, K, b);
        for (int32_t i = 0; i < n; ++i) {
            double y = i < accepted_len[b] ? 1.0 : 0.0;
            double f = feat[b * K + i];
            double s = sigmoid(omega_beta[0] * f + omega_beta[1 + i]);
            g_omega += (s - y) * f;
            g_beta[i] += s - y;
            ++N;
        }
    }
    if (N > 0) {
        omega_beta[0] -= lr * g_omega / (double)N;
        for (int32_t i = 0; i < K; ++i) omega_beta[1 + i] -= lr * g_beta[i] / (double)N;
    }
    free(g_beta);
}

/* ------------------------------------------------------------------------
 * Newton (IRLS) refit of the scorer over rounds ([AV] "Ajuste de los
 * Coeficientes").  Per step the labelled drafts of the batch add to the
 * gradient g and Hessian H of the summed log-loss at the current
 * coefficients theta = (omega, beta_0..beta_{K-1}); x_n = (f_n, e_{i_n}):
 *   g += (s_n - y_n) x_n,   H += s_n (1 - s_n) x_n x_n^T,
 * and cnt counts the labels behind each coefficient (all labels for omega,
 * the labels at position i for beta_i).  At the round's end the system
 * H dtheta = -g is solved and each coefficient moves by dtheta_k scaled by
 * cnt_k / (cnt_k + c_damp).
 * ------------------------------------------------------------------------ */
void ref_irls_accumulate(const double *feat, const int32_t *accepted_len, const int32_t *kept_len,
                         int32_t B, int32_t K, const double *omega_beta, double *g, double *H,
                         int64_t *cnt) {
    const int32_t D = K + 1;
    for (int32_t b = 0; b < B; ++b) {
        int32_t n = n_labels_of(accepted_len, kept_len, K, b);
        for (int32_t i = 0; i < n; ++i) {
            double y = i < accepted_len[b] ? 1.0 : 0.0;
            double f = feat[b * K + i];
            double s = sigmoid(omega_beta[0] * f + omega_beta[1 + i]);
            double x[2] = {f, 1.0};
            int32_t idx[2] = {0, 1 + i};
            for (int r = 0; r < 2; ++r) {
                g[idx[r]] += (s - y) * x[r];
                for (int q = 0; q < 2; ++q) H[idx[r] * D + idx[q]] += s * (1.0 - s) * x[r] * x[q];
            }
            cnt[0] += 1;
            cnt[1 + i] += 1;
        }
    }
}

/* Cholesky solve of the n x n system A x = rhs (A symmetric, row-major, the
 * lower triangle is overwritten).  Returns -1 when a pivot is at most
 * tol (the system is treated as singular). */
static int chol_solve(double *A, int n, double *rhs, double tol) {
    for (int j = 0; j < n; ++j) {
        double d = A[j * n + j];
        for (int k = 0; k < j; ++k) d -= A[j * n + k] * A[j * n + k];
        if (!(d > tol)) return -1;
        double l = sqrt(d);
        A[j * n + j] = l;
        for (int i = j + 1; i < n; ++i) {
            double v = A[i * n + j];
            for (int k = 0; k < j; ++k) v -= A[i * n + k] * A[j * n + k];
            A[i * n + j] = v / l;
        }
    }
    for (int i = 0; i < n; ++i) { /* L y = rhs */
        double v = rhs[i];
        for (int k = 0; k < i; ++k) v -= A[i * n + k] * rhs[k];
        rhs[i] = v / A[i * n + i];
    }
    for (int i = n - 1; i >= 0; --i) { /* L^T x = y */
        double v = rhs[i];
        for (int k = i + 1; k < n; ++k) v -= A[k * n + i] * rhs[k];
        rhs[i] = v / A[i * n + i];
    }
    return 0;
}

int ref_irls_solve(int32_t K, double c_damp, double *g, double *H, int64_t *cnt,
                   double *omega_beta) {
    const int32_t D = K + 1;
    int flags = 0;
    if (cnt[0] > 0) {
        /* coefficients with evidence; the system over the others is empty */
        int act[65], na = 0;
        double hmax = 0.0;
        for (int32_t k = 0; k < D; ++k)
            if (cnt[k] > 0 && H[k * D + k] > 0.0) {
                act[na++] = k;
                if (H[k * D + k] > hmax) hmax = H[k * D + k];
            }
        double A[65 * 65], x[65];
        int ok = -1;
        if (na > 0 && act[0] == 0) {
            for (int r = 0; r < na; ++r) {
                x[r] = -g[act[r]];
                for (int q = 0; q < na; ++q) A[r * na + q] = H[act[r] * D + act[q]];
            }
            ok = chol_solve(A, na, x, 1e-12 * hmax);
        }
        if (ok != 0) {
            /* no curvature left for the slope (e.g. every feature equal):
             * hold omega and give each intercept its own Newton step */
            flags |= 2;
            int nb = 0;
            for (int r = 0; r < na; ++r)
                if (act[r] != 0) act[nb++] = act[r];
            na = nb;
            for (int r = 0; r < na; ++r) x[r] = -g[act[r]] / H[act[r] * D + act[r]];
        }
        for (int r = 0; r < na; ++r) {
            int k = act[r];
            double n = (double)cnt[k];
            omega_beta[k] += x[r] * (n / (n + c_damp));
        }
        flags |= 1;
    }
    for (int32_t k = 0; k < D; ++k) {
        g[k] = 0.0;
        cnt[k] = 0;
        for (int32_t q = 0; q < D; ++q) H[k * D + q] = 0.0;
    }
    return flags;
}

/* ------------------------------------------------------------------------
 * Estimator diagnostics over one batch's labels ([AV] "Otras
 * Caracteristicas Consideradas", the AUC / log-loss / ECE axes).  With
 * z_n = omega f_n + beta_{i_n} and s_n = sigmoid(z_n):
 *   AUC     = P(z of a random accepted draft > z of a random rejected one),
 *             ties counting one half (NaN without both classes);
 *   logloss = mean of -log s_n (accepted) and -log(1 - s_n) (rejected);
 *   ECE     = sum over nbins equal-width bins of s of
 *             (n_bin / N) |mean s - mean y| over the bin.
 * out = {auc, logloss, ece, N}.  near (nullable): 1 when some s_n lies
 * within 1e-9 of a bin edge.
 * ------------------------------------------------------------------------ */
void ref_av_diagnostics(const double *feat, const int32_t *accepted_len, const int32_t *kept_len,
                        int32_t B, int32_t K, const double *omega_beta, int32_t nbins,
                        double *out, int32_t *near) {
    int64_t N = 0;
    for (int32_t b = 0; b < B; ++b) N += n_labels_of(accepted_len, kept_len, K, b);
    double *z = (double *)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
    int8_t *y = (int8_t *)malloc((size_t)(N > 0 ? N : 1));
    int64_t t = 0;
    for (int32_t b = 0; b < B; ++b) {
        int32_t n = n_labels_of(accepted_len, kept_len, K, b);
        for (int32_t i = 0; i < n; ++i) {
            z[t] = omega_beta[0] * feat[b * K + i] + omega_beta[1 + i];
            y[t] = (int8_t)(i < accepted_len[b]);
            ++t;
        }
    }
    /* AUC by counting every (accepted, rejected) pair */
    double pairs_won = 0.0;
    int64_t npos = 0, nneg = 0;
    for (int64_t a = 0; a < N; ++a) {
        if (y[a]) ++npos; else ++nneg;
    }
    for (int64_t a = 0; a < N; ++a) {
        if (!y[a]) continue;
        for (int64_t r = 0; r < N; ++r) {
            if (y[r]) continue;
            if (z[a] > z[r]) pairs_won += 1.0;
            else if (z[a] == z[r]) pairs_won += 0.5;
        }
    }
    double auc = (npos > 0 && nneg > 0) ? pairs_won / ((double)npos * (double)nneg) : NAN;
    double loss = 0.0;
    double *bs = (double *)calloc((size_t)(nbins > 0 ? nbins : 1), sizeof(double));
    int nearb = 0;
    for (int64_t a = 0; a < N; ++a) {
        loss += y[a] ? softplus(-z[a]) : softplus(z[a]);
        double s = sigmoid(z[a]);
        double sm = s * nbins;
        int bin = (int)floor(sm);
        if (bin > nbins - 1) bin = nbins - 1;
        if (bin < 0) bin = 0;
        if (fabs(sm - floor(sm + 0.5)) < 1e-9 * nbins) nearb = 1;
        bs[bin] += s - (double)y[a];
    }
    double ece = 0.0;
    for (int q = 0; q < nbins; ++q) ece += fabs(bs[q]);
    out[0] = auc;
    out[1] = N > 0 ? loss / (double)N : NAN;
    out[2] = N > 0 ? ece / (double)N : NAN;
    out[3] = (double)N;
    if (near) *near = nearb;
    free(z);
    free(y);
    free(bs);
}

/* ------------------------------------------------------------------------
 * Budgeted trimming ([AV] "Otras Caracteristicas Consideradas", the
 * survival / top-k and budget snippets).  Survival of draft (b, i) is the
 * running product of the confidences along the sequence, formed in float
 * as the device forms it.  With the B*K survivals sorted in decreasing order
 * (ties: lower flat index b*K+i first), the expected emitted tokens for a
 * budget of k drafts are n_requests + (sum of the first k survivals), and
 * the budget is the k in 0..B*K maximising that over cost[k] (the first
 * maximum).  The kept drafts are the first `budget` in that order; since
 * survival never grows along a sequence they form a prefix of each.
 * Returns the budget; near (nullable) is 1 when the best two ratios are
 * within 1e-12 relative.
 * ------------------------------------------------------------------------ */
static const float *g_sort_keys;
static int cmp_survival(const void *pa, const void *pb) {
    int64_t a = *(const int64_t *)pa, b = *(const int64_t *)pb;
    float sa = g_sort_keys[a], sb = g_sort_keys[b];
    if (sa > sb) return -1;
    if (sa < sb) return 1;
    return a < b ? -1 : (a > b ? 1 : 0);
}

int64_t ref_av_budget(const float *conf, int32_t B, int32_t K, const double *cost,
                      double n_requests, int32_t *kept_len, uint8_t *mask, double *best_ratio,
                      int32_t *near) {
    const int64_t M = (int64_t)B * K;
    float *surv = (float *)malloc((size_t)(M > 0 ? M : 1) * sizeof(float));
    int64_t *ord = (int64_t *)malloc((size_t)(M > 0 ? M : 1) * sizeof(int64_t));
    for (int32_t b = 0; b < B; ++b) {
        float P = 1.0f;
        for (int32_t i = 0; i < K; ++i) {
            P = P * conf[(int64_t)b * K + i];
            surv[(int64_t)b * K + i] = P;
        }
    }
    for (int64_t t = 0; t < M; ++t) ord[t] = t;
    g_sort_keys = surv;
    qsort(ord, (size_t)M, sizeof(int64_t), cmp_survival);
    double est = n_requests, best = est / cost[0], second = -INFINITY;
    int64_t budget = 0;
    for (int64_t k = 1; k <= M; ++k) {
        est += (double)surv[ord[k - 1]];
        double r = est / cost[k];
        if (r > best) {
            second = best;
            best = r;
            budget = k;
        } else if (r > second) {
            second = r;
        }
    }
    for (int32_t b = 0; b < B; ++b) kept_len[b] = 0;
    if (mask) memset(mask, 0, (size_t)M);
    for (int64_t t = 0; t < budget; ++t) {
        int64_t f = ord[t];
        kept_len[f / K] += 1;
        if (mask) mask[f] = 1;
    }
    if (best_ratio) *best_ratio = best;
    if (near) *near = (second > -INFINITY && best - second <= 1e-12 * fabs(best)) ? 1 : 0;
    free(surv);
    free(ord);
    return budget;
}

/* ------------------------------------------------------------------------
 * Prompt-lookup drafting ([SD] "N-gram (prompt lookup)"; [FLy] "B.
 * Aceleracao Multinivel"): for each sequence, the longest suffix n-gram
 * (n from n_max down to n_min) that also occurs earlier in the context; of
 * its earlier occurrences the latest (closest to the end) is taken, and the
 * up to K tokens that followed it are the draft.  ctx: [B][stride] tokens,
 * len: [B] context lengths.  draft: [B][K] (-1 after draft_len), draft_len
 * [B], match_pos [B] (start of the matched occurrence, -1 when none), match_n
 * [B] (its length, 0 when none).
 * ------------------------------------------------------------------------ */
void ref_ngram_propose(const int32_t *ctx, const int32_t *len, int32_t B, int64_t stride,
                       int32_t n_min, int32_t n_max, int32_t K, int32_t *draft,
                       int32_t *draft_len, int32_t *match_pos, int32_t *match_n) {
    for (int32_t b = 0; b < B; ++b) {
        const int32_t *c = ctx + (int64_t)b * stride;
        const int32_t n = len[b];
        int32_t pos = -1, gfound = 0;
        for (int32_t g = n_max; g >= n_min && pos < 0; --g) {
            if (g < 1 || g >= n) continue;
            for (int32_t p = n - g - 1; p >= 0; --p) {
                int32_t same = 1;
                for (int32_t q = 0; q < g; ++q)
                    if (c[p + q] != c[n - g + q]) {
                        same = 0;
                        break;
                    }
                if (same) {
                    pos = p;
                    gfound = g;
                    break;
                }
            }
        }
        int32_t dl = 0;
        if (pos >= 0) {
            dl = n - (pos + gfound);
            if (dl > K) dl = K;
        }
        for (int32_t k = 0; k < K; ++k) draft[(int64_t)b * K + k] = k < dl ? c[pos + gfound + k] : -1;
        draft_len[b] = dl;
        if (match_pos) match_pos[b] = pos;
        if (match_n) match_n[b] = gfound;
    }
}
