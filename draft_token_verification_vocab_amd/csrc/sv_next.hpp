// sv_next.hpp -- the estimator's Newton refit, its diagnostics, budgeted
// trimming and prompt-lookup drafting.
//
// Newton refit (page "Verificacion Adaptativa sin una cabeza de confianza",
// section "Ajuste de los Coeficientes"): each decoding step adds its labelled
// drafts to the gradient g and Hessian H of the summed log-loss at the current
// coefficients; at the end of a round the system H dtheta = -g is solved and
// each coefficient moves by dtheta scaled by n / (n + c), n being the labels
// behind it.  With one shared slope and one intercept per position a label
// touches (omega, beta_i) only, so H is an arrow: H[0][0], H[0][1+i] and the
// diagonal H[1+i][1+i].  The state keeps exactly those, O(K) doubles, and the
// solve eliminates the intercepts first (a Schur complement on the slope).
//
// Diagnostics (same page, section "Otras Caracteristicas Consideradas"):
// AUC counted over every (accepted, rejected) pair, ties one half; mean
// log-loss; ECE over equal-width bins of the predicted probability.
//
// Budgeted trimming (same section, the survival / top-k and budget
// snippets): survival = running product of the confidences along each
// sequence; the B*K survivals are sorted (decreasing, ties by flat index), the
// expected emitted tokens for a budget of k drafts are the number of requests
// plus the sum of the first k, and the budget is the first k maximising that
// over the caller's cost table.  The first `budget` drafts in that order are
// kept; they form a prefix of every sequence.
//
// Prompt lookup (page "Speculative Decoding: как черновая модель ускоряет
// генерацию LLM без потери качества", section "N-gram (prompt lookup)"; page
// "Training-Free Loosely Speculative Decoding...", section "B. Aceleracao
// Multinivel"): the longest suffix n-gram of the context that also occurs
// earlier, its latest earlier occurrence, and the up to K tokens after it.
#pragma once

#include "sv_av.hpp"
#include "sv_common.hpp"

namespace sv {

// Loads per lane per round in the diagnostics finish kernel: issued together
// (unconditionally, at clamped indices), so that a lane waits once per batch
// rather than once per element.
constexpr int kFinishBatch = 8;

// --------------------------------------------------------------------------
// Per-position sums over one batch's labels.  The labels of sequence b are its
// drafts i < min(a_b + 1, L_b): y = 1 for i < a_b (accepted), y = 0 at the
// first rejection.  For position i, with s = sigmoid(omega f + beta_i) and
// d = s - y, w = s (1 - s):
//   n = #labels, r = sum d, rf = sum d f, w, wf = sum w f, wff = sum w f^2.
// One wave per position (positions strided over the workgroup's waves), lanes
// strided over sequences, fixed-order DPP sums: deterministic.
// --------------------------------------------------------------------------
struct LabelSums {
    double n, r, rf, w, wf, wff;
};

// Accepted lengths as the label sums read them: acc(b) for sequence b, from an
// array here; the launch that also picks each step's tokens reads them from
// the race's candidates instead.
struct AcceptedArray {
    const int32_t *p;
    __device__ int operator()(int b) const { return p[b]; }
};

template <int NT, bool CURV, class ACC>
__device__ void label_sums(const float *feat, ACC acc, const int32_t *kept_len, int B, int K,
                           const float *omega_beta, LabelSums *out) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    const double omega = static_cast<double>(omega_beta[0]);
    for (int i = wv; i < K; i += NT / kWave) {
        const double beta = static_cast<double>(omega_beta[1 + i]);
        double n = 0.0, r = 0.0, rf = 0.0, w = 0.0, wf = 0.0, wff = 0.0;
        constexpr int U = 4;  // sequences per lane per pass: their loads go out together
        for (int b0 = lane; b0 < B; b0 += U * kWave) {
            int La[U], aa[U];
            float fa[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int b = b0 + u * kWave;
                const int bc = b < B ? b : B - 1;  // in range; masked out below
                La[u] = kept_len ? kept_len[bc] : K;
                aa[u] = acc(bc);
                fa[u] = feat[static_cast<int64_t>(bc) * K + i];
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int L = clamp_len(La[u], K);
                const int a = clamp_len(aa[u], K);
                const int nl = a + 1 < L ? a + 1 : L;
                if (b0 + u * kWave < B && i < nl) {
                    const double f = static_cast<double>(fa[u]);
                    const double s = 1.0 / (1.0 + exp(-(omega * f + beta)));
                    const double d = s - (i < a ? 1.0 : 0.0);
                    n += 1.0;
                    r += d;
                    rf += d * f;
                    if (CURV) {
                        const double ww = s * (1.0 - s);
                        w += ww;
                        wf += ww * f;
                        wff += ww * f * f;
                    }
                }
            }
        }
        n = wave_sum_f64(n);
        r = wave_sum_f64(r);
        rf = wave_sum_f64(rf);
        if (CURV) {
            w = wave_sum_f64(w);
            wf = wave_sum_f64(wf);
            wff = wave_sum_f64(wff);
        }
        if (lane == 0) out[i] = LabelSums{n, r, rf, w, wf, wff};
    }
    __syncthreads();
}

// One SGD step on the mean log-loss of the batch's labels (the update the
// adaptive-verification workloads run every step), by the whole workgroup.
template <int NT, class ACC>
__device__ __forceinline__ void sgd_step(const float *feat, ACC acc, const int32_t *kept_len, int B,
                                         int K, float lr, float *omega_beta) {
    __shared__ LabelSums sums[64];
    label_sums<NT, false>(feat, acc, kept_len, B, K, omega_beta, sums);
    __shared__ double s_n, s_go;
    if (threadIdx.x == 0) {
        double n = 0.0, go = 0.0;
        for (int i = 0; i < K; ++i) {
            n += sums[i].n;
            go += sums[i].rf;
        }
        s_n = n;
        s_go = go;
    }
    __syncthreads();
    if (s_n > 0.0) {
        const double l = static_cast<double>(lr) / s_n;
        // every thread has read omega_beta (inside label_sums) before the barrier
        if (threadIdx.x == 0)
            omega_beta[0] = static_cast<float>(static_cast<double>(omega_beta[0]) - l * s_go);
        const int t = threadIdx.x;
        if (t < K)
            omega_beta[1 + t] =
                static_cast<float>(static_cast<double>(omega_beta[1 + t]) - l * sums[t].r);
    }
}

template <int NT>
__global__ __launch_bounds__(NT) void av_sgd_kernel(const float *feat, const int32_t *accepted_len,
                                                   const int32_t *kept_len, int B, int K, float lr,
                                                   float *omega_beta) {
    sgd_step<NT>(feat, AcceptedArray{accepted_len}, kept_len, B, K, lr, omega_beta);
}

// A step with nothing trimmed, scored after its verification: the
// confidences of every draft at the coefficients before the update (as
// av_score_kernel with tau <= 0: every draft kept), then the SGD step, in one
// launch.  The scores read omega_beta before sgd_step's first barrier, and
// sgd_step writes it only after that barrier.
template <int NT>
__device__ __forceinline__ void score_untrimmed(const float *feat, int B, int K,
                                                const float *omega_beta, float *conf,
                                                uint8_t *keep_mask, int32_t *kept_len) {
    const double omega = static_cast<double>(omega_beta[0]);
    const int n = B * K;
    for (int f = threadIdx.x; f < n; f += NT) {
        const int i = f - (f / K) * K;
        if (conf) conf[f] = static_cast<float>(av_confidence(omega, feat[f], omega_beta[1 + i]));
        if (keep_mask) keep_mask[f] = 1;
    }
    if (kept_len)
        for (int b = threadIdx.x; b < B; b += NT) kept_len[b] = K;
}

template <int NT>
__global__ __launch_bounds__(NT) void av_score_update_kernel(const float *feat,
                                                            const int32_t *accepted_len, int B,
                                                            int K, float lr, float *omega_beta,
                                                            float *conf, uint8_t *keep_mask,
                                                            int32_t *kept_len) {
    score_untrimmed<NT>(feat, B, K, omega_beta, conf, keep_mask, kept_len);
    sgd_step<NT>(feat, AcceptedArray{accepted_len}, nullptr, B, K, lr, omega_beta);
}

// --------------------------------------------------------------------------
// Newton refit state, doubles: g[K+1] | h00 | h0[K] | hd[K] | cnt[K+1].
// --------------------------------------------------------------------------
__host__ __device__ inline int irls_state_doubles(int K) { return 4 * K + 3; }

struct IrlsView {
    double *g, *h00, *h0, *hd, *cnt;
};
__device__ inline IrlsView irls_view(double *st, int K) {
    return IrlsView{st, st + (K + 1), st + (K + 2), st + (2 * K + 2), st + (3 * K + 2)};
}

__global__ void fill_f64_kernel(double *p, int n, double v) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

template <int NT>
__global__ __launch_bounds__(NT) void irls_accumulate_kernel(const float *feat,
                                                            const int32_t *accepted_len,
                                                            const int32_t *kept_len, int B, int K,
                                                            const float *omega_beta, double *state) {
    __shared__ LabelSums sums[64];
    label_sums<NT, true>(feat, AcceptedArray{accepted_len}, kept_len, B, K, omega_beta, sums);
    const IrlsView v = irls_view(state, K);
    const int t = threadIdx.x;
    if (t == 0) {
        double n = 0.0, go = 0.0, a = 0.0;
        for (int i = 0; i < K; ++i) {
            n += sums[i].n;
            go += sums[i].rf;
            a += sums[i].wff;
        }
        v.g[0] += go;
        v.h00[0] += a;
        v.cnt[0] += n;
    }
    if (t < K) {
        v.g[1 + t] += sums[t].r;
        v.h0[t] += sums[t].wf;
        v.hd[t] += sums[t].w;
        v.cnt[1 + t] += sums[t].n;
    }
}

// Solve at the round's end (one wave).  Coefficients without labels (or
// without curvature) stay out of the system.  The intercepts are eliminated
// first: S = h00 - sum h0_i^2 / hd_i is the slope's own curvature; when
// S <= 1e-12 x the largest diagonal entry the slope is held and every
// intercept takes its own Newton step.  flags: bit 0 = updated, bit 1 =
// slope held.  The state is zeroed for the next round.
__global__ __launch_bounds__(kWave) void irls_solve_kernel(double *state, int K, double c_damp,
                                                           float *omega_beta, int32_t *flags) {
    const IrlsView v = irls_view(state, K);
    const int lane = threadIdx.x;
    __shared__ double s_dw;
    __shared__ int s_flags;
    const bool has = lane < K && v.cnt[1 + lane] > 0.0 && v.hd[lane] > 0.0;
    const double hd = has ? v.hd[lane] : 1.0;
    const double h0 = has ? v.h0[lane] : 0.0;
    const double gi = has ? v.g[1 + lane] : 0.0;
    const double dmax = wave_max_f64_nonneg(has ? hd : 0.0);
    const double sb = wave_sum_f64(has ? h0 * h0 / hd : 0.0);
    const double sg = wave_sum_f64(has ? h0 * gi / hd : 0.0);
    if (lane == 0) {
        int fl = 0;
        double dw = 0.0;
        if (v.cnt[0] > 0.0) {
            fl = 1;
            const double h00 = v.h00[0];
            const double hmax = h00 > dmax ? h00 : dmax;
            const double S = h00 - sb;
            if (h00 > 0.0 && S > 1e-12 * hmax) {
                dw = (-v.g[0] + sg) / S;
                omega_beta[0] = static_cast<float>(static_cast<double>(omega_beta[0]) +
                                                   dw * (v.cnt[0] / (v.cnt[0] + c_damp)));
            } else {
                fl |= 2;
            }
        }
        s_dw = dw;
        s_flags = fl;
    }
    __syncthreads();
    if ((s_flags & 1) && has) {
        const double db = (-gi - h0 * s_dw) / hd;
        const double n = v.cnt[1 + lane];
        omega_beta[1 + lane] =
            static_cast<float>(static_cast<double>(omega_beta[1 + lane]) + db * (n / (n + c_damp)));
    }
    if (lane == 0 && flags) *flags = s_flags;
    __syncthreads();  // every lane has read the state before it is cleared
    for (int k = lane; k < irls_state_doubles(K); k += kWave) state[k] = 0.0;
}

// --------------------------------------------------------------------------
// Diagnostics, spread over the GPU without atomics to global memory:
//   labels  a workgroup per 256 drafts: z and y of each label; within the
//           workgroup the accepted labels' z are packed at the front of its
//           256-slot region of zpos, the rejected ones' in zneg; its label
//           counts, loss sum and bin sums (fixed point: order-free) go to
//           per-workgroup slots;
//   pairs   a workgroup per (region i, region j): accepted of i against
//           rejected of j, 2 x wins + ties;
//   finish  one wave sums the slots and forms the ratios.
// Fixed point: loss in units of 2^-32, bin sums in 2^-40 per label.
// --------------------------------------------------------------------------
constexpr int kDiagTile = 256;
constexpr double kLossScale = 4294967296.0;        // 2^32
constexpr double kBinScale = 1099511627776.0;      // 2^40

struct DiagWs {
    double *zpos, *zneg;        // [regions * 256]
    int32_t *cnt;               // [regions][2]: accepted, rejected
    unsigned long long *loss;   // [regions]
    unsigned long long *bins;   // [regions][nbins]
    unsigned long long *pairs;  // [regions^2]
};

__global__ __launch_bounds__(kDiagTile) void diag_labels_kernel(
    const float *feat, const int32_t *accepted_len, const int32_t *kept_len, int B, int K,
    const float *omega_beta, int nbins, DiagWs ws) {
    constexpr int NW = kDiagTile / kWave;
    __shared__ unsigned long long sh_bins[64];
    __shared__ unsigned long long sh_loss[NW];
    __shared__ int sh_np[NW], sh_nn[NW];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
    const int reg = blockIdx.x;
    for (int q = tid; q < nbins; q += kDiagTile) sh_bins[q] = 0ull;
    __syncthreads();
    const int M = B * K;
    const int t = reg * kDiagTile + tid;
    const int b = t < M ? t / K : 0, i = t < M ? t - b * K : 0;
    const int L = t < M ? (kept_len ? clamp_len(kept_len[b], K) : K) : 0;
    const int a = t < M ? clamp_len(accepted_len[b], K) : 0;
    const int nl = a + 1 < L ? a + 1 : L;
    const bool lab = t < M && i < nl;
    const int yv = i < a ? 1 : 0;
    double z = 0.0;
    int bin = 0;
    uint64_t bv = 0ull, lv = 0ull;
    if (lab) {
        // z rounded after the product and after the sum, as plain double
        // arithmetic forms it
        z = __dadd_rn(__dmul_rn(static_cast<double>(omega_beta[0]), static_cast<double>(feat[t])),
                      static_cast<double>(omega_beta[1 + i]));
        // -log s = softplus(-z), -log(1 - s) = softplus(z)
        const double u = yv ? -z : z;
        const double loss = u > 0.0 ? u + log1p(exp(-u)) : log1p(exp(u));
        const double s = 1.0 / (1.0 + exp(-z));
        bin = static_cast<int>(floor(s * nbins));
        bin = bin < 0 ? 0 : (bin > nbins - 1 ? nbins - 1 : bin);
        bv = static_cast<uint64_t>(llrint((s - yv) * kBinScale));
        lv = static_cast<uint64_t>(llrint(loss * kLossScale));
    }
    wave_keyed_add(sh_bins, bin, bv, lab);
    const bool pos = lab && yv, neg = lab && !yv;
    const uint64_t bp = __ballot(pos), bn = __ballot(neg);
    const uint64_t below = lane ? (~0ull >> (kWave - lane)) : 0ull;  // lanes under this one
    const uint64_t wl = wave_sum_u64(lv);
    if (lane == 0) {
        sh_np[wv] = __popcll(bp);
        sh_nn[wv] = __popcll(bn);
        sh_loss[wv] = wl;
    }
    __syncthreads();
    int op = 0, on = 0;
    for (int w = 0; w < wv; ++w) {
        op += sh_np[w];
        on += sh_nn[w];
    }
    if (pos) ws.zpos[reg * kDiagTile + op + __popcll(bp & below)] = z;
    if (neg) ws.zneg[reg * kDiagTile + on + __popcll(bn & below)] = z;
    if (tid == 0) {
        int np = 0, nn = 0;
        unsigned long long ls = 0ull;
        for (int w = 0; w < NW; ++w) {
            np += sh_np[w];
            nn += sh_nn[w];
            ls += sh_loss[w];
        }
        ws.cnt[2 * reg] = np;
        ws.cnt[2 * reg + 1] = nn;
        ws.loss[reg] = ls;
    }
    for (int q = tid; q < nbins; q += kDiagTile) ws.bins[static_cast<int64_t>(reg) * nbins + q] = sh_bins[q];
}

__global__ __launch_bounds__(kDiagTile) void diag_pairs_kernel(DiagWs ws, int regions) {
    __shared__ double zn[kDiagTile];
    __shared__ unsigned long long acc;
    const int ri = blockIdx.x / regions, rj = blockIdx.x - ri * regions;
    const int np = ws.cnt[2 * ri], nn = ws.cnt[2 * rj + 1];
    if (np == 0 || nn == 0) {
        if (threadIdx.x == 0) ws.pairs[blockIdx.x] = 0ull;
        return;
    }
    const int t = threadIdx.x;
    if (t == 0) acc = 0ull;
    if (t < nn) zn[t] = ws.zneg[rj * kDiagTile + t];
    const double zp = t < np ? ws.zpos[ri * kDiagTile + t] : 0.0;
    __syncthreads();
    unsigned int c = 0;
    if (t < np)
        for (int k = 0; k < nn; ++k) c += zp > zn[k] ? 2u : (zp == zn[k] ? 1u : 0u);
    const uint64_t wc = wave_sum_u64(c);
    if ((threadIdx.x & (kWave - 1)) == 0) atomicAdd(&acc, static_cast<unsigned long long>(wc));
    __syncthreads();
    if (threadIdx.x == 0) ws.pairs[blockIdx.x] = acc;
}

__global__ __launch_bounds__(kWave) void diag_finish_kernel(DiagWs ws, int regions, int nbins,
                                                            double *out) {
    const int lane = threadIdx.x;
    uint64_t part = 0ull, np = 0ull, nn = 0ull, ls = 0ull;
    const int npairs = regions * regions;
    for (int q0 = lane; q0 < npairs; q0 += kFinishBatch * kWave) {
        uint64_t pv[kFinishBatch];
#pragma unroll
        for (int u = 0; u < kFinishBatch; ++u) pv[u] = ws.pairs[min(q0 + u * kWave, npairs - 1)];
#pragma unroll
        for (int u = 0; u < kFinishBatch; ++u)
            if (q0 + u * kWave < npairs) part += pv[u];
    }
    for (int r = lane; r < regions; r += kWave) {
        np += static_cast<uint64_t>(ws.cnt[2 * r]);
        nn += static_cast<uint64_t>(ws.cnt[2 * r + 1]);
        ls += ws.loss[r];
    }
    part = wave_sum_u64(part);
    np = wave_sum_u64(np);
    nn = wave_sum_u64(nn);
    ls = wave_sum_u64(ls);
    // ECE: |sum over regions| per bin, a lane per bin
    long long ece_fp = 0;
    for (int q = lane; q < nbins; q += kWave) {
        uint64_t v = 0ull;
        for (int r0 = 0; r0 < regions; r0 += kFinishBatch) {
            uint64_t bv[kFinishBatch];
#pragma unroll
            for (int u = 0; u < kFinishBatch; ++u)
                bv[u] = ws.bins[static_cast<int64_t>(min(r0 + u, regions - 1)) * nbins + q];
#pragma unroll
            for (int u = 0; u < kFinishBatch; ++u)
                if (r0 + u < regions) v += bv[u];
        }
        const long long sv = static_cast<long long>(v);
        ece_fp += sv < 0 ? -sv : sv;
    }
    ece_fp = static_cast<long long>(wave_sum_u64(static_cast<uint64_t>(ece_fp)));
    if (lane == 0) {
        const double npos = static_cast<double>(np), nneg = static_cast<double>(nn);
        const double N = npos + nneg;
        const double nan = __builtin_nan("");
        out[0] = (npos > 0.0 && nneg > 0.0) ? static_cast<double>(part) / (2.0 * npos * nneg) : nan;
        out[1] = N > 0.0 ? static_cast<double>(ls) / kLossScale / N : nan;
        out[2] = N > 0.0 ? static_cast<double>(ece_fp) / kBinScale / N : nan;
        out[3] = N;
    }
}

// --------------------------------------------------------------------------
// Budgeted trimming, spread over the GPU:
//   key      survival of a draft (its float running product) and its index
//            as one 64-bit key (~ordered(survival), flat index): ascending
//            keys = decreasing survival, ties by flat index; all distinct;
//   rank     a 2D grid of 256 x 256 tiles counts, for every draft, the keys
//            of one tile below its own (exact integer counts);
//   scatter  rank = sum of its counts; the draft's survival and index go to
//            that slot of the sorted arrays;
//   finish   one workgroup scans the sorted survivals (double), takes the
//            first best ratio, and marks the first `budget` drafts.
// Workspace: counts[tiles][M] u16 | sorted_s[M] f32 | sorted_e[M] i32.
// --------------------------------------------------------------------------
constexpr int kBudgetMax = 1 << 16;
constexpr int kBudgetTile = 256;
constexpr int kBudgetThreads = 1024;

struct BudgetWs {
    uint16_t *counts;
    float *sorted_s;
    int32_t *sorted_e;
};

// Key of draft f: its survival (the running float product along its
// sequence) and its index.
__device__ __forceinline__ unsigned long long budget_key(const float *conf, int K, int f) {
    const int b = f / K, i = f - b * K;
    float S = 1.0f;
    for (int q = 0; q <= i; ++q) S = S * conf[b * K + q];
    return (static_cast<unsigned long long>(~ordered_bits(S)) << 32) |
           static_cast<unsigned int>(f);
}

__global__ __launch_bounds__(kBudgetTile) void budget_rank_kernel(const float *conf, int K,
                                                                 BudgetWs ws, int M, int tiles) {
    __shared__ unsigned long long tk[kBudgetTile];
    const int te = blockIdx.x / tiles, tt = blockIdx.x - te * tiles;
    const int e = te * kBudgetTile + threadIdx.x;
    const int k = tt * kBudgetTile + threadIdx.x;
    tk[threadIdx.x] = k < M ? budget_key(conf, K, k) : ~0ull;  // padding sorts last
    const unsigned long long me = e < M ? budget_key(conf, K, e) : 0ull;
    __syncthreads();
    if (e >= M) return;
    unsigned int c = 0;
#pragma unroll 8
    for (int q = 0; q < kBudgetTile; ++q) c += tk[q] < me ? 1u : 0u;
    ws.counts[static_cast<int64_t>(tt) * M + e] = static_cast<uint16_t>(c);
}

__global__ __launch_bounds__(256) void budget_scatter_kernel(const float *conf, int K, BudgetWs ws,
                                                           int M, int tiles) {
    const int e = blockIdx.x * 256 + threadIdx.x;
    if (e >= M) return;
    int r = 0;
#pragma unroll 8
    for (int t = 0; t < tiles; ++t) r += ws.counts[static_cast<int64_t>(t) * M + e];
    const unsigned long long key = budget_key(conf, K, e);
    ws.sorted_s[r] = from_ordered_bits(~static_cast<unsigned int>(key >> 32));
    ws.sorted_e[r] = static_cast<int32_t>(key & 0xFFFFFFFFull);
}

template <int NT>
__global__ __launch_bounds__(NT) void budget_finish_kernel(BudgetWs ws, int B, int K,
                                                          const double *cost, double n_requests,
                                                          int32_t *kept_len, uint8_t *mask,
                                                          int64_t *budget_out, double *best_ratio) {
    const int M = B * K;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wv = tid / kWave;
    // prefix sums of the sorted survivals: each thread a contiguous segment
    const int seg = (M + NT - 1) / NT;
    const int s0 = tid * seg < M ? tid * seg : M;
    const int s1 = s0 + seg < M ? s0 + seg : M;
    double tot = 0.0;
#pragma unroll 8
    for (int t = s0; t < s1; ++t) tot += static_cast<double>(ws.sorted_s[t]);
    __shared__ double wsum[NT / kWave];
    double incl = tot;
    for (int o = 1; o < kWave; o <<= 1) {
        const double v = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += v;
    }
    double excl = __shfl_up(incl, 1, kWave);
    if (lane == 0) excl = 0.0;
    if (lane == kWave - 1) wsum[wv] = incl;
    __syncthreads();
    double before = 0.0;
    for (int w = 0; w < wv; ++w) before += wsum[w];
    double est = n_requests + (before + excl);
    double best = -__builtin_inf();
    int bk = INT_MAX;
    if (tid == 0) {
        best = n_requests / cost[0];
        bk = 0;
    }
    for (int t = s0; t < s1; ++t) {
        est += static_cast<double>(ws.sorted_s[t]);
        const double r = est / cost[t + 1];
        if (r > best) {
            best = r;
            bk = t + 1;
        }
    }
    for (int o = kWave / 2; o > 0; o /= 2) {  // first maximum
        const double ob = __shfl_xor(best, o, kWave);
        const int ok = __shfl_xor(bk, o, kWave);
        if (ob > best || (ob == best && ok < bk)) {
            best = ob;
            bk = ok;
        }
    }
    __shared__ double wb[NT / kWave];
    __shared__ int wk[NT / kWave];
    __shared__ int s_budget;
    if (lane == 0) {
        wb[wv] = best;
        wk[wv] = bk;
    }
    for (int b = tid; b < B; b += NT) kept_len[b] = 0;
    for (int f = tid; f < M && mask; f += NT) mask[f] = 0;
    __syncthreads();
    if (tid == 0) {
        double b0 = wb[0];
        int k0 = wk[0];
        for (int w = 1; w < NT / kWave; ++w)
            if (wb[w] > b0 || (wb[w] == b0 && wk[w] < k0)) {
                b0 = wb[w];
                k0 = wk[w];
            }
        s_budget = k0;
        *budget_out = k0;
        if (best_ratio) *best_ratio = b0;
    }
    __syncthreads();
    // kept drafts are a prefix of each sequence: kept_len = 1 + last kept position
    for (int t = tid; t < s_budget; t += NT) {
        const int e = ws.sorted_e[t];
        if (mask) mask[e] = 1;
        atomicMax(&kept_len[e / K], e % K + 1);
    }
}

// --------------------------------------------------------------------------
// Prompt lookup: one workgroup per sequence, one backward pass.  For an end
// position e <= n-2 let l(e) be the length of the match between the tokens
// ending at e and the context's last tokens (capped at n_max).  A g-gram
// occurrence ends at e iff l(e) >= g; the answer is the largest g with such
// an e, and the largest e for it.  The workgroup scans e = n-2, n-3, ...,
// NT*U positions per pass, keeps best_e[g] = max e with l(e) >= g in LDS, and
// stops once the longest possible length has an occurrence (the first pass
// that finds one holds its latest).
// --------------------------------------------------------------------------
constexpr int kNgramMax = 32;

template <int NT, int U>
__global__ __launch_bounds__(NT) void ngram_kernel(const int32_t *ctx, const int32_t *lengths,
                                                  int64_t stride, int n_min, int n_max, int K,
                                                  int32_t *draft, int32_t *draft_len,
                                                  int32_t *match_pos, int32_t *match_n) {
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int32_t *c = ctx + static_cast<int64_t>(b) * stride;
    const int nb = lengths[b];
    const int n = nb < 0 ? 0 : (nb > stride ? static_cast<int>(stride) : nb);
    __shared__ int32_t suf[kNgramMax];     // suf[q] = c[n-1-q]
    __shared__ int best_e[kNgramMax + 1];  // by length g
    __shared__ int s_stop;
    // the longest length that can occur: an occurrence ends at e <= n-2
    const int gmax = n_max < n - 1 ? n_max : n - 1;
    for (int q = tid; q <= kNgramMax; q += NT) best_e[q] = -1;
    if (tid < gmax) suf[tid] = c[n - 1 - tid];
    __syncthreads();
    if (gmax >= n_min) {
        for (int top = n - 2; top >= 0; top -= NT * U) {
            int32_t last[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {  // the tokens at e, loaded together
                const int e = top - tid - NT * u;
                last[u] = e >= 0 ? c[e] : -1;
            }
            const int32_t s0 = suf[0];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int e = top - tid - NT * u;
                if (e >= 0 && last[u] == s0) {
                    int l = 1;
                    while (l < gmax && l <= e && c[e - l] == suf[l]) ++l;
                    for (int g = n_min; g <= l; ++g) atomicMax(&best_e[g], e);
                }
            }
            __syncthreads();
            if (tid == 0) s_stop = best_e[gmax] >= 0;
            __syncthreads();
            if (s_stop) break;
        }
    }
    int pos = -1, gf = 0;
    for (int g = gmax; g >= n_min; --g)
        if (best_e[g] >= 0) {
            pos = best_e[g] - g + 1;
            gf = g;
            break;
        }
    int dl = 0;
    if (pos >= 0) {
        dl = n - (pos + gf);
        dl = dl > K ? K : dl;
    }
    for (int k = tid; k < K; k += NT)
        draft[static_cast<int64_t>(b) * K + k] = k < dl ? c[pos + gf + k] : -1;
    if (tid == 0) {
        draft_len[b] = dl;
        if (match_pos) match_pos[b] = pos;
        if (match_n) match_n[b] = gf;
    }
}

}  // namespace sv
