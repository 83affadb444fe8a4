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

#include "sv_common.hpp"

namespace sv {

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

template <int NT, bool CURV>
__device__ void label_sums(const float *feat, const int32_t *accepted_len,
                           const int32_t *kept_len, int B, int K, const float *omega_beta,
                           LabelSums *out) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    const double omega = static_cast<double>(omega_beta[0]);
    for (int i = wv; i < K; i += NT / kWave) {
        const double beta = static_cast<double>(omega_beta[1 + i]);
        double n = 0.0, r = 0.0, rf = 0.0, w = 0.0, wf = 0.0, wff = 0.0;
        for (int b = lane; b < B; b += kWave) {
            const int L = kept_len ? clamp_len(kept_len[b], K) : K;
            const int a = clamp_len(accepted_len[b], K);
            const int nl = a + 1 < L ? a + 1 : L;
            if (i < nl) {
                const double f = static_cast<double>(feat[static_cast<int64_t>(b) * K + i]);
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
// adaptive-verification workloads run every step).
template <int NT>
__global__ __launch_bounds__(NT) void av_sgd_kernel(const float *feat, const int32_t *accepted_len,
                                                   const int32_t *kept_len, int B, int K, float lr,
                                                   float *omega_beta) {
    __shared__ LabelSums sums[64];
    label_sums<NT, false>(feat, accepted_len, kept_len, B, K, omega_beta, sums);
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
        if (threadIdx.x < K)
            omega_beta[1 + threadIdx.x] = static_cast<float>(
                static_cast<double>(omega_beta[1 + threadIdx.x]) - l * sums[threadIdx.x].r);
    }
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
    label_sums<NT, true>(feat, accepted_len, kept_len, B, K, omega_beta, sums);
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
// Diagnostics.  Workspace: z[M] doubles (NaN where no label) | y[M] int8 |
// counters: loss (fixed point 2^-32), npos, nneg, bins[nbins] (fixed point
// 2^-40) | pair partials [tiles^2] uint64 (2 x wins + ties).
// Fixed-point sums make the order of additions irrelevant, so the figures are
// deterministic; the rounding is below 2^-32 per label.
// --------------------------------------------------------------------------
constexpr int kDiagTile = 256;
constexpr double kLossScale = 4294967296.0;        // 2^32
constexpr double kBinScale = 1099511627776.0;      // 2^40

struct DiagWs {
    double *z;
    int8_t *y;
    unsigned long long *ctr;  // [0] loss, [1] npos, [2] nneg, [3..3+nbins) bins
    unsigned long long *pairs;
};

template <int NT>
__global__ __launch_bounds__(NT) void diag_labels_kernel(const float *feat,
                                                        const int32_t *accepted_len,
                                                        const int32_t *kept_len, int B, int K,
                                                        const float *omega_beta, int nbins,
                                                        DiagWs ws) {
    __shared__ unsigned long long sh[3 + 64];
    for (int q = threadIdx.x; q < 3 + nbins; q += NT) sh[q] = 0ull;
    __syncthreads();
    const double omega = static_cast<double>(omega_beta[0]);
    const int M = B * K;
    for (int t = threadIdx.x; t < M; t += NT) {
        const int b = t / K, i = t - b * K;
        const int L = kept_len ? clamp_len(kept_len[b], K) : K;
        const int a = clamp_len(accepted_len[b], K);
        const int nl = a + 1 < L ? a + 1 : L;
        if (i < nl) {
            // z rounded after the product and after the sum, as plain double
            // arithmetic forms it
            const double z = __dadd_rn(__dmul_rn(omega, static_cast<double>(feat[t])),
                                       static_cast<double>(omega_beta[1 + i]));
            const int yv = i < a ? 1 : 0;
            ws.z[t] = z;
            ws.y[t] = static_cast<int8_t>(yv);
            // -log s = softplus(-z), -log(1 - s) = softplus(z)
            const double u = yv ? -z : z;
            const double loss = u > 0.0 ? u + log1p(exp(-u)) : log1p(exp(u));
            const double s = 1.0 / (1.0 + exp(-z));
            int bin = static_cast<int>(floor(s * nbins));
            bin = bin < 0 ? 0 : (bin > nbins - 1 ? nbins - 1 : bin);
            atomicAdd(&sh[0], static_cast<unsigned long long>(llrint(loss * kLossScale)));
            atomicAdd(&sh[yv ? 1 : 2], 1ull);
            atomicAdd(&sh[3 + bin],
                      static_cast<unsigned long long>(llrint((s - yv) * kBinScale)));
        } else {
            ws.z[t] = __builtin_nan("");
            ws.y[t] = -1;
        }
    }
    __syncthreads();
    for (int q = threadIdx.x; q < 3 + nbins; q += NT) ws.ctr[q] = sh[q];
}

// Tile (row tile, column tile): rows that are accepted against columns that
// are rejected.  One partial per workgroup.
__global__ __launch_bounds__(kDiagTile) void diag_pairs_kernel(DiagWs ws, int M, int tiles) {
    __shared__ double cz[kDiagTile];
    __shared__ int8_t cy[kDiagTile];
    __shared__ unsigned long long acc;
    const int rt = blockIdx.x / tiles, ct = blockIdx.x - rt * tiles;
    const int r = rt * kDiagTile + threadIdx.x, c = ct * kDiagTile + threadIdx.x;
    if (threadIdx.x == 0) acc = 0ull;
    cz[threadIdx.x] = c < M ? ws.z[c] : 0.0;
    cy[threadIdx.x] = c < M ? ws.y[c] : static_cast<int8_t>(-1);
    const bool pos = r < M && ws.y[r] == 1;
    const double zr = r < M ? ws.z[r] : 0.0;
    __syncthreads();
    unsigned int cnt = 0;
    if (pos) {
        for (int k = 0; k < kDiagTile; ++k) {
            if (cy[k] == 0) cnt += zr > cz[k] ? 2u : (zr == cz[k] ? 1u : 0u);
        }
    }
    atomicAdd(&acc, static_cast<unsigned long long>(cnt));
    __syncthreads();
    if (threadIdx.x == 0) ws.pairs[blockIdx.x] = acc;
}

__global__ __launch_bounds__(kWave) void diag_finish_kernel(DiagWs ws, int nbins, int npart,
                                                            double *out) {
    unsigned long long part = 0ull;
    for (int q = threadIdx.x; q < npart; q += kWave) part += ws.pairs[q];
    // integer sums: any order gives the same total
    for (int o = kWave / 2; o > 0; o /= 2)
        part += static_cast<unsigned long long>(__shfl_xor(static_cast<long long>(part), o));
    if (threadIdx.x == 0) {
        const double npos = static_cast<double>(ws.ctr[1]);
        const double nneg = static_cast<double>(ws.ctr[2]);
        const double N = npos + nneg;
        long long ece_fp = 0;
        for (int q = 0; q < nbins; ++q) {
            const long long v = static_cast<long long>(ws.ctr[3 + q]);
            ece_fp += v < 0 ? -v : v;
        }
        const double nan = __builtin_nan("");
        out[0] = (npos > 0.0 && nneg > 0.0) ? static_cast<double>(part) / (2.0 * npos * nneg) : nan;
        out[1] = N > 0.0 ? static_cast<double>(ws.ctr[0]) / kLossScale / N : nan;
        out[2] = N > 0.0 ? static_cast<double>(ece_fp) / kBinScale / N : nan;
        out[3] = N;
    }
}

// --------------------------------------------------------------------------
// Budgeted trimming: one workgroup, the B*K <= kBudgetMax survivals sorted in
// LDS by a bitonic network on 64-bit keys (~ordered(survival), flat index).
// --------------------------------------------------------------------------
constexpr int kBudgetMax = 16384;
constexpr int kBudgetThreads = 1024;

template <int NT>
__global__ __launch_bounds__(NT) void budget_kernel(const float *conf, int B, int K,
                                                   const double *cost, double n_requests,
                                                   int32_t *kept_len, uint8_t *mask,
                                                   int64_t *budget_out, double *best_ratio) {
    extern __shared__ unsigned long long keys[];  // [P] then M mask bytes
    const int M = B * K;
    int P = 1;
    while (P < M) P <<= 1;
    uint8_t *kmask = reinterpret_cast<uint8_t *>(keys + P);
    const int tid = threadIdx.x;
    // survival, formed in float along each sequence
    for (int b = tid; b < B; b += NT) {
        float S = 1.0f;
        for (int i = 0; i < K; ++i) {
            const int f = b * K + i;
            S = S * conf[f];
            keys[f] = (static_cast<unsigned long long>(~ordered_bits(S)) << 32) |
                      static_cast<unsigned int>(f);
        }
    }
    for (int f = M + tid; f < P; f += NT) keys[f] = ~0ull;
    for (int f = tid; f < M; f += NT) kmask[f] = 0;
    __syncthreads();
    // ascending bitonic sort: survival decreasing, ties by flat index
    for (int k = 2; k <= P; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int e = tid; e < P / 2; e += NT) {
                const int lo = (e / j) * 2 * j + (e % j);
                const int hi = lo + j;
                const bool up = (lo & k) == 0;
                const unsigned long long x = keys[lo], y = keys[hi];
                if ((x > y) == up) {
                    keys[lo] = y;
                    keys[hi] = x;
                }
            }
            __syncthreads();
        }
    }
    // prefix sums of the sorted survivals: each thread a contiguous segment
    const int seg = (M + NT - 1) / NT;
    const int s0 = tid * seg, s1 = min(M, s0 + seg);
    auto surv_at = [&](int t) -> double {
        return static_cast<double>(from_ordered_bits(~static_cast<unsigned int>(keys[t] >> 32)));
    };
    double tot = 0.0;
    for (int t = s0; t < s1; ++t) tot += surv_at(t);
    // exclusive scan of the segment totals (fixed order)
    __shared__ double wsum[NT / kWave];
    const int lane = tid & (kWave - 1), wv = tid / kWave;
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
    // best ratio over this segment's budgets k = t+1 (and k = 0 for thread 0)
    double best = -__builtin_inf();
    int bk = INT_MAX;
    if (tid == 0) {
        best = n_requests / cost[0];
        bk = 0;
    }
    for (int t = s0; t < s1; ++t) {
        est += surv_at(t);
        const double r = est / cost[t + 1];
        if (r > best) {
            best = r;
            bk = t + 1;
        }
    }
    // first maximum over the workgroup
    for (int o = kWave / 2; o > 0; o /= 2) {
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
    for (int t = tid; t < s_budget; t += NT) kmask[keys[t] & 0xFFFFFFFFull] = 1;
    __syncthreads();
    for (int f = tid; f < M && mask; f += NT) mask[f] = kmask[f];
    for (int b = tid; b < B; b += NT) {
        int n = 0;
        for (int i = 0; i < K; ++i) n += kmask[b * K + i];
        kept_len[b] = n;
    }
}

// --------------------------------------------------------------------------
// Prompt lookup: one workgroup per sequence.  For n-gram length g from n_max
// down, the workgroup scans start positions p = n-g-1, n-g-2, ... NT at a
// time and stops at the first block of positions holding a match; the
// largest matching p there is the latest earlier occurrence.
// --------------------------------------------------------------------------
constexpr int kNgramMax = 32;

template <int NT>
__global__ __launch_bounds__(NT) void ngram_kernel(const int32_t *ctx, const int32_t *lengths,
                                                  int64_t stride, int n_min, int n_max, int K,
                                                  int32_t *draft, int32_t *draft_len,
                                                  int32_t *match_pos, int32_t *match_n) {
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int32_t *c = ctx + static_cast<int64_t>(b) * stride;
    const int nb = lengths[b];
    const int n = nb < 0 ? 0 : (nb > stride ? static_cast<int>(stride) : nb);
    __shared__ int32_t suf[kNgramMax];
    __shared__ int s_hit;
    __shared__ int wmin[NT / kWave];
    int pos = -1, gf = 0;
    for (int g = n_max; g >= n_min && pos < 0; --g) {
        if (g >= n) continue;
        __syncthreads();
        if (tid < g) suf[tid] = c[n - g + tid];
        __syncthreads();
        for (int base = n - g - 1; base >= 0; base -= NT) {
            const int p = base - tid;
            bool ok = p >= 0;
            // last token first: most start positions fail there
            for (int q = g - 1; q >= 0 && ok; --q) ok = c[p + q] == suf[q];
            // smallest thread index with a match = largest p
            const unsigned long long m = __ballot(ok);
            if ((tid & (kWave - 1)) == 0)
                wmin[tid / kWave] = m ? (tid + __ffsll(static_cast<long long>(m)) - 1) : INT_MAX;
            __syncthreads();
            if (tid == 0) {
                int mn = INT_MAX;
                for (int w = 0; w < NT / kWave; ++w) mn = wmin[w] < mn ? wmin[w] : mn;
                s_hit = mn;
            }
            __syncthreads();
            const int hit = s_hit;
            if (hit != INT_MAX) {
                pos = base - hit;
                gf = g;
                break;
            }
        }
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
