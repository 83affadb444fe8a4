// sv_av.hpp -- adaptive-verification scorer, trimming and online update
// (page "Verificacion Adaptativa sin una cabeza de confianza").
//
// Scorer (sections "Solucion" and "Puntuar la Distribucion"): one logistic
// regression per draft position i with a slope omega shared by all positions
// and an intercept beta_i, on the single feature logit(q_max):
//   c_i = sigmoid(omega * logit(q_max,i) + beta_i).
// Trimming: survival is the running product of c over positions (section
// "Otras Caracteristicas Consideradas"); a position is kept while it stays at
// or above tau.
// The update that runs every step (section "Ajuste de los Coeficientes" for
// which drafts carry a label) lives with the Newton refit in sv_next.hpp.
#pragma once

#include "sv_common.hpp"
#include "sv_rowstats.hpp"

namespace sv {

// Confidence of a draft with feature f at a position with intercept beta.
__device__ __forceinline__ double av_confidence(double omega, float f, float beta) {
    const double z = omega * static_cast<double>(f) + static_cast<double>(beta);
    return 1.0 / (1.0 + exp(-z));
}

// The same behind a call, for a loop over rows (see row_emit_stats).
__device__ __attribute__((noinline)) double av_confidence_call(double omega, float f,
                                                               float beta) {
    return av_confidence(omega, f, beta);
}

// One thread per sequence.  feat: [B*K] (draft statistics).
__global__ void av_score_kernel(const float *feat, int B, int K, const float *omega_beta,
                                float tau, float *conf, uint8_t *keep_mask, int32_t *kept_len) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= B) return;
    const double omega = static_cast<double>(omega_beta[0]);
    const double t = static_cast<double>(tau);
    double P = 1.0;
    bool open = true;
    int L = 0;
    for (int i = 0; i < K; ++i) {
        const double ci = av_confidence(omega, feat[b * K + i], omega_beta[1 + i]);
        P *= ci;
        const bool keep = open && (t <= 0.0 || P >= t);
        if (conf) conf[b * K + i] = static_cast<float>(ci);
        if (keep_mask) keep_mask[b * K + i] = keep ? 1 : 0;
        if (keep)
            ++L;
        else
            open = false;
    }
    if (kept_len) kept_len[b] = L;
}

// Scoring and trimming that read only the draft rows the trim needs.
// Workgroup b streams draft row (b, i) with the row pass for i = 0, 1, ...,
// scores it as av_score_kernel does (same arithmetic, same order) and stops
// after the first position whose survival falls below tau: that row decides
// the trim, the rows after it cannot change anything a step uses (they are
// neither verified nor labelled).  Their confidence and statistics are
// reported as NaN and their mask as 0.
struct PrefixArgs {
    const void *draft;        // [B][K] rows
    int64_t stride;           // elements between rows
    int32_t V, K;
    const int32_t *tokens;    // [B][K]
    float c;                  // log2(e) / T
    float pad_;
    double inv_ln_v;
    // draft statistics, [B*K] each
    double *lse2, *logq2;
    float *qmax, *feat;
};

template <typename T, int BLOCK, int UNROLL>
__global__ __launch_bounds__(BLOCK) void av_prefix_kernel(PrefixArgs pa, const float *omega_beta,
                                                          float tau, float *conf,
                                                          uint8_t *keep_mask, int32_t *kept_len) {
    __shared__ uint4 sh_saved[UNROLL][BLOCK];
    __shared__ int s_open;
    // The row pass's arguments with every output it need not write left null
    // as literals, so that the loop keeps few values live.
    RowArgs a{};
    RowGroup &g = a.g[0];
    g.base = pa.draft;
    g.stride = pa.stride;
    g.rows_per_seq = pa.K;
    g.gather_rows = pa.K;
    g.lse2 = pa.lse2;
    g.logtok2 = pa.logq2;
    g.qmax_int = pa.qmax;
    g.feat_int = pa.feat;
    a.g[1].rows_per_seq = 1;
    a.V = pa.V;
    a.K = pa.K;
    a.tokens = pa.tokens;
    a.c = pa.c;
    a.inv_ln_v = pa.inv_ln_v;
    const int b = blockIdx.x;
    const int K = pa.K;
    const double t = static_cast<double>(tau);
    double P = 1.0;  // thread 0's running survival
    int L = 0;
    int i = 0;
    while (i < K) {
        const int64_t row = static_cast<int64_t>(b) * K + i;
        // V and the thread index made opaque to the loop: otherwise the
        // compiler hoists every per-thread value derived from them (the
        // partial chunk's element masks, the saved chunk's ids) out of the
        // loop and keeps them all live, which more than doubles the row
        // pass's registers
        int Vi = pa.V;
        asm volatile("" : "+s"(Vi));
        a.V = Vi;
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        row_one<T, BLOCK, UNROLL, false, false, true>(a, g, row, sh_saved, tid);
        if (threadIdx.x == 0) {
            // thread 0 wrote this row's feature itself (row_emit_stats)
            const double ci = av_confidence_call(static_cast<double>(omega_beta[0]),
                                                 pa.feat[row], omega_beta[1 + i]);
            P *= ci;
            const bool keep = t <= 0.0 || P >= t;  // still open: every earlier one was kept
            if (conf) conf[row] = static_cast<float>(ci);
            if (keep_mask) keep_mask[row] = keep ? 1 : 0;
            if (keep) ++L;
            s_open = keep ? 1 : 0;
        }
        __syncthreads();
        // one value for the whole workgroup: readfirstlane tells the compiler
        // so, which keeps the loop control in scalar registers
        const bool more = __builtin_amdgcn_readfirstlane(s_open) != 0;
        ++i;
        __syncthreads();  // every thread has read s_open before the next row's write
        if (!more) break;
    }
    if (threadIdx.x == 0) {
        const float nanf = __builtin_nanf("");
        const double nand = __builtin_nan("");
        for (int r = i; r < K; ++r) {
            const int64_t row = static_cast<int64_t>(b) * K + r;
            if (conf) conf[row] = nanf;
            if (keep_mask) keep_mask[row] = 0;
            pa.lse2[row] = nand;
            pa.logq2[row] = nand;
            pa.qmax[row] = nanf;
            pa.feat[row] = nanf;
        }
        if (kept_len) kept_len[b] = L;
    }
}

}  // namespace sv
