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
// Update (section "Ajuste de los Coeficientes" for which drafts carry a
// label): one gradient step on the mean log-loss over the batch's labels.
#pragma once

#include "sv_common.hpp"

namespace sv {

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
        const double z = omega * static_cast<double>(feat[b * K + i]) +
                         static_cast<double>(omega_beta[1 + i]);
        const double ci = 1.0 / (1.0 + exp(-z));
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

// Single workgroup; fixed-order double reduction.  Labels of sequence b:
// positions i < min(a_b + 1, L_b), y = 1 for i < a_b (accepted), y = 0 at the
// first rejection; trimmed positions and those after the rejection have none.
template <int NT>
__global__ __launch_bounds__(NT) void av_update_kernel(const float *feat,
                                                      const int32_t *accepted_len,
                                                      const int32_t *kept_len, int B, int K,
                                                      float lr, float *omega_beta) {
    __shared__ double red[NT];
    __shared__ double gbeta[64];
    __shared__ double gomega;
    __shared__ double nlab;
    const int tid = threadIdx.x;
    const double omega = static_cast<double>(omega_beta[0]);

    auto block_sum = [&](double v) -> double {
        red[tid] = v;
        __syncthreads();
#pragma unroll
        for (int s = NT / 2; s > 0; s >>= 1) {
            if (tid < s) red[tid] += red[tid + s];
            __syncthreads();
        }
        const double r = red[0];
        __syncthreads();
        return r;
    };

    double go = 0.0, n = 0.0;
    for (int i = 0; i < K; ++i) {
        const double beta = static_cast<double>(omega_beta[1 + i]);
        double gb = 0.0;
        for (int b = tid; b < B; b += NT) {
            const int L = kept_len ? clamp_len(kept_len[b], K) : K;
            const int acc = clamp_len(accepted_len[b], K);
            const int nl = acc + 1 < L ? acc + 1 : L;
            if (i < nl) {
                const double f = static_cast<double>(feat[b * K + i]);
                const double s = 1.0 / (1.0 + exp(-(omega * f + beta)));
                const double d = s - (i < acc ? 1.0 : 0.0);
                gb += d;
                go += d * f;
                n += 1.0;
            }
        }
        const double tot = block_sum(gb);
        if (tid == 0) gbeta[i] = tot;
    }
    const double tgo = block_sum(go);
    const double tn = block_sum(n);
    if (tid == 0) {
        gomega = tgo;
        nlab = tn;
    }
    __syncthreads();
    if (nlab > 0.0) {
        const double l = static_cast<double>(lr) / nlab;
        if (tid == 0) omega_beta[0] = static_cast<float>(omega - l * gomega);
        if (tid < K)
            omega_beta[1 + tid] =
                static_cast<float>(static_cast<double>(omega_beta[1 + tid]) - l * gbeta[tid]);
    }
}

}  // namespace sv
