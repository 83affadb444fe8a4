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

namespace sv {

// Confidence of a draft with feature f at a position with intercept beta.
__device__ __forceinline__ double av_confidence(double omega, float f, float beta) {
    const double z = omega * static_cast<double>(f) + static_cast<double>(beta);
    return 1.0 / (1.0 + exp(-z));
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

}  // namespace sv
