// sv_step.hpp -- the launch that ends an adaptive-verification step: each
// sequence's emitted token (the race's combine) and, in one more workgroup of
// the same launch, the estimator's update (page "Verificacion Adaptativa sin
// una cabeza de confianza", section "Ajuste de los Coeficientes").
//
// The update's labels need only each sequence's accepted length, and every
// segment candidate of the race already carries it (the first rejected
// position, or L_b), so the update does not wait for the combine: the two run
// side by side, where separate launches would run one after the other.
#pragma once

#include "sv_finish.hpp"
#include "sv_next.hpp"

namespace sv {

// Accepted length of sequence b from its first segment candidate.
struct AcceptedFromCand {
    const RaceCand *cand;
    int segs;
    __device__ int operator()(int b) const {
        return static_cast<int>(cand[static_cast<int64_t>(b) * segs].info & 0xFFu);
    }
};

struct StepUpdate {
    const float *feat;        // [B*K] draft log-odds (the draft statistics' feat)
    const int32_t *kept_len;  // [B] or null (= K)
    float *omega_beta;        // [K+1], updated in place
    float *conf;              // [B*K] or null: confidences before the update
    uint8_t *keep_mask;       // [B*K] or null
    int32_t *kept_out;        // [B] or null
    int32_t B;
    float lr;
    int32_t score;            // nonzero: write conf, keep_mask, kept_out (untrimmed step)
};

// Workgroups 0..ceil(B/NW)-1 pick tokens, one wave per sequence, as
// race_combine_kernel does; the last workgroup scores (when asked) and takes
// the SGD step as av_score_update_kernel / av_sgd_kernel do.  A residual that
// vanished in floating point is raced again over p by its whole workgroup.
template <typename T, int NT>
__global__ __launch_bounds__(NT) void race_step_kernel(RaceArgs a, const int32_t *tokens,
                                                      int32_t *accepted_len, int32_t *out_tokens,
                                                      uint32_t *boundary, StepUpdate u) {
    constexpr int NW = NT / kWave;
    const int ncomb = (u.B + NW - 1) / NW;
    if (static_cast<int>(blockIdx.x) < ncomb) {
        const int lane = threadIdx.x & (kWave - 1);
        const int wv = threadIdx.x / kWave;
        const int b = static_cast<int>(blockIdx.x) * NW + wv;
        __shared__ int s_fb[NW], s_j[NW];
        __shared__ double s_k1, s_k2;
        __shared__ int s_y;
        SeqPick s{};
        if (b < u.B) s = combine_reduce(a, tokens, b, lane);
        if (lane == 0) {
            s_fb[wv] = b < u.B && s.y < 0;
            s_j[wv] = s.jstar;
        }
        __syncthreads();
        for (int w = 0; w < NW; ++w) {  // s_fb is the same for every thread
            if (!s_fb[w]) continue;
            double k = -__builtin_inf(), kk2 = -__builtin_inf();
            int x = -1;
            combine_fallback<T, NT>(a, static_cast<int>(blockIdx.x) * NW + w, s_j[w], &k, &x,
                                    &kk2);
            if (threadIdx.x == 0) {
                s_y = x;
                s_k1 = k;
                s_k2 = kk2;
            }
            __syncthreads();
            if (wv == w) {
                s.y = s_y;
                s.k1 = s_k1;
                s.k2 = s_k2;
                s.flags |= kResidualEmpty;
            }
            __syncthreads();  // s_y is read before the next fallback writes it
        }
        if (b < u.B) combine_emit(a, b, lane, s, accepted_len, out_tokens, boundary);
        return;
    }
    if (u.score)
        score_untrimmed<NT>(u.feat, u.B, a.K, u.omega_beta, u.conf, u.keep_mask, u.kept_out);
    sgd_step<NT>(u.feat, AcceptedFromCand{a.cand, a.segs}, u.kept_len, u.B, a.K, u.lr,
                 u.omega_beta);
}

}  // namespace sv
