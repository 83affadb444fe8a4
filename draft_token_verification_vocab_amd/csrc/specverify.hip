// specverify.hip -- host side of the C ABI declared in include/specverify.h:
// argument validation, workspace layout, kernel selection and launches on
// the caller's stream.  No allocation, no synchronisation.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstddef>
#include <cstdint>

#include "specverify.h"
#include "sv_av.hpp"
#include "sv_common.hpp"
#include "sv_finish.hpp"
#include "sv_next.hpp"
#include "sv_rowstats.hpp"
#include "sv_step.hpp"

namespace {

using namespace sv;

static_assert(kNearAccept == SPEC_NEAR_ACCEPT && kNearRace == SPEC_NEAR_RACE &&
                  kResidualEmpty == SPEC_RESIDUAL_EMPTY && kNearGate == SPEC_NEAR_GATE,
              "the kernels' boundary bits are the ABI's");

// Race shape and the number of race workgroups to aim for per launch: at the
// race's 71 registers a SIMD holds seven waves, so seven 256-thread
// workgroups per compute unit, 1792 on MI355X's 256 compute units, run in one
// round (2048 left an eighth of them waiting for a slot: B = 64 and B = 256
// lossless steps 1.3 and 2.4 us slower).
constexpr int kRaceBlock = 256;
constexpr int kRaceTargetBlocks = 7 * 256;
constexpr int kMaxSegs = 64;
static_assert(kMaxSegs <= kWave, "the combine reads one segment per lane of one wave");
constexpr int kSmallBlock = 64;
// FLy resolver: one wave per sequence.
constexpr int kFlyBlock = 256;
// Label reductions (SGD step, Newton accumulation): a wave per position.
constexpr int kLabelBlock = 512;
// Sequences per token-picking workgroup of race_step_kernel (a wave each).
constexpr int kStepSeqs = kLabelBlock / kWave;
// Diagnostics: labels per call, bins, label-kernel workgroup.
constexpr int64_t kDiagMaxLabels = 1 << 16;
constexpr int kDiagMaxBins = 64;
// Prompt lookup: one workgroup per sequence.
constexpr int kNgramBlock = 256;
constexpr int kNgramUnroll = 8;

size_t align_up(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

int elem_size(int32_t dtype) { return dtype == SPEC_DTYPE_F32 ? 4 : 2; }

int race_segments(int32_t B, int32_t V) {
    if (B <= 0) return 1;
    const int ngroups = (V + kRaceGroup - 1) / kRaceGroup;
    int segs = (kRaceTargetBlocks + B - 1) / B;
    const int max_by_len = ngroups / kRaceBlock;  // keep at least one group per thread
    if (segs > max_by_len) segs = max_by_len;
    if (segs > kMaxSegs) segs = kMaxSegs;
    return segs < 1 ? 1 : segs;
}

struct WsLayout {
    size_t t_lse2, t_logp2, t_h, t_am, dstats, cand, bonus_cnt, bonus_list, total;
};

WsLayout layout_for(int32_t B, int32_t K, int32_t V) {
    const size_t rows_t = static_cast<size_t>(B) * (K + 1);
    const size_t n = static_cast<size_t>(B) * K;
    WsLayout w;
    size_t off = 0;
    w.t_lse2 = off;
    off = align_up(off + 8 * rows_t);
    w.t_logp2 = off;
    off = align_up(off + 8 * n);
    w.t_h = off;
    off = align_up(off + 4 * rows_t);
    w.t_am = off;
    off = align_up(off + 4 * rows_t);
    w.dstats = off;
    off = align_up(off + 24 * n);
    w.cand = off;
    off = align_up(off + sizeof(RaceCand) * static_cast<size_t>(B) * race_segments(B, V));
    w.bonus_cnt = off;
    off = align_up(off + 4 * static_cast<size_t>(B));
    w.bonus_list = off;
    off = align_up(off + sizeof(int2) * kMaxBonusCand * static_cast<size_t>(B));
    w.total = off;
    return w;
}

// Draft-statistics buffer views (see spec_draft_stats_bytes).
struct DraftStats {
    double *lse2, *logq2;
    float *qmax, *feat;
};
DraftStats draft_stats_view(void *p, size_t n) {
    char *c = static_cast<char *>(p);
    return DraftStats{reinterpret_cast<double *>(c), reinterpret_cast<double *>(c + 8 * n),
                      reinterpret_cast<float *>(c + 16 * n), reinterpret_cast<float *>(c + 20 * n)};
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

spec_status check_logits_shape(int32_t V, int64_t stride, int32_t dtype, float temperature) {
    if (dtype != SPEC_DTYPE_F32 && dtype != SPEC_DTYPE_BF16) return SPEC_ERR_ARG;
    if (V < 2 || stride < V) return SPEC_ERR_ARG;
    if ((stride * elem_size(dtype)) % 16 != 0) return SPEC_ERR_ARG;
    // rows are addressed with 32-bit byte offsets
    if (static_cast<int64_t>(V) * elem_size(dtype) > INT32_MAX) return SPEC_ERR_UNSUPPORTED;
    if (!(temperature >= 1e-4f && temperature <= 1e4f)) return SPEC_ERR_ARG;
    return SPEC_OK;
}

spec_status check_params(const spec_params *p) {
    if (!p) return SPEC_ERR_ARG;
    if (p->batch < 0 || p->num_draft < 1 || p->reserved != 0) return SPEC_ERR_ARG;
    if (p->num_draft > 64) return SPEC_ERR_UNSUPPORTED;
    const spec_status s = check_logits_shape(p->vocab, p->row_stride, p->dtype, p->temperature);
    if (s != SPEC_OK) return s;
    // all row indices and b*(K+1)+j products must fit in int32
    if (static_cast<int64_t>(p->batch) * (2 * p->num_draft + 1) > INT32_MAX) return SPEC_ERR_UNSUPPORTED;
    return SPEC_OK;
}

spec_status launch_status() {
    return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

// ---------------------------------------------------------------------------
// Row-pass dispatch over (dtype, entropy for group 0).  Group 1 (draft rows)
// never needs the entropy numerator.
// ---------------------------------------------------------------------------
template <typename T, bool E0, bool CAND>
void launch_rows_t(const RowArgs &a, int nblocks, bool trimmed, hipStream_t st) {
    constexpr int kBlock = row_block<T>();
    constexpr int kTrimmed = kRowBlockTrimmed;
    if (trimmed && kTrimmed != kBlock)
        row_stats_kernel<T, kTrimmed, RowUnroll<T>::value, E0, CAND>
            <<<dim3(nblocks), dim3(kTrimmed), 0, st>>>(a);
    else
        row_stats_kernel<T, kBlock, RowUnroll<T>::value, E0, CAND>
            <<<dim3(nblocks), dim3(kBlock), 0, st>>>(a);
}

template <typename T>
void launch_rows_dt(const RowArgs &a, int nblocks, bool e0, bool cand, bool trimmed,
                    hipStream_t st) {
    if (cand) {
        if (e0)
            launch_rows_t<T, true, true>(a, nblocks, trimmed, st);
        else
            launch_rows_t<T, false, true>(a, nblocks, trimmed, st);
    } else {
        if (e0)
            launch_rows_t<T, true, false>(a, nblocks, trimmed, st);
        else
            launch_rows_t<T, false, false>(a, nblocks, trimmed, st);
    }
}

// cand: group 0 holds a lossless call's target rows, which also list the
// bonus candidates (a.seed, a.cand_cnt, a.cand_list set).  trimmed: a launch
// with kept lengths over target rows alone (see kRowBlockTrimmed).
void launch_rows(int32_t dtype, const RowArgs &a, int nblocks, bool e0, hipStream_t st,
                 bool cand = false, bool trimmed = false) {
    if (nblocks <= 0) return;
    if (dtype == SPEC_DTYPE_BF16)
        launch_rows_dt<uint16_t>(a, nblocks, e0, cand, trimmed, st);
    else
        launch_rows_dt<float>(a, nblocks, e0, cand, trimmed, st);
}

RowGroup empty_group() {
    RowGroup g{};
    g.rows_per_seq = 1;
    return g;
}

float log2e_over(float temperature) { return kLog2e / temperature; }

}  // namespace

extern "C" {

const char *spec_status_string(int32_t status) {
    switch (status) {
        case SPEC_OK: return "ok";
        case SPEC_ERR_ARG: return "invalid argument";
        case SPEC_ERR_UNSUPPORTED: return "unsupported configuration";
        case SPEC_ERR_WORKSPACE: return "workspace missing or too small";
        case SPEC_ERR_HIP: return "HIP launch failed";
        default: return "unknown status";
    }
}

size_t spec_workspace_bytes(const spec_params *p) {
    if (check_params(p) != SPEC_OK) return 0;
    return layout_for(p->batch, p->num_draft, p->vocab).total;
}

size_t spec_draft_stats_bytes(int32_t batch, int32_t num_draft) {
    if (batch < 0 || num_draft < 1) return 0;
    return 24 * static_cast<size_t>(batch) * static_cast<size_t>(num_draft);
}

// spec_verify, and with upd the step's update in its last launch.
static spec_status verify_impl(const void *target, const void *draft, const int32_t *draft_tokens,
                               const int32_t *kept_len, const void *draft_stats, uint64_t seed,
                               int32_t mode, const spec_params *params,
                               const spec_verify_out *out, void *workspace,
                               size_t workspace_bytes, void *stream, StepUpdate *upd) {
    spec_status s = check_params(params);
    if (s != SPEC_OK) return s;
    if (mode != SPEC_MODE_LOSSLESS && mode != SPEC_MODE_FLY) return SPEC_ERR_ARG;
    if (!out) return SPEC_ERR_ARG;
    const spec_params &p = *params;
    if (mode == SPEC_MODE_FLY && (p.fly_window < 0 || p.fly_window > (1 << 20) ||
                                  std::isnan(p.fly_theta)))
        return SPEC_ERR_ARG;
    if (p.batch == 0) return SPEC_OK;
    if (!target || !aligned16(target) || !draft_tokens || !out->accepted_len || !out->tokens)
        return SPEC_ERR_ARG;
    const bool lossless = mode == SPEC_MODE_LOSSLESS;
    const bool own_draft = lossless && draft_stats == nullptr;
    // Lossless mode re-reads the draft row of a rejected position, so the
    // draft logits are needed even when their statistics are supplied.
    if (lossless && (!draft || !aligned16(draft))) return SPEC_ERR_ARG;
    if (draft_stats && !aligned16(draft_stats)) return SPEC_ERR_ARG;
    const int32_t B = p.batch, K = p.num_draft, V = p.vocab;
    const WsLayout ws = layout_for(B, K, V);
    if (!workspace || workspace_bytes < ws.total) return SPEC_ERR_WORKSPACE;
    if (!aligned16(workspace)) return SPEC_ERR_ARG;

    hipStream_t st = static_cast<hipStream_t>(stream);
    char *w = static_cast<char *>(workspace);
    double *t_lse2 = reinterpret_cast<double *>(w + ws.t_lse2);
    double *t_logp2 = reinterpret_cast<double *>(w + ws.t_logp2);
    float *t_h = reinterpret_cast<float *>(w + ws.t_h);
    int32_t *t_am = reinterpret_cast<int32_t *>(w + ws.t_am);
    const size_t n = static_cast<size_t>(B) * K;
    if (out->draft_stats_out && !aligned16(out->draft_stats_out)) return SPEC_ERR_ARG;
    void *own_stats = out->draft_stats_out ? out->draft_stats_out : static_cast<void *>(w + ws.dstats);
    DraftStats ds =
        draft_stats_view(own_draft ? own_stats : const_cast<void *>(draft_stats), n);

    const float c = log2e_over(p.temperature);
    RowArgs ra{};
    RowGroup &gt = ra.g[0];
    gt.base = target;
    gt.stride = p.row_stride;
    gt.rows_per_seq = K + 1;
    gt.active_extra = 1;
    gt.gather_rows = lossless ? K : 0;
    gt.lse = out->target_lse;
    gt.entropy = out->target_entropy;
    gt.argmax = out->target_argmax;
    gt.lse2 = lossless ? t_lse2 : nullptr;  // the FLy resolver reads only h and the top token
    gt.logtok2 = t_logp2;
    gt.h_int = t_h;
    gt.am_int = t_am;
    RowGroup &gd = ra.g[1];
    gd = empty_group();
    if (own_draft) {
        gd.base = draft;
        gd.stride = p.row_stride;
        gd.rows_per_seq = K;
        gd.active_extra = 0;
        gd.gather_rows = K;
        gd.lse = out->draft_lse;
        gd.qmax = out->draft_qmax;
        gd.feat = out->draft_feat;
        gd.lse2 = ds.lse2;
        gd.logtok2 = ds.logq2;
        gd.qmax_int = ds.qmax;
        gd.feat_int = ds.feat;
    }
    ra.nrows0 = B * (K + 1);
    ra.V = V;
    ra.K = K;
    ra.tokens = draft_tokens;
    ra.kept_len = kept_len;
    ra.c = c;
    ra.inv_ln_v = 1.0 / std::log(static_cast<double>(V));
    const int nrows = ra.nrows0 + (own_draft ? B * K : 0);
    const bool ent0 = !lossless || out->target_entropy != nullptr;
    int32_t *bonus_cnt = reinterpret_cast<int32_t *>(w + ws.bonus_cnt);
    int2 *bonus_list = reinterpret_cast<int2 *>(w + ws.bonus_list);
    if (lossless) {
        ra.seed = seed;
        ra.cand_cnt = bonus_cnt;
        ra.cand_list = bonus_list;
    }
    launch_rows(p.dtype, ra, nrows, ent0, st, lossless, kept_len != nullptr && !own_draft);
    if ((s = launch_status()) != SPEC_OK) return s;

    if (!lossless) {
        constexpr int seqs_per_block = kFlyBlock / kWave;
        fly_kernel<kFlyBlock><<<dim3((B + seqs_per_block - 1) / seqs_per_block), dim3(kFlyBlock), 0,
                                st>>>(
            draft_tokens, kept_len, t_am, t_h, B, K, p.fly_theta, p.fly_window,
            out->accepted_len, out->tokens, out->boundary);
        return launch_status();
    }

    RaceArgs rg{};
    rg.target = target;
    rg.draft = draft;
    rg.stride = p.row_stride;
    rg.V = V;
    rg.K = K;
    rg.kept_len = kept_len;
    rg.t_lse2 = t_lse2;
    rg.t_logp2 = t_logp2;
    rg.d_lse2 = ds.lse2;
    rg.d_logq2 = ds.logq2;
    rg.t_am = t_am;
    rg.c = c;
    rg.inv_t = 1.0 / static_cast<double>(p.temperature);
    rg.seed = seed;
    rg.segs = race_segments(B, V);
    const int ngroups = (V + kRaceGroup - 1) / kRaceGroup;
    rg.seg_groups = (ngroups + rg.segs - 1) / rg.segs;
    rg.cand = reinterpret_cast<RaceCand *>(w + ws.cand);
    rg.bonus_cnt = bonus_cnt;
    rg.bonus_list = bonus_list;
    const dim3 grid(static_cast<unsigned>(rg.segs) * static_cast<unsigned>(B));
    const bool bf16 = p.dtype == SPEC_DTYPE_BF16;
    if (bf16)
        race_kernel<uint16_t, kRaceBlock><<<grid, dim3(kRaceBlock), 0, st>>>(rg);
    else
        race_kernel<float, kRaceBlock><<<grid, dim3(kRaceBlock), 0, st>>>(rg);
    if (upd) {
        // the tokens and the update in one launch: a workgroup per kStepSeqs
        // sequences, then one for the update
        upd->feat = ds.feat;
        upd->B = B;
        const dim3 sgrid(static_cast<unsigned>((B + kStepSeqs - 1) / kStepSeqs + 1));
        if (bf16)
            race_step_kernel<uint16_t, kLabelBlock><<<sgrid, dim3(kLabelBlock), 0, st>>>(
                rg, draft_tokens, out->accepted_len, out->tokens, out->boundary, *upd);
        else
            race_step_kernel<float, kLabelBlock><<<sgrid, dim3(kLabelBlock), 0, st>>>(
                rg, draft_tokens, out->accepted_len, out->tokens, out->boundary, *upd);
    } else if (bf16) {
        race_combine_kernel<uint16_t, kSmallBlock><<<dim3(B), dim3(kSmallBlock), 0, st>>>(
            rg, draft_tokens, out->accepted_len, out->tokens, out->boundary);
    } else {
        race_combine_kernel<float, kSmallBlock><<<dim3(B), dim3(kSmallBlock), 0, st>>>(
            rg, draft_tokens, out->accepted_len, out->tokens, out->boundary);
    }
    return launch_status();
}

spec_status spec_verify(const void *target, const void *draft, const int32_t *draft_tokens,
                        const int32_t *kept_len, const void *draft_stats, uint64_t seed,
                        int32_t mode, const spec_params *params, const spec_verify_out *out,
                        void *workspace, size_t workspace_bytes, void *stream) {
    return verify_impl(target, draft, draft_tokens, kept_len, draft_stats, seed, mode, params, out,
                       workspace, workspace_bytes, stream, nullptr);
}

spec_status spec_verify_update(const void *target, const void *draft, const int32_t *draft_tokens,
                               const int32_t *kept_len, const void *draft_stats, uint64_t seed,
                               const spec_params *params, const spec_verify_out *out, float lr,
                               float *omega_beta, float *conf, uint8_t *keep_mask,
                               int32_t *kept_len_out, void *workspace, size_t workspace_bytes,
                               void *stream) {
    const bool score = conf || keep_mask || kept_len_out;
    if (!std::isfinite(lr)) return SPEC_ERR_ARG;
    if (score && (kept_len || draft_stats)) return SPEC_ERR_ARG;  // scores need an untrimmed step
    if (params && params->batch > 0 && !omega_beta) return SPEC_ERR_ARG;
    StepUpdate u{};
    u.kept_len = kept_len;
    u.omega_beta = omega_beta;
    u.conf = conf;
    u.keep_mask = keep_mask;
    u.kept_out = kept_len_out;
    u.lr = lr;
    u.score = score ? 1 : 0;
    return verify_impl(target, draft, draft_tokens, kept_len, draft_stats, seed,
                       SPEC_MODE_LOSSLESS, params, out, workspace, workspace_bytes, stream, &u);
}

spec_status spec_av_score(const void *draft, const int32_t *draft_tokens,
                          const spec_params *params, const float *omega_beta, float tau,
                          float *conf, uint8_t *keep_mask, int32_t *kept_len, void *draft_stats,
                          void *stream) {
    spec_status s = check_params(params);
    if (s != SPEC_OK) return s;
    const spec_params &p = *params;
    if (std::isnan(tau)) return SPEC_ERR_ARG;
    if (p.batch == 0) return SPEC_OK;
    if (!draft || !aligned16(draft) || !draft_tokens || !omega_beta || !draft_stats ||
        !aligned16(draft_stats))
        return SPEC_ERR_ARG;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int32_t B = p.batch, K = p.num_draft;
    const size_t n = static_cast<size_t>(B) * K;
    DraftStats ds = draft_stats_view(draft_stats, n);
    RowArgs ra{};
    RowGroup &gd = ra.g[0];
    gd.base = draft;
    gd.stride = p.row_stride;
    gd.rows_per_seq = K;
    gd.active_extra = 0;
    gd.gather_rows = K;
    gd.lse2 = ds.lse2;
    gd.logtok2 = ds.logq2;
    gd.qmax_int = ds.qmax;
    gd.feat_int = ds.feat;
    ra.g[1] = empty_group();
    ra.nrows0 = B * K;
    ra.V = p.vocab;
    ra.K = K;
    ra.tokens = draft_tokens;
    ra.kept_len = nullptr;
    ra.c = log2e_over(p.temperature);
    ra.inv_ln_v = 1.0 / std::log(static_cast<double>(p.vocab));
    launch_rows(p.dtype, ra, B * K, false, st);
    if ((s = launch_status()) != SPEC_OK) return s;
    av_score_kernel<<<dim3((B + kSmallBlock - 1) / kSmallBlock), dim3(kSmallBlock), 0, st>>>(
        ds.feat, B, K, omega_beta, tau, conf, keep_mask, kept_len);
    return launch_status();
}

spec_status spec_av_score_prefix(const void *draft, const int32_t *draft_tokens,
                                 const spec_params *params, const float *omega_beta, float tau,
                                 float *conf, uint8_t *keep_mask, int32_t *kept_len,
                                 void *draft_stats, void *stream) {
    spec_status s = check_params(params);
    if (s != SPEC_OK) return s;
    const spec_params &p = *params;
    if (std::isnan(tau)) return SPEC_ERR_ARG;
    if (p.batch == 0) return SPEC_OK;
    if (!draft || !aligned16(draft) || !draft_tokens || !omega_beta || !draft_stats ||
        !aligned16(draft_stats))
        return SPEC_ERR_ARG;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int32_t B = p.batch, K = p.num_draft;
    const size_t n = static_cast<size_t>(B) * K;
    DraftStats ds = draft_stats_view(draft_stats, n);
    PrefixArgs pa{};
    pa.draft = draft;
    pa.stride = p.row_stride;
    pa.V = p.vocab;
    pa.K = K;
    pa.tokens = draft_tokens;
    pa.c = log2e_over(p.temperature);
    pa.inv_ln_v = 1.0 / std::log(static_cast<double>(p.vocab));
    pa.lse2 = ds.lse2;
    pa.logq2 = ds.logq2;
    pa.qmax = ds.qmax;
    pa.feat = ds.feat;
    if (p.dtype == SPEC_DTYPE_BF16)
        av_prefix_kernel<uint16_t, row_block<uint16_t>(), RowUnroll<uint16_t>::value>
            <<<dim3(B), dim3(row_block<uint16_t>()), 0, st>>>(pa, omega_beta, tau, conf, keep_mask,
                                                              kept_len);
    else
        av_prefix_kernel<float, row_block<float>(), RowUnroll<float>::value>
            <<<dim3(B), dim3(row_block<float>()), 0, st>>>(pa, omega_beta, tau, conf, keep_mask,
                                                           kept_len);
    return launch_status();
}

spec_status spec_av_score_stats(const void *draft_stats, int32_t batch, int32_t num_draft,
                                const float *omega_beta, float tau, float *conf,
                                uint8_t *keep_mask, int32_t *kept_len, void *stream) {
    if (batch < 0 || num_draft < 1) return SPEC_ERR_ARG;
    if (num_draft > 64) return SPEC_ERR_UNSUPPORTED;
    if (std::isnan(tau)) return SPEC_ERR_ARG;
    if (batch == 0) return SPEC_OK;
    if (!draft_stats || !aligned16(draft_stats) || !omega_beta) return SPEC_ERR_ARG;
    const size_t n = static_cast<size_t>(batch) * num_draft;
    DraftStats ds = draft_stats_view(const_cast<void *>(draft_stats), n);
    av_score_kernel<<<dim3((batch + kSmallBlock - 1) / kSmallBlock), dim3(kSmallBlock), 0,
                      static_cast<hipStream_t>(stream)>>>(ds.feat, batch, num_draft, omega_beta,
                                                         tau, conf, keep_mask, kept_len);
    return launch_status();
}

spec_status spec_av_score_update(const void *draft_stats, const int32_t *accepted_len,
                                 int32_t batch, int32_t num_draft, float lr, float *omega_beta,
                                 float *conf, uint8_t *keep_mask, int32_t *kept_len,
                                 void *stream) {
    if (batch < 0 || num_draft < 1) return SPEC_ERR_ARG;
    if (num_draft > 64) return SPEC_ERR_UNSUPPORTED;
    if (!std::isfinite(lr)) return SPEC_ERR_ARG;
    if (batch == 0) return SPEC_OK;
    if (!draft_stats || !aligned16(draft_stats) || !accepted_len || !omega_beta)
        return SPEC_ERR_ARG;
    const size_t n = static_cast<size_t>(batch) * num_draft;
    DraftStats ds = draft_stats_view(const_cast<void *>(draft_stats), n);
    av_score_update_kernel<kLabelBlock>
        <<<dim3(1), dim3(kLabelBlock), 0, static_cast<hipStream_t>(stream)>>>(
            ds.feat, accepted_len, batch, num_draft, lr, omega_beta, conf, keep_mask, kept_len);
    return launch_status();
}

spec_status spec_av_update(const void *draft_stats, const int32_t *accepted_len,
                           const int32_t *kept_len, int32_t batch, int32_t num_draft, float lr,
                           float *omega_beta, void *stream) {
    if (batch < 0 || num_draft < 1) return SPEC_ERR_ARG;
    if (num_draft > 64) return SPEC_ERR_UNSUPPORTED;
    if (!std::isfinite(lr)) return SPEC_ERR_ARG;
    if (batch == 0) return SPEC_OK;
    if (!draft_stats || !aligned16(draft_stats) || !accepted_len || !omega_beta)
        return SPEC_ERR_ARG;
    const size_t n = static_cast<size_t>(batch) * num_draft;
    DraftStats ds = draft_stats_view(const_cast<void *>(draft_stats), n);
    av_sgd_kernel<kLabelBlock><<<dim3(1), dim3(kLabelBlock), 0, static_cast<hipStream_t>(stream)>>>(
        ds.feat, accepted_len, kept_len, batch, num_draft, lr, omega_beta);
    return launch_status();
}

size_t spec_irls_state_bytes(int32_t num_draft) {
    if (num_draft < 1 || num_draft > 64) return 0;
    return sizeof(double) * static_cast<size_t>(irls_state_doubles(num_draft));
}

spec_status spec_irls_reset(void *state, int32_t num_draft, void *stream) {
    if (num_draft < 1) return SPEC_ERR_ARG;
    if (num_draft > 64) return SPEC_ERR_UNSUPPORTED;
    if (!state || (reinterpret_cast<uintptr_t>(state) & 7u)) return SPEC_ERR_ARG;
    const int nd = irls_state_doubles(num_draft);
    fill_f64_kernel<<<dim3((nd + 255) / 256), dim3(256), 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<double *>(state), nd, 0.0);
    return launch_status();
}

spec_status spec_irls_accumulate(const void *draft_stats, const int32_t *accepted_len,
                                 const int32_t *kept_len, int32_t batch, int32_t num_draft,
                                 const float *omega_beta, void *state, void *stream) {
    if (batch < 0 || num_draft < 1) return SPEC_ERR_ARG;
    if (num_draft > 64) return SPEC_ERR_UNSUPPORTED;
    if (batch == 0) return SPEC_OK;
    if (!draft_stats || !aligned16(draft_stats) || !accepted_len || !omega_beta || !state ||
        (reinterpret_cast<uintptr_t>(state) & 7u))
        return SPEC_ERR_ARG;
    const size_t n = static_cast<size_t>(batch) * num_draft;
    DraftStats ds = draft_stats_view(const_cast<void *>(draft_stats), n);
    irls_accumulate_kernel<kLabelBlock>
        <<<dim3(1), dim3(kLabelBlock), 0, static_cast<hipStream_t>(stream)>>>(
            ds.feat, accepted_len, kept_len, batch, num_draft, omega_beta,
            static_cast<double *>(state));
    return launch_status();
}

spec_status spec_irls_solve(void *state, int32_t num_draft, double c_damp, float *omega_beta,
                            int32_t *flags, void *stream) {
    if (num_draft < 1) return SPEC_ERR_ARG;
    if (num_draft > 64) return SPEC_ERR_UNSUPPORTED;
    if (!(c_damp >= 0.0) || !std::isfinite(c_damp)) return SPEC_ERR_ARG;
    if (!state || (reinterpret_cast<uintptr_t>(state) & 7u) || !omega_beta) return SPEC_ERR_ARG;
    irls_solve_kernel<<<dim3(1), dim3(kWave), 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<double *>(state), num_draft, c_damp, omega_beta, flags);
    return launch_status();
}

namespace {
struct DiagLayout {
    size_t zpos, zneg, cnt, loss, bins, pairs, total;
    int regions;
};
DiagLayout diag_layout(int32_t B, int32_t K, int32_t nbins) {
    DiagLayout l{};
    const size_t M = static_cast<size_t>(B) * K;
    l.regions = static_cast<int>((M + kDiagTile - 1) / kDiagTile);
    const size_t R = static_cast<size_t>(l.regions);
    l.zpos = 0;
    l.zneg = align_up(8 * R * kDiagTile);
    l.cnt = align_up(l.zneg + 8 * R * kDiagTile);
    l.loss = align_up(l.cnt + 8 * R);
    l.bins = align_up(l.loss + 8 * R);
    l.pairs = align_up(l.bins + 8 * R * static_cast<size_t>(nbins));
    l.total = align_up(l.pairs + 8 * R * R);
    return l;
}
}  // namespace

size_t spec_av_diagnostics_workspace_bytes(int32_t batch, int32_t num_draft, int32_t nbins) {
    if (batch < 1 || num_draft < 1 || num_draft > 64 || nbins < 1 || nbins > kDiagMaxBins ||
        static_cast<int64_t>(batch) * num_draft > kDiagMaxLabels)
        return 0;
    return diag_layout(batch, num_draft, nbins).total;
}

spec_status spec_av_diagnostics(const void *draft_stats, const int32_t *accepted_len,
                                const int32_t *kept_len, int32_t batch, int32_t num_draft,
                                const float *omega_beta, int32_t nbins, double *out,
                                void *workspace, size_t workspace_bytes, void *stream) {
    if (batch < 1 || num_draft < 1 || nbins < 1) return SPEC_ERR_ARG;
    if (num_draft > 64 || nbins > kDiagMaxBins ||
        static_cast<int64_t>(batch) * num_draft > kDiagMaxLabels)
        return SPEC_ERR_UNSUPPORTED;
    if (!draft_stats || !aligned16(draft_stats) || !accepted_len || !omega_beta || !out ||
        (reinterpret_cast<uintptr_t>(out) & 7u))
        return SPEC_ERR_ARG;
    const DiagLayout l = diag_layout(batch, num_draft, nbins);
    if (!workspace || workspace_bytes < l.total) return SPEC_ERR_WORKSPACE;
    if (!aligned16(workspace)) return SPEC_ERR_ARG;
    char *w = static_cast<char *>(workspace);
    DiagWs ws{reinterpret_cast<double *>(w + l.zpos), reinterpret_cast<double *>(w + l.zneg),
              reinterpret_cast<int32_t *>(w + l.cnt),
              reinterpret_cast<unsigned long long *>(w + l.loss),
              reinterpret_cast<unsigned long long *>(w + l.bins),
              reinterpret_cast<unsigned long long *>(w + l.pairs)};
    const size_t n = static_cast<size_t>(batch) * num_draft;
    DraftStats ds = draft_stats_view(const_cast<void *>(draft_stats), n);
    hipStream_t st = static_cast<hipStream_t>(stream);
    diag_labels_kernel<<<dim3(l.regions), dim3(kDiagTile), 0, st>>>(
        ds.feat, accepted_len, kept_len, batch, num_draft, omega_beta, nbins, ws);
    diag_pairs_kernel<<<dim3(l.regions * l.regions), dim3(kDiagTile), 0, st>>>(ws, l.regions);
    diag_finish_kernel<<<dim3(1), dim3(kWave), 0, st>>>(ws, l.regions, nbins, out);
    return launch_status();
}

namespace {
struct BudgetLayout {
    size_t counts, sorted_s, sorted_e, total;
    int tiles;
};
BudgetLayout budget_layout(int32_t B, int32_t K) {
    BudgetLayout l{};
    const size_t M = static_cast<size_t>(B) * K;
    l.tiles = static_cast<int>((M + kBudgetTile - 1) / kBudgetTile);
    l.counts = 0;
    l.sorted_s = align_up(l.counts + 2 * M * static_cast<size_t>(l.tiles));
    l.sorted_e = align_up(l.sorted_s + 4 * M);
    l.total = align_up(l.sorted_e + 4 * M);
    return l;
}
}  // namespace

size_t spec_av_budget_workspace_bytes(int32_t batch, int32_t num_draft) {
    if (batch < 1 || num_draft < 1 || static_cast<int64_t>(batch) * num_draft > kBudgetMax)
        return 0;
    return budget_layout(batch, num_draft).total;
}

spec_status spec_av_budget(const float *conf, int32_t batch, int32_t num_draft, const double *cost,
                           double n_requests, int32_t *kept_len, uint8_t *keep_mask,
                           int64_t *budget, double *best_ratio, void *workspace,
                           size_t workspace_bytes, void *stream) {
    if (batch < 1 || num_draft < 1 || !std::isfinite(n_requests)) return SPEC_ERR_ARG;
    const int64_t M = static_cast<int64_t>(batch) * num_draft;
    if (M > kBudgetMax) return SPEC_ERR_UNSUPPORTED;
    if (!conf || !cost || !kept_len || !budget || (reinterpret_cast<uintptr_t>(cost) & 7u) ||
        (reinterpret_cast<uintptr_t>(budget) & 7u) ||
        (best_ratio && (reinterpret_cast<uintptr_t>(best_ratio) & 7u)))
        return SPEC_ERR_ARG;
    const BudgetLayout l = budget_layout(batch, num_draft);
    if (!workspace || workspace_bytes < l.total) return SPEC_ERR_WORKSPACE;
    if (!aligned16(workspace)) return SPEC_ERR_ARG;
    char *w = static_cast<char *>(workspace);
    BudgetWs ws{reinterpret_cast<uint16_t *>(w + l.counts), reinterpret_cast<float *>(w + l.sorted_s),
                reinterpret_cast<int32_t *>(w + l.sorted_e)};
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int m = static_cast<int>(M);
    budget_rank_kernel<<<dim3(l.tiles * l.tiles), dim3(kBudgetTile), 0, st>>>(conf, num_draft, ws,
                                                                            m, l.tiles);
    budget_scatter_kernel<<<dim3((m + 255) / 256), dim3(256), 0, st>>>(conf, num_draft, ws, m,
                                                                     l.tiles);
    budget_finish_kernel<kBudgetThreads><<<dim3(1), dim3(kBudgetThreads), 0, st>>>(
        ws, batch, num_draft, cost, n_requests, kept_len, keep_mask, budget, best_ratio);
    return launch_status();
}

spec_status spec_ngram_propose(const int32_t *context, const int32_t *lengths, int32_t batch,
                               int64_t stride, int32_t n_min, int32_t n_max, int32_t num_draft,
                               int32_t *draft, int32_t *draft_len, int32_t *match_pos,
                               int32_t *match_n, void *stream) {
    if (batch < 0 || stride < 1 || n_min < 1 || n_max < n_min || num_draft < 1) return SPEC_ERR_ARG;
    if (n_max > kNgramMax || stride > INT32_MAX || num_draft > 64) return SPEC_ERR_UNSUPPORTED;
    if (batch == 0) return SPEC_OK;
    if (!context || !lengths || !draft || !draft_len) return SPEC_ERR_ARG;
    ngram_kernel<kNgramBlock, kNgramUnroll><<<dim3(batch), dim3(kNgramBlock), 0, static_cast<hipStream_t>(stream)>>>(
        context, lengths, stride, n_min, n_max, num_draft, draft, draft_len, match_pos, match_n);
    return launch_status();
}

spec_status spec_row_stats(const void *logits, int64_t rows, int32_t vocab, int64_t row_stride,
                           int32_t dtype, float temperature, float *lse, float *entropy,
                           int32_t *argmax, float *qmax, float *feat, void *stream) {
    spec_status s = check_logits_shape(vocab, row_stride, dtype, temperature);
    if (s != SPEC_OK) return s;
    if (rows < 0) return SPEC_ERR_ARG;
    if (rows > INT32_MAX) return SPEC_ERR_UNSUPPORTED;
    if (rows == 0) return SPEC_OK;
    if (!logits || !aligned16(logits)) return SPEC_ERR_ARG;
    RowArgs ra{};
    RowGroup &g = ra.g[0];
    g.base = logits;
    g.stride = row_stride;
    g.rows_per_seq = static_cast<int32_t>(rows);
    g.active_extra = 0;
    g.gather_rows = 0;
    g.lse = lse;
    g.entropy = entropy;
    g.argmax = argmax;
    g.qmax = qmax;
    g.feat = feat;
    ra.g[1] = empty_group();
    ra.nrows0 = static_cast<int32_t>(rows);
    ra.V = vocab;
    ra.K = 1;
    ra.c = log2e_over(temperature);
    ra.inv_ln_v = 1.0 / std::log(static_cast<double>(vocab));
    launch_rows(dtype, ra, static_cast<int>(rows), entropy != nullptr,
                static_cast<hipStream_t>(stream));
    return launch_status();
}

spec_status spec_read_probe(const void *logits, int64_t rows, int64_t row_bytes,
                            int64_t row_stride_bytes, uint32_t *sink, void *stream) {
    if (rows < 0 || row_bytes < 0 || row_bytes % 16 != 0 || row_stride_bytes % 16 != 0 ||
        row_bytes > row_stride_bytes)
        return SPEC_ERR_ARG;
    if (rows > INT32_MAX || row_bytes > INT32_MAX) return SPEC_ERR_UNSUPPORTED;
    if (rows == 0) return SPEC_OK;
    if (!logits || !aligned16(logits) || !sink) return SPEC_ERR_ARG;
    read_probe_kernel<kRowBlockBf16, RowUnroll<uint16_t>::value>
        <<<dim3(static_cast<unsigned>(rows)), dim3(kRowBlockBf16), 0,
           static_cast<hipStream_t>(stream)>>>(
            logits, row_bytes / 16, row_stride_bytes / 16, sink);
    return launch_status();
}

}  // extern "C"
