// sv_rowstats.hpp -- the streaming row pass: one workgroup per logits row,
// 16-byte loads, a single pass with an online (max, sum, entropy numerator,
// argmax) state per thread, then a short epilogue of DPP wave reductions and
// one LDS exchange.
//
// Per row it yields the quantities the verification rules read: the
// log-normaliser, the normalised entropy h = H(p)/log V that the FLy gate
// compares with theta (page "Training-Free Loosely Speculative Decoding...",
// section "2. Metodologia", part A), the top token, the probability of the
// drafted token, and q_max with its log-odds logit(q_max), the feature of the
// adaptive-verification estimator (page "Verificacion Adaptativa sin una
// cabeza de confianza", section "Puntuar la Distribucion").
//
// Rows are streamed with non-temporal 16-byte buffer loads.
//
// In a lossless call the target row L_b of each sequence (the only row where a
// draw from p can happen) also lists the ids such a draw could pick, so that
// the race need not read that row again (see row_one, CAND).
//
// Arithmetic is in base 2: with c = log2(e)/T every term is 2^(l*c - mc),
// where mc = m*c and m is the running maximum of the raw logits.  A thread
// reads its share of the row in chunks of UNROLL vectors (UNROLL*8 bfloat16
// or UNROLL*4 float logits); the sums within a thread and within a wave are
// float (every term has one sign), the sums across waves double.  Each
// thread keeps the chunk that holds its maximum apart (its sums in registers,
// its raw data in LDS), so the end can replace that chunk by its terms other
// than the argmax and form 1 - q_max without cancellation, however peaked the
// row.
#pragma once

#include "sv_common.hpp"
#include "sv_philox.hpp"

namespace sv {

// A count of vectors as a type (the row pass's chunk variants).
template <int NV>
struct Vecs {
    static constexpr int value = NV;
};

// Launch shape: threads per workgroup and 16-byte vectors per thread per
// chunk.  A chunk holds 16 bfloat16 or 16 float logits.  bfloat16 rows take
// 768-thread workgroups, two per compute unit (at the entropy variant's 76
// registers a SIMD holds six waves), which measured 1-1.5 % faster than 512
// threads on the bfloat16 passes that read every row; float rows keep 512.
// Every pass that reads draft rows takes its dtype's shape, so that draft
// statistics are the same bits whichever call produces them (the verify pass,
// the scorer's pass or the scorer's per-sequence prefix loop).
constexpr int kRowBlockF32 = 512;
constexpr int kRowBlockBf16 = 768;
template <typename T>
constexpr int row_block() {
    return sizeof(T) == 2 ? kRowBlockBf16 : kRowBlockF32;
}
// Launches with kept lengths that read target rows alone take 512 threads
// whatever the dtype: most of their workgroups (rows past a kept length) exit
// after one load, and the extra waves of a 768-thread workgroup make each
// such exit dearer (the adaptive pipeline's verify pass, 9216 workgroups of
// which ~7500 exit: 75-78 us at 512 threads against 83-85 us at 768).  No
// draft statistics come from such a launch.
constexpr int kRowBlockTrimmed = 512;
template <typename T>
struct RowUnroll;
template <>
struct RowUnroll<uint16_t> {
    static constexpr int value = 2;
};
template <>
struct RowUnroll<float> {
    static constexpr int value = 4;
};
// One group of rows processed by the same launch (target rows and draft rows
// share a launch).  Row j of sequence b is row b*rows_per_seq + j.
struct RowGroup {
    const void *base;
    int64_t stride;        // elements between consecutive rows
    int32_t rows_per_seq;  // K+1 target rows, K draft rows, or all rows
    int32_t active_extra;  // with kept_len: row j is read iff j < L_b + active_extra
    int32_t gather_rows;   // rows j < gather_rows gather tokens[b*K + j]
    int32_t pad_;
    // caller-visible results, one entry per row, each nullable
    float *lse;
    float *entropy;
    int32_t *argmax;
    float *qmax;
    float *feat;
    // internal results, nullable
    double *lse2;     // [rows] log2 normaliser: log2 sum_x 2^(l_x c)
    double *logtok2;  // [B*K]  log2 probability of the gathered token
    float *h_int;     // [rows]
    int32_t *am_int;  // [rows]
    float *qmax_int;  // [rows]
    float *feat_int;  // [rows]
};

struct RowArgs {
    RowGroup g[2];
    int32_t nrows0;  // workgroups 0..nrows0-1 serve group 0, the rest group 1
    int32_t V;
    int32_t K;
    int32_t pad_;
    const int32_t *tokens;    // [B][K] or null
    const int32_t *kept_len;  // [B] or null
    float c;                  // log2(e) / T
    float pad2_;
    double inv_ln_v;          // 1 / ln V
    // Bonus candidates (launches with CAND): for row L_b of sequence b, the
    // ids a race over p at that row could pick (see row_one).
    uint64_t seed;
    int32_t *cand_cnt;  // [B]: number of ids, or -1 when the list is not complete
    int2 *cand_list;    // [B][kMaxBonusCand]: (id, logit bits)
};

// Candidates are the ids whose l*c reaches the top token's race key less this
// (the race's largest gain from a uniform near 1, 23.47, plus both screening
// margins, rounded up).
constexpr float kBonusBelow = 24.0f;

// L_b: the verified drafts of sequence b (kept_len clamped to [0, K], or K).
__device__ __forceinline__ int kept_of(const RowArgs &a, int b) {
    return a.kept_len ? clamp_len(a.kept_len[b], a.K) : a.K;
}

// What a row that was not read reports.
__device__ __forceinline__ void write_unread(const RowGroup &g, int64_t row) {
    const float nan = __builtin_nanf("");
    if (g.lse) g.lse[row] = nan;
    if (g.entropy) g.entropy[row] = nan;
    if (g.argmax) g.argmax[row] = -1;
    if (g.qmax) g.qmax[row] = nan;
    if (g.feat) g.feat[row] = nan;
}

// The row's results from its maximum M, the first id P attaining it (INT_MAX
// when none), the sum r of 2^(l*c - Mc) over the other ids (Mc = M*c rounded
// to float) and the matching sum `to` of term * exponent.
template <bool ENT>
__device__ __forceinline__ void row_emit(const RowArgs &a, const RowGroup &g, int64_t row, float M,
                                         int P, double r, double to, bool gather, int gidx,
                                         float ltok) {
    const float c = a.c;
    const float Mc = mul_rn(M, c);
    // The argmax term is 2^r0 with r0 = M*c - Mc, the rounding residue of Mc
    // (exact in float); the row's sum of terms is 2^r0 + r.
    const double r0 = static_cast<double>(fmaf(M, c, -Mc));
    // 2^r0 and 2^-r0: the residue is tiny unless M*c is very large, and then
    // short series are exact to double rounding (the next term is below
    // 1e-26)
    const double xr = r0 * kLn2;
    double e0, ie0;
    if (fabs(r0) < 0x1p-16) {
        e0 = 1.0 + xr * (1.0 + xr * (0.5 + xr * (1.0 / 6.0 + xr * (1.0 / 24.0))));
        ie0 = 1.0 - xr * (1.0 - xr * (0.5 - xr * (1.0 / 6.0 - xr * (1.0 / 24.0))));
    } else {
        e0 = exp2(r0);
        ie0 = 1.0 / e0;
    }
    const double rho = r * ie0;     // (1 - q_max) / q_max
    const double l1p = log1p(rho);  // ln(sum / 2^r0)
    const double lse2 = static_cast<double>(Mc) + r0 + l1p * kLog2eD;
    if (g.lse2) g.lse2[row] = lse2;
    if (g.lse) g.lse[row] = static_cast<float>(lse2 * kLn2);
    const int am = P == INT_MAX ? -1 : P;
    if (g.argmax) g.argmax[row] = am;
    if (g.am_int) g.am_int[row] = am;
    // q_max = 1 / (1 + rho), the one division
    const bool want_q = g.qmax || g.qmax_int;
    const double inv1p = ENT || want_q ? 1.0 / (1.0 + rho) : 0.0;
    if (ENT) {
        // H = ln(sum) - ln2 * (sum of term*exponent) / sum, rewritten around
        // the argmax term: H = ln(1 + rho) + ln2 (r0 r - t_o) / (2^r0 + r)
        //                    = ln(1 + rho) + ln2 (r0 rho - t_o 2^-r0) q_max.
        const double H = l1p + kLn2 * (r0 * rho - to * ie0) * inv1p;
        const float h = static_cast<float>(H * a.inv_ln_v);
        if (g.entropy) g.entropy[row] = h;
        if (g.h_int) g.h_int[row] = h;
    }
    if (want_q) {
        const float qm = static_cast<float>(inv1p);
        if (g.qmax) g.qmax[row] = qm;
        if (g.qmax_int) g.qmax_int[row] = qm;
    }
    if (g.feat || g.feat_int) {
        const float ft = static_cast<float>(-log(fmax(rho, 0x1.0p-126)));  // logit(q_max)
        if (g.feat) g.feat[row] = ft;
        if (g.feat_int) g.feat_int[row] = ft;
    }
    if (gather && g.logtok2)
        g.logtok2[gidx] = static_cast<double>(ltok) * static_cast<double>(c) - lse2;
}

// row_emit for a row group that writes only the draft statistics (lse2,
// logtok2, qmax_int, feat_int), behind a call.  A kernel that runs row_one in
// a loop over rows calls this: inlined, the double-precision logarithm's and
// exponential's constants are hoisted out of that loop and each held in a
// register for the whole kernel (102 registers instead of 63), which halves
// the workgroups a compute unit holds.  Lane 0 alone makes the call, once per
// row.
__device__ __attribute__((noinline)) void row_emit_stats(float c, double *lse2, double *logtok2,
                                                         float *qmax_int, float *feat_int,
                                                         int64_t row, float M, int P, double r,
                                                         double to, bool gather, int gidx,
                                                         float ltok) {
    RowArgs a{};
    a.c = c;
    RowGroup g{};
    g.lse2 = lse2;
    g.logtok2 = logtok2;
    g.qmax_int = qmax_int;
    g.feat_int = feat_int;
    row_emit<false>(a, g, row, M, P, r, to, gather, gidx, ltok);
}

// CAND: target rows of a lossless call; row L_b of each sequence also lists
// the ids a race over p at that row could pick.  Each thread tracks, besides
// its max chunk (saved in LDS), the largest maximum m2 of its other chunks
// (one median-of-three per chunk): when no thread's m2 reaches the threshold,
// every candidate is in a saved max chunk; otherwise the list is marked
// incomplete and the race reads the row.
// tid: threadIdx.x (a caller that loops over rows passes it through an
// opaque copy, so that values derived from it are not kept live across rows).
// STATS_CALL: g writes only the draft statistics, emitted by row_emit_stats
// (for callers that loop over rows).
template <typename T, int BLOCK, int UNROLL, bool ENT, bool CAND, bool STATS_CALL = false>
__device__ __forceinline__ void row_one(const RowArgs &a, const RowGroup &g, int64_t row,
                                        uint4 (&sh_saved)[UNROLL][BLOCK], const int tid) {
    static_assert(!STATS_CALL || (!ENT && !CAND), "the statistics call emits a plain row");
    using E = Elem<T>;
    constexpr int EPV = E::kPerVec;
    constexpr int N = UNROLL * EPV;
    constexpr int NW = BLOCK / kWave;
    const int V = a.V;
    const float c = a.c;

    const int b = static_cast<int>(row / g.rows_per_seq);
    const int j = static_cast<int>(row - static_cast<int64_t>(b) * g.rows_per_seq);
    const int Lb = kept_of(a, b);
    if (a.kept_len && j >= Lb + g.active_extra) {  // trimmed away: report "not read"
        if (tid == 0) write_unread(g, row);
        return;
    }
    const T *rp = static_cast<const T *>(g.base) + row * g.stride;
    const bool gather = a.tokens != nullptr && j < g.gather_rows;
    const int gidx = b * a.K + j;
    float ltok = -__builtin_inff();
    if (gather && tid == 0) {
        const int x = a.tokens[gidx];
        if (x >= 0 && x < V) ltok = E::at(rp, x);
    }

    const int nfull = V / EPV;
    const int nvec = (V + EPV - 1) / EPV;

    // Thread state.  s, t: sums outside the chunk that holds the maximum;
    // cs, ct: that chunk's sums; itb: its index.  Its raw data is kept in
    // LDS (sh_saved), out of the registers.
    // A thread adds a few tens of chunk sums of one sign, so float carries
    // them to ~1e-6; the sums over threads are formed in double.
    float m = kNoMax, mc = mul_rn(kNoMax, c), cs = 0.f, ct = 0.f;
    float s = 0.f, t = 0.f;
    int itb = -1;
    float m2 = kNoMax;  // CAND: the largest maximum of the other chunks

    // it: the chunk's index; thread tid's chunk `it` starts at vector
    // it*UNROLL*BLOCK + tid.  nv (Vecs<NV>): the chunk's first NV vectors are
    // processed, NV < UNROLL only for a last chunk whose later vectors are
    // padding in every thread: padding's terms are exactly 0 and its value
    // lies below every maximum that can change the state, so leaving it out
    // gives the same bits.
    auto consume = [&](const uint4 (&buf)[UNROLL], int it, auto nv) {
        constexpr int NL = decltype(nv)::value * EPV;  // logits processed
        float x[N];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) E::unpack(buf[u], x + u * EPV);
        // the chunk maximum in a chain of three-input maxima
        float cm = max3f(x[0], x[1], x[2]);
#pragma unroll
        for (int k = 3; k + 1 < NL; k += 2) cm = max3f(cm, x[k], x[k + 1]);
        if (NL % 2 == 0) cm = max3f(cm, x[NL - 1], x[NL - 1]);
        const bool up = cm > m;
        const float mcn = up ? mul_rn(cm, c) : mc;
        // Terms of this chunk against the (possibly new) maximum.
        float s4[4], t4[4];
#pragma unroll
        for (int k = 0; k < NL; ++k) {
            const float d = fmaf(x[k], c, -mcn);
            const float e = hw_exp2(d);
            if (k < 4) {
                s4[k] = e;
                if (ENT) t4[k] = e * d;
            } else {
                s4[k & 3] += e;
                if (ENT) t4[k & 3] = fmaf(e, d, t4[k & 3]);
            }
        }
        const float csum = (s4[0] + s4[1]) + (s4[2] + s4[3]);
        float ctsum = 0.f;
        if (ENT) {
            ctsum = (t4[0] + t4[1]) + (t4[2] + t4[3]);
            // A -inf logit gives the term 0 * -inf = NaN; such chunks (masked
            // vocabulary, padding) are summed again with exponents clamped
            // where 2^d is zero anyway.
            if (!(ctsum == ctsum)) {
                ctsum = 0.f;
#pragma unroll
                for (int k = 0; k < NL; ++k) {
                    const float d = fmaxf(fmaf(x[k], c, -mcn), kMinExp2);
                    ctsum = fmaf(hw_exp2(d), d, ctsum);
                }
            }
        }
        // m2 = max(m2, the chunk that is not (or no longer) the max chunk):
        // with m2 <= m that is the median of (m2, cm, m)
        if (CAND) m2 = __builtin_amdgcn_fmed3f(m2, cm, m);
        if (up) {
            // A new thread maximum (rare after the first chunks): the old max
            // chunk joins the rest, which is rescaled to the new maximum by
            // 2^dl, and this chunk becomes the max chunk.
            const float dl = mc - mcn;
            const float al = hw_exp2(dl);
            const float stot = s + cs;
            if (ENT) t = al * (t + ct + dl * stot);
            s = al * stot;
            cs = csum;
            ct = ctsum;
            m = cm;
            mc = mcn;
            itb = it;
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) sh_saved[u][tid] = buf[u];
        } else {
            s += csum;
            if (ENT) t += ctsum;
        }
    };

    // Full chunks for every thread: a wave-uniform trip count and a uniform
    // base address, so the loop control and addressing stay scalar.
    constexpr int kChunkVecs = UNROLL * BLOCK;
    const int nit = nfull / kChunkVecs;
    // The next chunk's loads are issued before this chunk's arithmetic, so
    // every wave keeps a chunk in flight while it computes.
    // Loads are buffer-addressed over the row's full vectors: the chunk's
    // byte offset is wave-uniform (a scalar register), each lane's offset
    // inside the chunk is fixed.
    const buf_rsrc rs = make_rsrc(rp, static_cast<uint32_t>(nfull) * 16u);
    auto load_chunk = [&](uint4 (&buf)[UNROLL], int it) {
        const uint32_t soff = static_cast<uint32_t>(it) * (kChunkVecs * 16u);
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
            buf[u] = load_stream_buf(rs, static_cast<uint32_t>(tid + u * BLOCK) * 16u, soff);
    };
    // Each thread's last chunk (index nit) is partly filled: its vector
    // v + u*BLOCK is a full vector (below nfull), the row's ragged last
    // vector (nfull, when V is not a multiple of the vector) or past the end
    // (padding).  Its full vectors are loaded together with the chunk before
    // it, so that no wave waits a whole memory latency at the end of the row:
    // every lane loads, with its offset clamped into the row's full vectors,
    // and lanes past them then take the ragged vector or padding.
    const int v = nit * kChunkVecs + tid;
    const uint32_t ni = E::pad_word();
    auto load_last = [&](uint4 (&buf)[UNROLL]) {  // needs nfull >= 1
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int vi = v + u * BLOCK;
            const int vc = vi < nfull ? vi : nfull - 1;
            buf[u] = load_stream_buf(rs, static_cast<uint32_t>(vc) * 16u, 0u);
        }
    };
    // When the last chunks hold at most BLOCK vectors, every thread's vectors
    // u >= 1 there are padding and only the first is processed.
    const bool tail_one = nvec - nit * kChunkVecs <= BLOCK;
    auto consume_last = [&](uint4 (&buf)[UNROLL]) {
        if (v < nvec) {
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                const int vi = v + u * BLOCK;
                if (vi >= nfull)
                    buf[u] = vi < nvec ? E::partial(rp, vi, V) : make_uint4(ni, ni, ni, ni);
            }
            if (tail_one)
                consume(buf, nit, Vecs<1>{});
            else
                consume(buf, nit, Vecs<UNROLL>{});
        }
    };
    // One chunk in flight: two register buffers take turns.  The loop issues
    // its loads unconditionally: a load under a branch makes the compiler's
    // wait before the following chunk's arithmetic cover that load too, which
    // drains the prefetch.  The last full chunks are peeled off the loop.
    uint4 bufA[UNROLL], bufB[UNROLL];
    if (nit >= 1) {
        load_chunk(bufA, 0);
        int it = 0;
        for (; it + 3 <= nit; it += 2) {  // loads it+1 and it+2, both < nit
            load_chunk(bufB, it + 1);
            consume(bufA, it, Vecs<UNROLL>{});
            load_chunk(bufA, it + 2);
            consume(bufB, it + 1, Vecs<UNROLL>{});
        }
        if (it + 1 < nit) {  // two full chunks left, the first in bufA
            load_chunk(bufB, it + 1);
            consume(bufA, it, Vecs<UNROLL>{});
            load_last(bufA);
            consume(bufB, it + 1, Vecs<UNROLL>{});
        } else {  // one full chunk left, in bufA
            load_last(bufB);
            consume(bufA, it, Vecs<UNROLL>{});
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) bufA[u] = bufB[u];
        }
    } else {
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int vi = v + u * BLOCK;
            bufA[u] = vi < nfull ? load_stream_buf(rs, static_cast<uint32_t>(vi) * 16u, 0u)
                                 : make_uint4(ni, ni, ni, ni);
        }
    }
    consume_last(bufA);

    // (1) Row maximum M (a 32-bit max of the ordered bits), then its first
    // id: only threads whose maximum is M search their max chunk (element
    // order inside it: vector u-major, lane k-minor), and the lowest id wins.
    __shared__ uint32_t sh_m[NW], sh_p[NW];
    __shared__ double sh_s[NW], sh_t[NW];
    __shared__ int sh_cnt;                  // CAND: bonus candidates listed
    __shared__ int sh_lb[NW], sh_bw[NW];    // CAND: per-wave holder counts, outside flags
    const int lane = tid & (kWave - 1), wv = tid / kWave;
    // m + 0 turns -0 into +0, so that a row maximum of zero is one key and
    // its first id is the lowest of every zero, whatever its sign.
    const uint32_t om = ordered_bits(m + 0.0f);
    const uint32_t wm = wave_max_u32(om);
    if (lane == 0) sh_m[wv] = wm;
    if (CAND && tid == 0) sh_cnt = 0;
    __syncthreads();
    uint32_t bm = sh_m[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) bm = sh_m[w] > bm ? sh_m[w] : bm;
    const float M = from_ordered_bits(bm);
    const int v0b = itb < 0 ? -1 : itb * kChunkVecs + tid;  // first vector of the max chunk
    float xs[N];
    int pos = INT_MAX;
    if (om == bm && v0b >= 0) {
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) E::unpack(sh_saved[u][tid], xs + u * EPV);
#pragma unroll
        for (int k = N - 1; k >= 0; --k)
            if (xs[k] == m) pos = (v0b + (k / EPV) * BLOCK) * EPV + (k % EPV);
    }
    // lowest id = largest complement; no candidate leaves ~INT_MAX
    const uint32_t wp = wave_max_u32(~static_cast<uint32_t>(pos));
    if (lane == 0) sh_p[wv] = wp;
    __syncthreads();
    uint32_t bp = sh_p[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) bp = sh_p[w] > bp ? sh_p[w] : bp;
    const int P = static_cast<int>(~bp);
    const float Mc = mul_rn(M, c);

    // Bonus candidates of row L_b (WG-uniform branch).
    const bool list_row = CAND && j == Lb && P != INT_MAX;
    // Phase A (row L_b): threads whose saved max chunk holds candidates (at
    // least one each), and whether a candidate could lie outside the saved
    // chunks.  Flat rows, with far more than kMaxBonusCand, stop there.
    // Thresholds are taken relative to the row maximum, (l - M)*c >= tc, so
    // that they stay small whatever the temperature and the logits' size.
    float tc = 0.f;
    if (list_row) {
        // the race's key of the top token, in its units (l*c - log2(E/ln2)),
        // less M*c
        const uint32_t w = race_word(philox_key(a.seed), static_cast<uint32_t>(P),
                                     static_cast<uint32_t>(j), static_cast<uint32_t>(b));
        tc = -hw_log2(-hw_log2(lattice_u32f(w))) - kBonusBelow;
        const uint64_t holders = __ballot(v0b >= 0 && (m - M) * c >= tc);
        const uint64_t outside = __ballot((m2 - M) * c >= tc);
        if (lane == 0) {
            sh_lb[wv] = __popcll(holders);
            sh_bw[wv] = outside != 0ull ? 1 : 0;
        }
    }
    // (2) Every thread rescales its sums to M.  The thread holding the
    // argmax swaps its max chunk for that chunk's other terms, so the block
    // sums are r = sum_{x != argmax} 2^(l_x c - Mc) and the matching entropy
    // numerator t_o.
    // Every term has one sign (terms >= 0, exponents <= 0 relative to M),
    // so float sums over a thread and over a wave lose at most a few ulps;
    // the sums over waves are double.
    const float dl = mc - Mc;
    const float al = hw_exp2(dl);
    const float st = s + cs;
    float X = al * st, Y = 0.f;
    if (ENT) Y = al * (t + ct + dl * st);
    // The wave holding the argmax replaces its holder's value: s plus the
    // max chunk's terms other than P.  Lane k < N of that wave takes element
    // k of the holder's saved chunk from LDS, and a DPP sum over lanes 0..15
    // adds them, instead of one lane adding sixteen terms in turn.
    const uint64_t hold = __ballot(pos == P && P != INT_MAX);
    if (hold != 0ull) {
        const int hl = __ffsll(static_cast<long long>(hold)) - 1;
        const int v0h = __builtin_amdgcn_readlane(v0b, hl);
        float e = 0.f, ed = 0.f;
        if (lane < N) {
            const int u = lane / EPV, q = lane % EPV;
            const T *saved = reinterpret_cast<const T *>(&sh_saved[0][0]);
            const float x = E::at(saved, (u * BLOCK + wv * kWave + hl) * EPV + q);
            float d = fmaf(x, c, -Mc);
            if (ENT) d = fmaxf(d, kMinExp2);
            e = (v0h + u * BLOCK) * EPV + q != P ? hw_exp2(d) : 0.f;
            if (ENT) ed = e * d;
        }
        static_assert(N == 16, "the argmax chunk's terms are summed over one DPP row");
        e += dpp_pull_f<0x111, 0xF>(e);  // row_shr:1 .. 8: lane 15 ends with lanes 0..15
        ed += dpp_pull_f<0x111, 0xF>(ed);
        e += dpp_pull_f<0x112, 0xF>(e);
        ed += dpp_pull_f<0x112, 0xF>(ed);
        e += dpp_pull_f<0x114, 0xF>(e);
        ed += dpp_pull_f<0x114, 0xF>(ed);
        e += dpp_pull_f<0x118, 0xF>(e);
        ed += dpp_pull_f<0x118, 0xF>(ed);
        const float os = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(e), 15));
        const float ot = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(ed), 15));
        if (lane == hl) {
            X = s + os;
            if (ENT) Y = t + ot;
        }
    }
    if (ENT)
        wave_sum2_f32(X, Y);
    else
        X = wave_sum_f32(X);
    if (lane == 0) {
        sh_s[wv] = static_cast<double>(X);
        sh_t[wv] = static_cast<double>(Y);
    }
    __syncthreads();

    // Phase B (row L_b, after the wave counts are in): write the list when
    // it is complete and can fit, before thread 0's double-precision finish,
    // so that the workgroup's other waves need not wait for that.  Rows whose
    // list cannot fit skip the barrier.
    bool fits = false;
    if (CAND && j == Lb) {
        int total = 0, bad = 0;
        if (list_row) {
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                total += sh_lb[w];
                bad |= sh_bw[w];
            }
        }
        fits = list_row && !bad && total <= kMaxBonusCand;
        if (fits) {
            int2 *dst = a.cand_list + static_cast<int64_t>(b) * kMaxBonusCand;
            // every id of a chunk at or above the threshold takes the next slot
            auto take = [&](const uint4 (&vb)[UNROLL], int v0) {
                float xv[N];
#pragma unroll
                for (int u = 0; u < UNROLL; ++u) E::unpack(vb[u], xv + u * EPV);
#pragma unroll
                for (int k = 0; k < N; ++k) {
                    const int id = (v0 + (k / EPV) * BLOCK) * EPV + (k % EPV);
                    if ((xv[k] - M) * c >= tc && id < V) {
                        const int o = atomicAdd(&sh_cnt, 1);
                        if (o < kMaxBonusCand) dst[o] = make_int2(id, __float_as_int(xv[k]));
                    }
                }
            };
            if (v0b >= 0 && (m - M) * c >= tc) {
                uint4 vb[UNROLL];
#pragma unroll
                for (int u = 0; u < UNROLL; ++u) vb[u] = sh_saved[u][tid];
                take(vb, v0b);
            }
            __syncthreads();
        }
        if (tid == 0) a.cand_cnt[b] = fits && sh_cnt <= kMaxBonusCand ? sh_cnt : -1;
    }

    if (tid == 0) {
        double r = 0.0, to = 0.0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            r += sh_s[w];
            to += sh_t[w];
        }
        if constexpr (STATS_CALL)
            row_emit_stats(a.c, g.lse2, g.logtok2, g.qmax_int, g.feat_int, row, M, P, r, to,
                           gather, gidx, ltok);
        else
            row_emit<ENT>(a, g, row, M, P, r, to, gather, gidx, ltok);
    }
}

// CAND: group 0 holds a lossless call's target rows (bonus candidates).
template <typename T, int BLOCK, int UNROLL, bool ENT0, bool CAND>
__global__ __launch_bounds__(BLOCK) void row_stats_kernel(RowArgs a) {
    // the max chunks of the workgroup's threads (one buffer for either group)
    __shared__ uint4 sh_saved[UNROLL][BLOCK];
    const int blk = blockIdx.x;
    if (blk < a.nrows0)
        row_one<T, BLOCK, UNROLL, ENT0, CAND>(a, a.g[0], blk, sh_saved, threadIdx.x);
    else
        row_one<T, BLOCK, UNROLL, false, false>(a, a.g[1], blk - a.nrows0, sh_saved, threadIdx.x);
}

// Load-only twin of the row pass: the same grid (a workgroup per row), the
// same workgroup shape and the same buffer-addressed non-temporal 16-byte
// loads in whole chunks, with the data folded by XOR so that nothing is
// optimised away.
template <int BLOCK, int UNROLL>
__global__ __launch_bounds__(BLOCK) void read_probe_kernel(const void *base, int64_t row_vecs,
                                                          int64_t stride_vecs, uint32_t *sink) {
    const uint4 *row = static_cast<const uint4 *>(base) + blockIdx.x * stride_vecs;
    const int tid = threadIdx.x;
    const buf_rsrc rs = make_rsrc(row, static_cast<uint32_t>(row_vecs) * 16u);
    constexpr int kChunkVecs = UNROLL * BLOCK;
    const int nit = static_cast<int>(row_vecs / kChunkVecs);
    uint32_t acc = 0;
    for (int it = 0; it < nit; ++it) {
        const uint32_t soff = static_cast<uint32_t>(it) * (kChunkVecs * 16u);
        uint4 b[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
            b[u] = load_stream_buf(rs, static_cast<uint32_t>(tid + u * BLOCK) * 16u, soff);
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) acc ^= b[u].x ^ b[u].y ^ b[u].z ^ b[u].w;
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {  // the rest, one vector per lane and u
        const int64_t j = static_cast<int64_t>(nit) * kChunkVecs + tid + u * BLOCK;
        if (j < row_vecs) {
            const uint4 b = load_stream_buf(rs, static_cast<uint32_t>(j) * 16u, 0u);
            acc ^= b.x ^ b.y ^ b.z ^ b.w;
        }
    }
    // XOR over the workgroup: lanes through shuffles, waves through LDS
#pragma unroll
    for (int o = kWave / 2; o > 0; o /= 2) acc ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(acc), o));
    __shared__ uint32_t sh[BLOCK / kWave];
    if ((tid & (kWave - 1)) == 0) sh[tid / kWave] = acc;
    __syncthreads();
    if (tid == 0) {
        uint32_t r = 0;
#pragma unroll
        for (int w = 0; w < BLOCK / kWave; ++w) r ^= sh[w];
        sink[blockIdx.x] = r;
    }
}

}  // namespace sv
