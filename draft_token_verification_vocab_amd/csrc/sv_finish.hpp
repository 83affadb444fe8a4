// sv_finish.hpp -- per-sequence decisions after the row pass.
//
// Lossless (page "Speculative Decoding: как черновая модель ускоряет
// генерацию LLM без потери качества", sections "Основная идея: черновик и
// верификация" and "Математика верификации"): accept draft x_j while
// u_j < p(x_j)/q(x_j); at the first rejection j* draw from
// norm(max(0, p - q)); if all L verified drafts pass, draw from p at row L
// (row K is the bonus row; L < K is the trim point of adaptive verification,
// where the target samples its own distribution -- page "Verificacion
// Adaptativa sin una cabeza de confianza", footnote 1).  Draws are the
// exponential race argmax_x w(x)/E_x, E_x = -ln u_x, with per-id Philox u_x.
//
// The race re-streams one (target, draft) row pair per sequence; rows are
// split into segments so that small batches still fill the GPU.  Each
// segment screens keys in float (log2 domain), re-evaluates every candidate
// within a margin of the segment's best in double, and reports its best
// double key; a combine kernel takes the best segment.  Work is pruned by
// bounds: the key of the target's top token (then the wave's best) bounds
// the row's best from below; an id's key is at most log2 p plus 23.5 on the
// 2^-24 lattice, and at most log2 p + 0.5 + (leading one bits of its race
// word).  Groups of eight ids below the first bound skip their draws (on
// peaked rows nearly all of them); the others draw one screening block, whose
// 16 high word bits per id settle the second bound for all but a few ids, and
// draw the rest of the word only for blocks of four with an id still in;
// ids below the second bound skip their exact weight and logarithms.
//
// FLy (page "Training-Free Loosely Speculative Decoding...", section
// "2. Metodologia", part A): one wave per sequence; deviations and gate
// passes are two ballots and the scan walks those bit masks.
//
// Both rules also log, per sequence, the near-ties where float arithmetic may
// legitimately decide the other way than exact arithmetic: an evaluated
// accept test with |u - p/q| < 1e-5, race keys whose two largest lie within
// 1e-6 relative, a residual that vanished, an evaluated FLy gate with
// |h - theta| < 1e-5.
#pragma once

#include "sv_common.hpp"
#include "sv_philox.hpp"

namespace sv {

// Boundary-case bits, one word per sequence.
constexpr uint32_t kNearAccept = 1u;     // an evaluated accept test had |u - p/q| < 1e-5
constexpr uint32_t kNearRace = 2u;       // the two largest race keys within 1e-6 relative
constexpr uint32_t kResidualEmpty = 4u;  // max(0, p - q) vanished; the draw used p
constexpr uint32_t kNearGate = 8u;       // an evaluated FLy gate had |h - theta| < 1e-5

// A segment's race result: its largest key (ln units) with its id, and its
// second largest key, exact whenever it lies within the screening margin of
// the largest (below that it is only a lower bound, which decides the
// near-tie flag the same way).
struct RaceCand {
    double key;
    double key2;
    int32_t x;     // -1: no candidate in this segment
    uint32_t info; // verified position the race ran at | boundary bits << 8
};

// The two largest keys of a set of race candidates and the first one's id
// (lowest id on equal keys; a key equal to the largest counts as the second).
struct Top2 {
    double k1, k2;
    int x1;
    __device__ __forceinline__ void init() {
        k1 = k2 = -__builtin_inf();
        x1 = INT_MAX;
    }
    __device__ __forceinline__ void add(double k, int x) {
        if (x == INT_MAX) return;  // no candidate
        if (k > k1 || (k == k1 && x < x1)) {
            k2 = k1;
            k1 = k;
            x1 = x;
        } else if (k > k2) {
            k2 = k;
        }
    }
    // Another set's top two: the largest of everything but the winner is the
    // new second.
    __device__ __forceinline__ void merge(double ok1, int ox1, double ok2) {
        add(ok1, ox1);
        if (ok2 > k2) k2 = ok2;
    }
};

// The near-tie test (k1 - k2)/k1 <= 1e-6 on the linear keys w/E, written for
// keys in ln units: 1 - exp(k2 - k1) <= 1e-6.  No candidate at all counts as
// a near-tie.
__device__ __forceinline__ bool near_race(double k1, double k2) {
    if (!(k1 > -__builtin_inf())) return true;
    return !(-expm1(k2 - k1) > 1e-6);
}

struct RaceArgs {
    const void *target;
    const void *draft;
    int64_t stride;
    int32_t V, K;
    const int32_t *kept_len;  // [B] or null
    const double *t_lse2;     // [B*(K+1)]
    const double *t_logp2;    // [B*K]
    const double *d_lse2;     // [B*K]
    const double *d_logq2;    // [B*K]
    const int32_t *t_am;      // [B*(K+1)] target top token per row
    float c;                  // log2(e)/T (float, as in the row pass)
    double inv_t;             // 1/T in double
    uint64_t seed;
    int32_t segs;             // segments per row
    int32_t seg_groups;       // groups of eight ids per segment
    RaceCand *cand;           // [B][segs]
    // The row pass's candidate list of row L_b (the only row a draw from p
    // can use): count (-1 when incomplete) and (id, logit bits) entries.
    const int32_t *bonus_cnt;  // [B]
    const int2 *bonus_list;    // [B][kMaxBonusCand]
};

// Screening margin in log2 units.  Float screening keys carry errors of a
// few 1e-6; every thread best within the margin is re-evaluated in double.
constexpr float kScreenMargin = 1e-3f;

// What the race needs of the row it runs on, besides the row itself.
struct RowPick {
    int jstar;       // first rejected position (L when all verified drafts pass)
    int am;          // the target's top token at row jstar
    int listed;      // ids the row pass listed for a draw from p at row jstar, or -1
    uint32_t flags;  // kNearAccept when an evaluated test sat within 1e-5 of its ratio
    double lt;       // target log2-normaliser of row jstar
    double ld;       // draft log2-normaliser of row jstar (residual rows only)
};

// The accept tests of sequence b and what the race needs at the first
// rejected position, for every workgroup of the sequence (they all agree).
// The first wave does it: lane j loads row j's accept ratio, top token and
// normalisers at once (lane 0 also the listed count), so that the decision
// and the chosen row's values come from one round of loads; row K = 64 has
// no lane and is loaded after the decision.  The logits at the top token
// depend on it, so the race loads them together with its first vectors.
template <typename T>
__device__ __forceinline__ RowPick decide_lossless(const RaceArgs &a, int b, int L,
                                                   PhiloxKey key) {
    __shared__ RowPick s_pick;
    const int tid = threadIdx.x;
    const int K = a.K;
    if (tid < kWave) {
        double lp = 0.0, lq = 0.0, lt = 0.0, ld = 0.0;
        int am = -1;
        if (tid < K) {
            const int i = b * K + tid;
            lp = a.t_logp2[i];
            lq = a.d_logq2[i];
            ld = a.d_lse2[i];
        }
        if (tid <= K) {
            am = a.t_am[b * (K + 1) + tid];
            lt = a.t_lse2[b * (K + 1) + tid];
        }
        const int cnt = a.bonus_cnt ? a.bonus_cnt[b] : -1;
        const uint32_t uw = draw_u32(key, 0u, tid, b, kTagAccept);
        bool rej = false, near = false;
        if (tid < L) {
            const double u = lattice_u64(uw);
            const double ratio = exp2(lp - lq);  // p(x_j)/q(x_j)
            rej = !(u < ratio);
            near = fabs(u - ratio) < 1e-5;  // false for a NaN ratio
        }
        const unsigned long long m = __ballot(rej);
        const int jstar = m ? __ffsll(m) - 1 : L;
        const int listed = jstar == L ? cnt : -1;  // only a draw from p can use the list
        // the tests evaluated are those at positions 0..jstar
        const unsigned long long done = jstar >= kWave - 1 ? ~0ull : (2ull << jstar) - 1ull;
        const uint32_t flags = (__ballot(near) & done) != 0ull ? kNearAccept : 0u;
        if (tid == jstar) s_pick = RowPick{jstar, am, listed, flags, lt, ld};
        if (jstar == kWave && tid == 0) {  // K = 64 and every draft accepted: row 64
            const int r = b * (K + 1) + kWave;
            s_pick = RowPick{jstar, a.t_am[r], listed, flags, a.t_lse2[r], 0.0};
        }
    }
    __syncthreads();
    return s_pick;
}

// Largest value -log2(E/ln2) can take on the 2^-24 lattice (u <= 1 - 2^-24
// gives E/ln2 >= 8.6e-8, i.e. 23.47), rounded up: no id's key exceeds its
// log2 weight by more.
constexpr float kMaxNegLogE = 23.5f;

// The key the race gives the target's top token am (logits xt, xd there),
// less the screening margin: a floor that the row's best key is known to
// reach.  -inf when am has no weight (then nothing is screened out).  Keys
// are in log2 units of the normalised weight (log2 p for a draw from p), so
// they stay small whatever the temperature and the logits' magnitude.
__device__ __forceinline__ float race_floor(bool residual, int am, float xt, float xd, float c,
                                            double lse2_t, double lse2_d, PhiloxKey key,
                                            uint32_t pos, uint32_t seq) {
    if (am < 0) return -__builtin_inff();
    float lw;
    if (residual) {
        const float p = hw_exp2(fmaf(xt, c, -static_cast<float>(lse2_t)));
        const float qq = hw_exp2(fmaf(xd, c, -static_cast<float>(lse2_d)));
        const float w = p - qq;
        lw = w > 0.f ? hw_log2(w) : -__builtin_inff();
    } else {
        lw = fmaf(xt, c, -static_cast<float>(lse2_t));  // log2 p
    }
    if (!(lw > -__builtin_inff())) return -__builtin_inff();
    const float e2 = -hw_log2(lattice_u32f(race_word(key, static_cast<uint32_t>(am), pos, seq)));
    return lw - hw_log2(e2) - kScreenMargin;
}

// thr - 0.5 + lsub rounded down to float: the bound tests below compare
// fmaf(l, -c, this) with small integers, and rounding down keeps them on the
// side of evaluating an id however large |lsub| is.
__device__ __forceinline__ float bound_base(float thr, float lsub) {
    return __double2float_rd(static_cast<double>(thr) - 0.5 + static_cast<double>(lsub));
}

// Ids are raced in groups of eight (one bfloat16 vector, two float vectors),
// the ids one screening block serves.
constexpr int kRaceGroup = 8;
template <typename T>
constexpr int group_vecs() {
    return kRaceGroup / Elem<T>::kPerVec;
}

// Race over groups [g_lo, g_hi) of one row (pair) with NT threads, one group
// per thread per trip.  RES: w = max(0, p - q) from the target and draft
// rows; otherwise w = p of the target row.  am: the target's top token, whose
// key (less the margin) is a floor the row's best is known to reach; its
// logits are loaded together with the first groups.  Returns (in thread 0)
// the best double key and id (id -1 when no id of the range can win) and the
// second largest double key (see RaceCand).
template <typename T, int NT, bool RES>
__device__ void race_range(const T *trow, const T *drow, int g_lo, int g_hi, int V, float c,
                           double cd, double inv_t, double lse2_t, double lse2_d, PhiloxKey key,
                           uint32_t pos, uint32_t seq, int am, double *out_key, int *out_x,
                           double *out_key2) {
    using E = Elem<T>;
    constexpr int EPV = E::kPerVec;
    constexpr int G = group_vecs<T>();
    constexpr int NW = NT / kWave;
    const int tid = threadIdx.x;
    const int nfull = V / EPV;
    const int nvec = (V + EPV - 1) / EPV;
    const uint4 *tv = reinterpret_cast<const uint4 *>(trow);
    const uint4 *dv = reinterpret_cast<const uint4 *>(drow);
    const float lt2 = static_cast<float>(lse2_t);
    const float ld2 = static_cast<float>(lse2_d);
    // Whole trips cover groups of full vectors only (every thread has one);
    // one last trip takes the rest, the row's partial vector included.  The
    // whole trips' loads are unconditional, so that the wait before a trip's
    // arithmetic covers its own group and not the next trip's.
    const int g_hf = min(g_hi, nfull / G);
    const int nit = g_hf > g_lo ? (g_hf - g_lo) / NT : 0;
    struct Grp {
        uint4 t[G], d[G];
    };
    // Whole trips are buffer-addressed over the rows' full vectors: the trip's
    // byte offset is wave-uniform, each lane's offset inside it fixed.
    const buf_rsrc rt = make_rsrc(trow, static_cast<uint32_t>(nfull) * 16u);
    const buf_rsrc rd = make_rsrc(RES ? drow : trow, static_cast<uint32_t>(nfull) * 16u);
    auto load_trip = [&](Grp &q, int it) {
        const uint32_t soff = static_cast<uint32_t>(g_lo + it * NT) * (G * 16u);
#pragma unroll
        for (int v = 0; v < G; ++v) {
            const uint32_t voff = static_cast<uint32_t>(tid * G + v) * 16u;
            q.t[v] = load_stream_buf(rt, voff, soff);
            if (RES) q.d[v] = load_stream_buf(rd, voff, soff);
        }
    };
    Grp qa, qb;
#pragma unroll
    for (int v = 0; v < G; ++v) qa.t[v] = qa.d[v] = qb.t[v] = qb.d[v] = make_uint4(0u, 0u, 0u, 0u);
    // the top token's logits first, so that the floor waits for them alone
    const bool am_ok = am >= 0 && am < V;
    const float am_xt = am_ok ? E::at(trow, am) : -__builtin_inff();
    const float am_xd = RES && am_ok ? E::at(drow, am) : -__builtin_inff();
    if (nit > 0) load_trip(qa, 0);
    const float floor =
        race_floor(RES, am_ok ? am : -1, am_xt, am_xd, c, lse2_t, lse2_d, key, pos, seq);

    // best, best2: this lane's two best screening keys; thr: the wave's best
    // less the margin.  An id whose key cannot reach thr is never a candidate,
    // so it needs neither its exact weight nor its logarithms.
    float best = floor, best2 = -__builtin_inff();
    int bx = INT_MAX, b2x = INT_MAX;
    float bt = 0.f, bd = 0.f;  // the best id's target and draft logits
    uint32_t bw = 0u;          // and its race word
    float thr = floor - kScreenMargin;
    // lb = l*c - lsub bounds the log2 weight: log2 p, and w = max(0, p - q)
    // <= p for a residual row.  The tests use a = thr - 0.5 - lb, one FMA per
    // id: the key is below lb + 0.5 + (leading ones of the race word), so an
    // id is a candidate only if its leading ones reach a.
    const float lsub = lt2;
    float abase = bound_base(thr, lsub);
    // One trip over group gi (live: gi is in the range).  Wave-uniform: the
    // skip tests are ballots.
    //  - A group none of whose ids has a <= 23 (lb + 23.5 < thr) draws
    //    nothing.
    //  - Otherwise its screening block gives each id's 16 high word bits and
    //    so its leading ones when below 16: an id with fewer than a is out.
    //  - A block of four ids draws its race stream only if one of them is
    //    still in (at least a leading ones, or at least 16 of them); then the
    //    exact count decides.
    auto trip = [&](const Grp &q, int gi, bool live) {
        bool evaluated = false;
        float xt[kRaceGroup], av[kRaceGroup];
#pragma unroll
        for (int v = 0; v < G; ++v) E::unpack(q.t[v], xt + v * EPV);
#pragma unroll
        for (int k = 0; k < kRaceGroup; ++k) av[k] = fmaf(xt[k], -c, abase);
        float amin = av[0];
#pragma unroll
        for (int k = 1; k < kRaceGroup; ++k) amin = fminf(amin, av[k]);
        const bool need = live && amin <= kMaxNegLogE - 0.5f;
        if (__ballot(need) == 0ull) return;  // no lane's group can win: no draws
        const uint32_t x0 = static_cast<uint32_t>(live ? gi : g_lo) * kRaceGroup;
        const uint4 sw = philox10(make_uint4(x0 >> 3, pos, seq, kTagScreen), key);
#pragma unroll
        for (int blk = 0; blk < kRaceGroup / 4; ++blk) {
            bool maybe[4];
            bool any = false;
#pragma unroll
            for (int qi = 0; qi < 4; ++qi) {
                const int k = blk * 4 + qi;
                // bitwise, so that no lane branches per id
                maybe[qi] = need & (screen_ones(sw, static_cast<uint32_t>(k)) >= av[k]);
                any |= maybe[qi];
            }
            if (__ballot(any) == 0ull) continue;
            const uint32_t base = x0 + blk * 4;
            const uint4 rw = philox10(make_uint4(base >> 2, pos, seq, kTagRace), key);
#pragma unroll
            for (int qi = 0; qi < 4; ++qi) {
                const int k = blk * 4 + qi;
                const uint32_t word = race_word_of(screen_half(sw, static_cast<uint32_t>(k)),
                                                   pick_word(rw, static_cast<uint32_t>(qi)));
                const bool cand = maybe[qi] && static_cast<float>(leading_ones(word)) >= av[k];
                const int x = static_cast<int>(base) + qi;
                if (cand && x < V) {
                    const float p = fmaf(xt[k], c, -lt2);  // log2 p
                    float lw;
                    const float xd = RES ? E::elem(q.d[k / EPV], k % EPV) : 0.f;
                    if (RES) {
                        const float qq = hw_exp2(fmaf(xd, c, -ld2));
                        const float w = hw_exp2(p) - qq;
                        lw = w > 0.f ? hw_log2(w) : -__builtin_inff();
                    } else {
                        lw = p;
                    }
                    const float e2 = -hw_log2(lattice_u32f(word));  // E / ln 2 > 0
                    const float g = lw - hw_log2(e2);
                    if (g > best) {
                        best2 = best;
                        b2x = bx;
                        best = g;
                        bx = x;
                        bt = xt[k];
                        if (RES) bd = xd;
                        bw = word;
                    } else if (g > best2) {
                        best2 = g;
                        b2x = x;
                    }
                    evaluated = true;
                }
            }
        }
        if (__ballot(evaluated) != 0ull) {
            thr = fmaxf(thr, from_ordered_bits(wave_max_u32(ordered_bits(best))) - kScreenMargin);
            abase = bound_base(thr, lsub);
        }
    };
    int it = 0;
    for (; it + 2 < nit; it += 2) {
        load_trip(qb, it + 1);
        trip(qa, g_lo + it * NT + tid, true);
        load_trip(qa, it + 2);
        trip(qb, g_lo + (it + 1) * NT + tid, true);
    }
    if (it + 1 < nit) {
        load_trip(qb, it + 1);
        trip(qa, g_lo + it * NT + tid, true);
        trip(qb, g_lo + (it + 1) * NT + tid, true);
    } else if (it < nit) {
        trip(qa, g_lo + it * NT + tid, true);
    }
    if (g_lo + nit * NT < g_hi) {  // the rest of the range, fewer groups than threads
        const int gi = g_lo + nit * NT + tid;
        const bool live = gi < g_hi;
        Grp q;
        const uint32_t ni = E::pad_word();
#pragma unroll
        for (int v = 0; v < G; ++v) {
            const int vi = gi * G + v;
            q.t[v] = q.d[v] = make_uint4(ni, ni, ni, ni);
            if (live && vi < nfull) {
                q.t[v] = load_stream(tv + vi);
                if (RES) q.d[v] = load_stream(dv + vi);
            } else if (live && vi < nvec) {
                q.t[v] = E::partial(trow, vi, V);
                if (RES) q.d[v] = E::partial(drow, vi, V);
            }
        }
        trip(q, gi, live);
    }

    // Workgroup maximum of the screening keys (DPP within waves, LDS across).
    __shared__ float sh_best[NW];
    __shared__ double sh_key[NW], sh_key2[NW];
    __shared__ int sh_x[NW];
    const int lane = tid & (kWave - 1), wv = tid / kWave;
    const float m = from_ordered_bits(wave_max_u32(ordered_bits(best)));
    if (lane == 0) sh_best[wv] = m;
    __syncthreads();
    float g1 = sh_best[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) g1 = fmaxf(g1, sh_best[w]);

    // Double-precision keys of the candidates within the margin: a thread's
    // best from the Philox word kept with it (no second draw), its second
    // best (rarely within the margin) from its logits and word again.
    auto exact_key = [&](float lt, float ld, uint32_t word, double *k, int *kx, int x) {
        const double lnE = log(-log(lattice_u64(word)));
        if (RES) {
            const double w = exp2(static_cast<double>(lt) * cd - lse2_t) -
                             exp2(static_cast<double>(ld) * cd - lse2_d);
            if (w > 0.0) {
                *k = log(w) - lnE;
                *kx = x;
            }
        } else {
            *k = static_cast<double>(lt) * inv_t - lnE;  // ln p(x) + lse: the same for every id
            *kx = x;
        }
    };
    double k64 = -__builtin_inf(), k64b = -__builtin_inf();
    int kx = INT_MAX, kxb = INT_MAX;
    const bool near = bx != INT_MAX && best >= g1 - kScreenMargin;
    const bool near2 = b2x != INT_MAX && best2 >= g1 - kScreenMargin;
    if (near) exact_key(bt, bd, bw, &k64, &kx, bx);
    if (near2)
        exact_key(E::at(trow, b2x), RES ? E::at(drow, b2x) : 0.f,
                  race_word(key, static_cast<uint32_t>(b2x), pos, seq), &k64b, &kxb, b2x);
    // The wave's two best candidates: usually one lane is near, so its values
    // are read lane by lane rather than reduced over the whole wave.
    Top2 wt;
    wt.init();
    auto read_lane = [](double v, int l) {
        const uint64_t kb = static_cast<uint64_t>(__double_as_longlong(v));
        // readlane returns a signed int: take each half as 32 unsigned bits
        const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(kb >> 32), l);
        const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(kb), l);
        return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
    };
    for (uint64_t nb = __ballot(near || near2); nb != 0ull; nb &= nb - 1ull) {
        const int l = __builtin_ctzll(nb);
        wt.add(read_lane(k64, l), __builtin_amdgcn_readlane(kx, l));
        wt.add(read_lane(k64b, l), __builtin_amdgcn_readlane(kxb, l));
    }
    if (lane == 0) {  // sh_key, sh_key2 and sh_x are not the arrays read above: no barrier
        sh_key[wv] = wt.k1;
        sh_key2[wv] = wt.k2;
        sh_x[wv] = wt.x1;
    }
    __syncthreads();
    if (tid == 0) {
        Top2 t;
        t.init();
#pragma unroll
        for (int w = 0; w < NW; ++w) t.merge(sh_key[w], sh_x[w], sh_key2[w]);
        *out_key = t.k1;
        *out_x = t.x1 == INT_MAX ? -1 : t.x1;
        *out_key2 = t.k2;
    }
    __syncthreads();
}

// A draw from p at row L over the ids the row pass listed, which hold every
// id that could win it: exact double keys, no second read of the row.  The
// first wave does it; the best key and id (-1: none) and the second key land
// in thread 0.
__device__ __forceinline__ void race_listed(const RaceArgs &a, int b, int jstar, int n,
                                            PhiloxKey key, double *out_key, int *out_x,
                                            double *out_key2) {
    const int tid = threadIdx.x;
    if (tid >= kWave) return;
    Top2 t;
    t.init();
    if (tid < n) {
        const int2 e = a.bonus_list[static_cast<int64_t>(b) * kMaxBonusCand + tid];
        const double u = lattice_u64(race_word(key, static_cast<uint32_t>(e.x),
                                               static_cast<uint32_t>(jstar),
                                               static_cast<uint32_t>(b)));
        t.add(static_cast<double>(__int_as_float(e.y)) * a.inv_t - log(-log(u)), e.x);
    }
#pragma unroll
    for (int msk = kWave / 2; msk > 0; msk >>= 1) {
        const double ok1 = __shfl_xor(t.k1, msk, kWave);
        const double ok2 = __shfl_xor(t.k2, msk, kWave);
        const int ox = __shfl_xor(t.x1, msk, kWave);
        t.merge(ok1, ox, ok2);
    }
    if (tid == 0) {
        *out_key = t.k1;
        *out_x = t.x1 == INT_MAX ? -1 : t.x1;
        *out_key2 = t.k2;
    }
}

// Race over groups [g_lo, g_hi) of sequence b's row at the decided position.
template <typename T, int NT>
__device__ __forceinline__ void race_decided(const RaceArgs &a, int b, const RowPick &pk,
                                             bool residual, PhiloxKey key, int g_lo, int g_hi,
                                             double *k, int *x, double *k2) {
    const int jstar = pk.jstar;
    const T *trow = static_cast<const T *>(a.target) +
                    (static_cast<int64_t>(b) * (a.K + 1) + jstar) * a.stride;
    if (residual) {
        const T *drow = static_cast<const T *>(a.draft) +
                        (static_cast<int64_t>(b) * a.K + jstar) * a.stride;
        race_range<T, NT, true>(trow, drow, g_lo, g_hi, a.V, a.c, static_cast<double>(a.c),
                                a.inv_t, pk.lt, pk.ld, key, jstar, b, pk.am, k, x, k2);
    } else {
        race_range<T, NT, false>(trow, nullptr, g_lo, g_hi, a.V, a.c, static_cast<double>(a.c),
                                 a.inv_t, pk.lt, 0.0, key, jstar, b, pk.am, k, x, k2);
    }
}

// Segmented race: workgroup i takes segment i % segs of sequence i / segs (a
// 1-D grid, so B is not bound by the grid's y limit) and reports its best
// candidate; race_combine_kernel then picks each sequence's winner.
template <typename T, int NT>
__global__ __launch_bounds__(NT) void race_kernel(RaceArgs a) {
    const int b = static_cast<int>(blockIdx.x) / a.segs;
    const int seg = static_cast<int>(blockIdx.x) - b * a.segs;
    const PhiloxKey key = philox_key(a.seed);
    const int L = a.kept_len ? clamp_len(a.kept_len[b], a.K) : a.K;
    const RowPick pk = decide_lossless<T>(a, b, L, key);
    const int jstar = pk.jstar;
    const bool residual = jstar < L;
    const int n = pk.listed;
    double k = -__builtin_inf(), k2 = -__builtin_inf();
    int x = -1;
    if (n >= 0) {
        if (seg == 0) race_listed(a, b, jstar, n, key, &k, &x, &k2);
    } else {
        const int ngroups = (a.V + kRaceGroup - 1) / kRaceGroup;
        const int g_lo = seg * a.seg_groups;
        race_decided<T, NT>(a, b, pk, residual, key, g_lo, min(ngroups, g_lo + a.seg_groups), &k, &x,
                            &k2);
    }
    if (threadIdx.x == 0)
        a.cand[b * a.segs + seg] =
            RaceCand{k, k2, x, static_cast<uint32_t>(jstar) | (pk.flags << 8)};
}

// Best segment per sequence (largest key, then lowest id); writes
// accepted_len, the emitted tokens and the boundary bits.  One wave per
// sequence: lane s reads segment s's candidate (segs <= 64) and lane j the
// draft token j (K <= 64), in one round of loads; a shuffle reduction picks
// the winner and the second largest key.  A residual that vanished in
// floating point (no candidate anywhere; only possible within rounding of
// u_j = p/q) falls back to a race over p at the same row.
struct SeqPick {
    double k1, k2;   // the winner's key and the second largest
    int y;           // the winner, -1 when no segment has a candidate
    int jstar;       // accepted drafts (the first rejected position, or L)
    int tk;          // this lane's draft token (lane j holds token j)
    uint32_t flags;  // boundary bits from the race
};

// The reduction of sequence b's segment candidates by one wave (every lane
// ends with the result).
__device__ __forceinline__ SeqPick combine_reduce(const RaceArgs &a, const int32_t *tokens, int b,
                                                  int lane) {
    const int K = a.K;
    const RaceCand cnd = lane < a.segs ? a.cand[b * a.segs + lane]
                                       : RaceCand{-__builtin_inf(), -__builtin_inf(), -1, 0u};
    const int tk = lane < K ? tokens[b * K + lane] : -1;
    Top2 t;
    t.init();
    if (cnd.x >= 0) {
        t.k1 = cnd.key;
        t.k2 = cnd.key2;
        t.x1 = cnd.x;
    }
#pragma unroll
    for (int msk = kWave / 2; msk > 0; msk >>= 1) {
        const double ok1 = __shfl_xor(t.k1, msk, kWave);
        const double ok2 = __shfl_xor(t.k2, msk, kWave);
        const int ox = __shfl_xor(t.x1, msk, kWave);
        t.merge(ok1, ox, ok2);
    }
    const uint32_t info = __shfl(cnd.info, 0);  // the same in every segment
    SeqPick s;
    s.jstar = static_cast<int>(info & 0xFFu);
    s.flags = info >> 8;
    s.y = t.x1 == INT_MAX ? -1 : t.x1;
    s.k1 = t.k1;
    s.k2 = t.k2;
    s.tk = tk;
    return s;
}

// The fallback race over p at row jstar of sequence b, by a whole workgroup
// of NT threads; the key, id and second key land in thread 0.
template <typename T, int NT>
__device__ __forceinline__ void combine_fallback(const RaceArgs &a, int b, int jstar, double *k,
                                                 int *x, double *k2) {
    const int K = a.K;
    const T *trow = static_cast<const T *>(a.target) +
                    (static_cast<int64_t>(b) * (K + 1) + jstar) * a.stride;
    const int ngroups = (a.V + kRaceGroup - 1) / kRaceGroup;
    const double lt = a.t_lse2[b * (K + 1) + jstar];
    const PhiloxKey key = philox_key(a.seed);
    const int am = a.t_am[b * (K + 1) + jstar];
    race_range<T, NT, false>(trow, nullptr, 0, ngroups, a.V, a.c, static_cast<double>(a.c),
                             a.inv_t, lt, 0.0, key, jstar, b, am, k, x, k2);
}

// Sequence b's outputs from its pick, by one wave.
__device__ __forceinline__ void combine_emit(const RaceArgs &a, int b, int lane, SeqPick s,
                                             int32_t *accepted_len, int32_t *out_tokens,
                                             uint32_t *boundary) {
    const int K = a.K;
    if (near_race(s.k1, s.k2)) s.flags |= kNearRace;
    if (lane == 0) {
        accepted_len[b] = s.jstar;
        if (boundary) boundary[b] = s.flags;
    }
    for (int j = lane; j <= K; j += kWave) {
        // j < jstar <= 64 only on the first pass, where j == lane holds token j
        out_tokens[b * (K + 1) + j] = j < s.jstar ? s.tk : (j == s.jstar ? s.y : -1);
    }
}

template <typename T, int NT>
__global__ __launch_bounds__(NT) void race_combine_kernel(RaceArgs a, const int32_t *tokens,
                                                         int32_t *accepted_len,
                                                         int32_t *out_tokens,
                                                         uint32_t *boundary) {
    static_assert(NT == kWave, "one wave per sequence");
    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    SeqPick s = combine_reduce(a, tokens, b, lane);
    if (s.y < 0) {
        double k = -__builtin_inf(), kk2 = -__builtin_inf();
        int x = -1;
        combine_fallback<T, NT>(a, b, s.jstar, &k, &x, &kk2);
        s.y = __shfl(x, 0);
        s.k1 = __shfl(k, 0);
        s.k2 = __shfl(kk2, 0);
        s.flags |= kResidualEmpty;
    }
    combine_emit(a, b, lane, s, accepted_len, out_tokens, boundary);
}

// FLy: a deviation is a draft token different from the target's top token.
// Deviations with h < theta are rejected at once; others are accepted only
// when the next W drafts exist and all match (else rejected, retroactively
// when the target deviates again inside the window).  The replacement or
// bonus token is the target's top token at the stopping row.
template <int NT>
__global__ __launch_bounds__(NT) void fly_kernel(const int32_t *tokens, const int32_t *kept_len,
                                                 const int32_t *am, const float *h, int B, int K,
                                                 float theta, int W, int32_t *accepted_len,
                                                 int32_t *out_tokens, uint32_t *boundary) {
    // One wave per sequence: lane k holds position k (K <= 64), the
    // deviation and gate tests become two ballots, and the scan runs on
    // wave-uniform bit masks.
    const int lane = threadIdx.x & (kWave - 1);
    const int b = __builtin_amdgcn_readfirstlane(
        static_cast<int>((static_cast<int64_t>(blockIdx.x) * NT + threadIdx.x) / kWave));
    if (b >= B) return;
    const int L = kept_len ? __builtin_amdgcn_readfirstlane(clamp_len(kept_len[b], K)) : K;
    const int32_t *tok = tokens + static_cast<int64_t>(b) * K;
    const int32_t *top = am + static_cast<int64_t>(b) * (K + 1);
    const float *hb = h + static_cast<int64_t>(b) * (K + 1);
    const bool live = lane < L;
    // loaded for every drafted position, so that they do not wait for L
    const int32_t tk = lane < K ? tok[lane] : 0;
    const int32_t tp = lane < K + 1 ? top[lane] : 0;
    const float hv = lane < K ? hb[lane] : 0.f;
    const uint64_t dev = __ballot(live && tk != tp);
    const uint64_t gate = __ballot(live && hv >= theta);  // NaN entropy fails the gate
    const uint64_t gnear = __ballot(live && fabsf(hv - theta) < 1e-5f);

    int j = 0, jstar = L;
    uint64_t rest = dev;   // deviations at positions >= j
    uint64_t seen = 0ull;  // the deviations whose gate the scan evaluated
    while (rest != 0) {
        j = __builtin_ctzll(rest);
        seen |= 1ull << j;
        if (!((gate >> j) & 1ull) || j + W > L - 1) {
            jstar = j;
            break;
        }
        // here 0 <= W <= L-1-j <= 63: the window is positions j+1 .. j+W
        const uint64_t win = W == 0 ? 0ull : (((1ull << W) - 1ull) << (j + 1));
        if (dev & win) {
            jstar = j;
            break;
        }
        const int nj = j + W + 1;
        rest = nj >= 64 ? 0ull : (dev & (~0ull << nj));
    }
    if (lane == 0) {
        accepted_len[b] = jstar;
        if (boundary) boundary[b] = (seen & gnear) != 0ull ? kNearGate : 0u;
    }
    // the stopping row may be row K = 64, which no lane holds
    const int32_t topj = jstar < kWave ? __shfl(tp, jstar) : top[jstar];
    int32_t *ot = out_tokens + static_cast<int64_t>(b) * (K + 1);
    for (int k = lane; k <= K; k += kWave) {
        // k < jstar <= L <= 64 only on the first pass, where k == lane
        ot[k] = k < jstar ? tk : (k == jstar ? topj : -1);
    }
}

}  // namespace sv
