// sv_rowstats.hpp -- the streaming row pass: one workgroup per logits row,
// 16-byte loads, a single pass that keeps an online (max, sum, entropy
// numerator, argmax) state per thread, merged across the wave with shuffles
// and across waves through LDS.
//
// Per row it yields the quantities the verification rules read: the
// log-normaliser, the normalised entropy h = H(p)/log V that the FLy gate
// compares with theta (page "Training-Free Loosely Speculative Decoding...",
// section "2. Metodologia", part A), the top token, the probability of the
// drafted token, and for draft rows q_max and logit(q_max), the feature of the
// adaptive-verification estimator (page "Verificacion Adaptativa sin una
// cabeza de confianza", section "Puntuar la Distribucion").
//
// Arithmetic is in base 2: with c = log2(e)/T every term is 2^(l*c - mc),
// where mc = m*c and m is the running maximum of the raw logits.  Terms are
// summed in float within a chunk of UNROLL vectors and chunk sums in double.
#pragma once

#include "sv_common.hpp"

namespace sv {

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
    double *lse2;     // [rows] log2 normaliser: mc + log2(s)
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
};

// Per-thread (and merged) state.  s and t hold every term except those of
// the chunk that holds the current argmax, whose float sums cs / ct ride
// alongside; keeping them apart lets the final step replace that chunk by its
// non-argmax terms without cancellation, however peaked the row.
struct RowState {
    float m;    // running maximum of the raw logits
    float mc;   // m * c: every term is 2^(l*c - mc)
    double s;   // sum of the terms outside the argmax chunk
    double t;   // sum of term * (l*c - mc) outside the argmax chunk
    float cs;   // sum of the argmax chunk's terms
    float ct;   // sum of the argmax chunk's term * (l*c - mc)
    int pos;    // first id attaining m (INT_MAX: none)
};

__device__ __forceinline__ RowState merge_states(const RowState &a, const RowState &b) {
    const bool bw = (b.m > a.m) || (b.m == a.m && b.pos < a.pos);
    const RowState &hi = bw ? b : a;
    const RowState &lo = bw ? a : b;
    const float dl = lo.mc - hi.mc;  // <= 0
    const double al = static_cast<double>(hw_exp2(dl));
    const double ls = lo.s + static_cast<double>(lo.cs);
    const double lt = lo.t + static_cast<double>(lo.ct);
    RowState r = hi;
    r.s = hi.s + al * ls;
    r.t = hi.t + al * (lt + static_cast<double>(dl) * ls);
    return r;
}

__device__ __forceinline__ RowState shfl_state(const RowState &s, int mask) {
    RowState o;
    o.m = __shfl_xor(s.m, mask, kWave);
    o.mc = __shfl_xor(s.mc, mask, kWave);
    o.s = __shfl_xor(s.s, mask, kWave);
    o.t = __shfl_xor(s.t, mask, kWave);
    o.cs = __shfl_xor(s.cs, mask, kWave);
    o.ct = __shfl_xor(s.ct, mask, kWave);
    o.pos = __shfl_xor(s.pos, mask, kWave);
    return o;
}

template <typename T, int BLOCK, int UNROLL, bool ENT>
__device__ __forceinline__ void row_one(const RowArgs &a, const RowGroup &g, int64_t row) {
    using E = Elem<T>;
    constexpr int EPV = E::kPerVec;
    constexpr int N = UNROLL * EPV;
    constexpr int NW = BLOCK / kWave;
    const int tid = threadIdx.x;
    const int V = a.V;
    const float c = a.c;

    const int b = static_cast<int>(row / g.rows_per_seq);
    const int j = static_cast<int>(row - static_cast<int64_t>(b) * g.rows_per_seq);
    if (a.kept_len) {
        const int L = clamp_len(a.kept_len[b], a.K);
        if (j >= L + g.active_extra) {  // trimmed away: report "not read"
            if (tid == 0) {
                const float nan = __builtin_nanf("");
                if (g.lse) g.lse[row] = nan;
                if (g.entropy) g.entropy[row] = nan;
                if (g.argmax) g.argmax[row] = -1;
                if (g.qmax) g.qmax[row] = nan;
                if (g.feat) g.feat[row] = nan;
            }
            return;
        }
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
    const uint4 *vrow = reinterpret_cast<const uint4 *>(rp);

    RowState st;
    st.m = kNoMax;
    st.mc = kNoMax * c;
    st.s = 0.0;
    st.t = 0.0;
    st.cs = 0.f;
    st.ct = 0.f;
    st.pos = INT_MAX;
    uint4 saved[UNROLL];
    int saved_v0 = -1;

    auto consume = [&](const uint4 (&buf)[UNROLL], int v0) {
        float x[N];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) E::unpack(buf[u], x + u * EPV);
        float cm = x[0];
#pragma unroll
        for (int k = 1; k < N; ++k) cm = fmaxf(cm, x[k]);
        const bool up = cm > st.m;
        const float mn = up ? cm : st.m;
        const float mcn = mn * c;
        float cs[4] = {0.f, 0.f, 0.f, 0.f}, ct[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < N; ++k) {
            float d = fmaf(x[k], c, -mcn);
            if (ENT) d = fmaxf(d, kMinExp2);
            const float e = hw_exp2(d);
            cs[k & 3] += e;
            if (ENT) ct[k & 3] = fmaf(e, d, ct[k & 3]);
        }
        const float csum = (cs[0] + cs[1]) + (cs[2] + cs[3]);
        const float ctsum = ENT ? (ct[0] + ct[1]) + (ct[2] + ct[3]) : 0.f;
        if (up) {
            // the old argmax chunk joins the rest; everything rescales to mn
            const float dl = st.mc - mcn;
            const double al = static_cast<double>(hw_exp2(dl));
            const double stot = st.s + static_cast<double>(st.cs);
            if (ENT) st.t = al * (st.t + static_cast<double>(st.ct) + static_cast<double>(dl) * stot);
            st.s = al * stot;
            st.cs = csum;
            st.ct = ctsum;
            st.m = mn;
            st.mc = mcn;
            saved_v0 = v0;
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) saved[u] = buf[u];
        } else {
            st.s += static_cast<double>(csum);
            if (ENT) st.t += static_cast<double>(ctsum);
        }
    };

    int v = tid;
    if (v + (UNROLL - 1) * BLOCK < nfull) {
        uint4 cur[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) cur[u] = vrow[v + u * BLOCK];
        for (;;) {
            const int vn = v + UNROLL * BLOCK;
            const bool more = vn + (UNROLL - 1) * BLOCK < nfull;
            uint4 nxt[UNROLL];
            if (more) {
#pragma unroll
                for (int u = 0; u < UNROLL; ++u) nxt[u] = vrow[vn + u * BLOCK];
            }
            consume(cur, v);
            v = vn;
            if (!more) break;
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) cur[u] = nxt[u];
        }
    }
    if (v < nvec) {  // last, partly filled chunk of this thread
        uint4 buf[UNROLL];
        const uint32_t ni = E::neg_inf_word();
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int vi = v + u * BLOCK;
            if (vi < nfull)
                buf[u] = vrow[vi];
            else if (vi < nvec)
                buf[u] = E::partial(rp, vi, V);
            else
                buf[u] = make_uint4(ni, ni, ni, ni);
        }
        consume(buf, v);
    }

    // Exact argmax of this thread: first element of the saved chunk equal to
    // the thread's maximum (element order: vector u-major, lane k-minor).
    if (saved_v0 >= 0) {
        float x[N];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) E::unpack(saved[u], x + u * EPV);
#pragma unroll
        for (int k = N - 1; k >= 0; --k)
            if (x[k] == st.m) st.pos = (saved_v0 + (k / EPV) * BLOCK) * EPV + (k % EPV);
    }
    const int own_pos = st.pos;

    // Wave, then workgroup reduction in a fixed order.
#pragma unroll
    for (int msk = kWave / 2; msk > 0; msk >>= 1) st = merge_states(st, shfl_state(st, msk));
    __shared__ RowState sh[NW];
    __shared__ RowState total;
    __shared__ float others_s, others_t;  // the argmax chunk's other terms
    const int lane = tid & (kWave - 1), wv = tid / kWave;
    if (lane == 0) sh[wv] = st;
    __syncthreads();
    if (tid == 0) {
        RowState acc = sh[0];
#pragma unroll
        for (int w = 1; w < NW; ++w) acc = merge_states(acc, sh[w]);
        total = acc;
        others_s = 0.f;
        others_t = 0.f;
    }
    __syncthreads();
    const RowState fin = total;

    // Replace the argmax chunk by its terms other than the argmax itself,
    // recomputed by the thread that holds it: r = sum_{x != argmax} terms and
    // t_o = sum_{x != argmax} term * exponent, free of cancellation.
    if (own_pos == fin.pos && fin.pos != INT_MAX) {
        float x[N];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) E::unpack(saved[u], x + u * EPV);
        float os = 0.f, ot = 0.f;
#pragma unroll
        for (int k = 0; k < N; ++k) {
            const int id = (saved_v0 + (k / EPV) * BLOCK) * EPV + (k % EPV);
            if (id != fin.pos) {
                float d = fmaf(x[k], c, -fin.mc);
                if (ENT) d = fmaxf(d, kMinExp2);
                const float e = hw_exp2(d);
                os += e;
                if (ENT) ot = fmaf(e, d, ot);
            }
        }
        others_s = os;
        others_t = ot;
    }
    __syncthreads();

    if (tid == 0) {
        // The argmax term is 2^r0 with r0 = m*c - mc, the rounding residue of
        // mc (exact in float); the row's sum is 2^r0 + r.
        const double r0 = static_cast<double>(fmaf(fin.m, c, -fin.mc));
        const double e0 = exp2(r0);
        const double r = fin.s + static_cast<double>(others_s);
        const double rho = r / e0;        // (1 - q_max) / q_max
        const double l1p = log1p(rho);    // ln(sum / 2^r0)
        const double lse2 = static_cast<double>(fin.mc) + r0 + l1p * kLog2eD;
        if (g.lse2) g.lse2[row] = lse2;
        if (g.lse) g.lse[row] = static_cast<float>(lse2 * kLn2);
        const int am = fin.pos == INT_MAX ? -1 : fin.pos;
        if (g.argmax) g.argmax[row] = am;
        if (g.am_int) g.am_int[row] = am;
        if (ENT) {
            // H = ln(sum) - ln2 * t_all / sum, rewritten around the argmax term:
            // H = ln(1 + rho) + ln2 (r0 r - t_o) / (2^r0 + r).
            const double to = fin.t + static_cast<double>(others_t);
            const double H = l1p + kLn2 * (r0 * r - to) / (e0 + r);
            const float h = static_cast<float>(H / log(static_cast<double>(V)));
            if (g.entropy) g.entropy[row] = h;
            if (g.h_int) g.h_int[row] = h;
        }
        const float qm = static_cast<float>(1.0 / (1.0 + rho));
        const float ft = static_cast<float>(-log(fmax(rho, 0x1.0p-126)));  // logit(q_max)
        if (g.qmax) g.qmax[row] = qm;
        if (g.qmax_int) g.qmax_int[row] = qm;
        if (g.feat) g.feat[row] = ft;
        if (g.feat_int) g.feat_int[row] = ft;
        if (gather && g.logtok2)
            g.logtok2[gidx] = static_cast<double>(ltok) * static_cast<double>(c) - lse2;
    }
}

template <typename T, int BLOCK, int UNROLL, bool ENT0>
__global__ __launch_bounds__(BLOCK) void row_stats_kernel(RowArgs a) {
    const int blk = blockIdx.x;
    if (blk < a.nrows0)
        row_one<T, BLOCK, UNROLL, ENT0>(a, a.g[0], blk);
    else
        row_one<T, BLOCK, UNROLL, false>(a, a.g[1], blk - a.nrows0);
}

}  // namespace sv
