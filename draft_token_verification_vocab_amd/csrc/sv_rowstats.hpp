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
// Rows are streamed with non-temporal 16-byte loads.
//
// Arithmetic is in base 2: with c = log2(e)/T every term is 2^(l*c - mc),
// where mc = m*c and m is the running maximum of the raw logits.  A thread
// reads its share of the row in chunks of UNROLL vectors (UNROLL*8 bfloat16
// or UNROLL*4 float logits); terms are summed in float inside a chunk and
// chunk sums in double.  Each thread keeps the chunk that holds its maximum
// apart (its sums and its raw data in registers), so the end can replace that
// chunk by its terms other than the argmax and form 1 - q_max without
// cancellation, however peaked the row.
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
};

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

    // Thread state.  s, t: sums outside the chunk that holds the maximum;
    // cs, ct: that chunk's sums; saved / v0b: that chunk's data and position.
    float m = kNoMax, mc = kNoMax * c, cs = 0.f, ct = 0.f;
    double s = 0.0, t = 0.0;
    int v0b = -1;
    uint4 saved[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) saved[u] = make_uint4(0u, 0u, 0u, 0u);

    auto consume = [&](const uint4 (&buf)[UNROLL], int v0) {
        float x[N];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) E::unpack(buf[u], x + u * EPV);
        float cm = x[0];
#pragma unroll
        for (int k = 1; k < N; ++k) cm = fmaxf(cm, x[k]);
        const bool up = cm > m;
        const float mn = fmaxf(cm, m);
        const float mcn = mn * c;
        float s4[4] = {0.f, 0.f, 0.f, 0.f}, t4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < N; ++k) {
            float d = fmaf(x[k], c, -mcn);
            if (ENT) d = fmaxf(d, kMinExp2);
            const float e = hw_exp2(d);
            s4[k & 3] += e;
            if (ENT) t4[k & 3] = fmaf(e, d, t4[k & 3]);
        }
        const float csum = (s4[0] + s4[1]) + (s4[2] + s4[3]);
        const float ctsum = ENT ? (t4[0] + t4[1]) + (t4[2] + t4[3]) : 0.f;
        // Branch-free update: if the maximum moved, the previous max chunk
        // joins the rest and everything is rescaled to the new maximum
        // (factor 2^dl); otherwise this chunk joins the rest (dl = 0).
        const float dl = mc - mcn;
        const double al = static_cast<double>(hw_exp2(dl));
        const double stot = s + static_cast<double>(up ? cs : csum);
        if (ENT) {
            const double ttot = t + static_cast<double>(up ? ct : ctsum);
            t = al * (ttot + static_cast<double>(dl) * (up ? stot : 0.0));
        }
        s = al * stot;
        cs = up ? csum : cs;
        ct = up ? ctsum : ct;
        m = mn;
        mc = mcn;
        v0b = up ? v0 : v0b;
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            saved[u].x = up ? buf[u].x : saved[u].x;
            saved[u].y = up ? buf[u].y : saved[u].y;
            saved[u].z = up ? buf[u].z : saved[u].z;
            saved[u].w = up ? buf[u].w : saved[u].w;
        }
    };

    int v = tid;
    for (; v + (UNROLL - 1) * BLOCK < nfull; v += UNROLL * BLOCK) {
        uint4 buf[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) buf[u] = load_stream(vrow + v + u * BLOCK);
        consume(buf, v);
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

    // First id attaining the thread maximum (element order inside the saved
    // chunk: vector u-major, lane k-minor).
    float xs[N];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) E::unpack(saved[u], xs + u * EPV);
    int pos = INT_MAX;
    if (v0b >= 0) {
#pragma unroll
        for (int k = N - 1; k >= 0; --k)
            if (xs[k] == m) pos = (v0b + (k / EPV) * BLOCK) * EPV + (k % EPV);
    }

    // (1) Row maximum and its first id in one key: (ordered max, -id).
    __shared__ uint64_t sh_key[NW];
    __shared__ double sh_s[NW], sh_t[NW];
    const int lane = tid & (kWave - 1), wv = tid / kWave;
    const uint64_t key =
        (static_cast<uint64_t>(ordered_bits(m)) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(pos));
    const uint64_t wkey = wave_max_u64(key);
    if (lane == 0) sh_key[wv] = wkey;
    __syncthreads();
    uint64_t bkey = sh_key[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) bkey = sh_key[w] > bkey ? sh_key[w] : bkey;
    const float M = from_ordered_bits(static_cast<uint32_t>(bkey >> 32));
    const int P = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(bkey));
    const float Mc = M * c;

    // (2) Every thread rescales its sums to M.  The thread holding the
    // argmax swaps its max chunk for that chunk's other terms, so the block
    // sums are r = sum_{x != argmax} 2^(l_x c - Mc) and the matching entropy
    // numerator t_o.
    double X, Y = 0.0;
    if (pos == P && P != INT_MAX) {
        float os = 0.f, ot = 0.f;
#pragma unroll
        for (int k = 0; k < N; ++k) {
            const int id = (v0b + (k / EPV) * BLOCK) * EPV + (k % EPV);
            if (id != P) {
                float d = fmaf(xs[k], c, -Mc);
                if (ENT) d = fmaxf(d, kMinExp2);
                const float e = hw_exp2(d);
                os += e;
                if (ENT) ot = fmaf(e, d, ot);
            }
        }
        X = s + static_cast<double>(os);
        if (ENT) Y = t + static_cast<double>(ot);
    } else {
        const float dl = mc - Mc;
        const double al = static_cast<double>(hw_exp2(dl));
        const double st = s + static_cast<double>(cs);
        X = al * st;
        if (ENT) Y = al * (t + static_cast<double>(ct) + static_cast<double>(dl) * st);
    }
    const double wx = wave_sum_f64(X);
    const double wy = ENT ? wave_sum_f64(Y) : 0.0;
    if (lane == 0) {
        sh_s[wv] = wx;
        sh_t[wv] = wy;
    }
    __syncthreads();

    if (tid == 0) {
        double r = 0.0, to = 0.0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            r += sh_s[w];
            to += sh_t[w];
        }
        // The argmax term is 2^r0 with r0 = M*c - Mc, the rounding residue of
        // Mc (exact in float); the row's sum of terms is 2^r0 + r.
        const double r0 = static_cast<double>(fmaf(M, c, -Mc));
        const double e0 = exp2(r0);
        const double rho = r / e0;      // (1 - q_max) / q_max
        const double l1p = log1p(rho);  // ln(sum / 2^r0)
        const double lse2 = static_cast<double>(Mc) + r0 + l1p * kLog2eD;
        if (g.lse2) g.lse2[row] = lse2;
        if (g.lse) g.lse[row] = static_cast<float>(lse2 * kLn2);
        const int am = P == INT_MAX ? -1 : P;
        if (g.argmax) g.argmax[row] = am;
        if (g.am_int) g.am_int[row] = am;
        if (ENT) {
            // H = ln(sum) - ln2 * (sum of term*exponent) / sum, rewritten
            // around the argmax term: H = ln(1 + rho) + ln2 (r0 r - t_o) / (2^r0 + r).
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
