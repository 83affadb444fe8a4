"""Pins of the oracle's lossless verification (accept with min(1, p/q),
residual norm(max(0, p - q)), bonus / trim-point sample from p).

What fixes them independently of the oracle's own code:
  * the worked two-token example of the adaptive-verification page, footnote 1
    (tests/golden/av_footnote_two_token.txt), exactly and by Monte Carlo,
    including the biased trimming rule it warns about as a failing control;
  * exact enumeration on V = 8 showing every emitted position is distributed
    as the target p (the lossless theorem of the speculative-decoding page);
  * chi-square tests over 10^6 independent draws of the end-to-end oracle.
"""
import itertools
import os

import numpy as np
import pytest
from scipy import stats

HERE = os.path.dirname(os.path.abspath(__file__))


def footnote():
    g = {}
    with open(os.path.join(HERE, "golden", "av_footnote_two_token.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            k, *v = line.split()
            g[k] = [float(t) for t in v]
    return g


def logits_of(p):
    with np.errstate(divide="ignore"):
        return np.log(np.asarray(p, dtype=np.float64)).astype(np.float32)


def test_footnote_accept_probability_and_residual(oracle):
    g = footnote()
    p, q = np.array(g["p"]), np.array(g["q"])
    # draft b is accepted with probability min(1, p(b)/q(b))
    assert min(1.0, p[1] / q[1]) == g["accept_prob_b"][0]
    # the residual norm(max(0, p - q)) puts all mass on a
    w = oracle.residual(p, q)
    assert np.array_equal(w / w.sum(), np.array(g["residual"]))


def _exact_output(oracle, p, q, trim=None):
    """Exact first-token distribution of one verified position, by enumeration
    over the draft token, using the oracle's residual and the min(1, p/q) rule.
    trim(x) -> True trims the position: the target samples its own p."""
    out = np.zeros_like(p)
    w = oracle.residual(p, q)
    r = w / w.sum()
    for x in range(len(p)):
        if trim is not None and trim(x):
            out += q[x] * p
            continue
        a = min(1.0, p[x] / q[x])
        out[x] += q[x] * a
        out += q[x] * (1 - a) * r
    return out


def test_footnote_output_distributions_exact(oracle):
    g = footnote()
    p, q = np.array(g["p"]), np.array(g["q"])
    lossless = _exact_output(oracle, p, q)
    biased = _exact_output(oracle, p, q, trim=lambda x: q[x] < g["trim_below"][0])
    assert np.allclose(lossless, g["lossless_output"], atol=1e-15)
    assert np.allclose(biased, g["biased_output"], atol=1e-15)


def _sample_from(rng, probs, n):
    return rng.choice(len(probs), size=n, p=probs).astype(np.int32)


@pytest.mark.parametrize("seed", [0, 77])
def test_footnote_monte_carlo(oracle, seed):
    """End-to-end oracle on the footnote example: lossless verification emits
    p; trimming on q(x_sampled) < 0.5 emits [0.4, 0.6] and is rejected."""
    g = footnote()
    p, q = np.array(g["p"]), np.array(g["q"])
    n = 200_000
    rng = np.random.default_rng(seed + 1)
    target = np.broadcast_to(logits_of(p), (n, 2, 2)).copy()
    draft = np.broadcast_to(logits_of(q), (n, 1, 2)).copy()
    x = _sample_from(rng, q, n).reshape(n, 1)
    r = oracle.verify(target, draft, x, seed)
    first = r["tokens"][:, 0]
    counts = np.bincount(first, minlength=2)
    assert stats.chisquare(counts, n * p).pvalue > 1e-4
    # acceptance frequency of b is 0.625
    acc_b = r["accepted_len"][x[:, 0] == 1].mean()
    assert abs(acc_b - 0.625) < 5 * np.sqrt(0.625 * 0.375 / (x == 1).sum())
    # biased control: trim when the sampled token's q is below 0.5
    kept = (q[x[:, 0]] >= g["trim_below"][0]).astype(np.int32)
    rb = oracle.verify(target, draft, x, seed, kept_len=kept)
    cb = np.bincount(rb["tokens"][:, 0], minlength=2)
    assert stats.chisquare(cb, n * np.array(g["biased_output"])).pvalue > 1e-4
    assert stats.chisquare(cb, n * p).pvalue < 1e-12


def _rand_dist(rng, V, masked=0):
    z = rng.standard_normal(V) * 1.5
    if masked:
        z[rng.choice(V, masked, replace=False)] = -np.inf
    e = np.exp(z - z.max())
    return e / e.sum()


@pytest.mark.parametrize("K", [1, 2, 3])
def test_bruteforce_v8_every_position_is_p(oracle, K):
    """Enumerate all 8^K draft sequences with their probabilities and the
    accept / residual branches: each emitted position is distributed as p_j."""
    rng = np.random.default_rng(100 + K)
    V = 8
    P = [_rand_dist(rng, V, masked=(j == 1) * 2) for j in range(K + 1)]
    Q = [_rand_dist(rng, V) for j in range(K)]
    # feed the distributions through the oracle's row statistics as logits
    rowsP = [oracle.row_probs(logits_of(pj)) for pj in P]
    rowsQ = [oracle.row_probs(logits_of(qj)) for qj in Q]
    R = []
    for j in range(K):
        w = oracle.residual(rowsP[j], rowsQ[j])
        R.append(w / w.sum())
    emit = [np.zeros(V) for _ in range(K + 1)]
    reach = np.zeros(K + 1)
    for xs in itertools.product(range(V), repeat=K):
        pr = np.prod([rowsQ[j][xs[j]] for j in range(K)])
        alive = pr
        for j in range(K):
            reach[j] += alive
            a = min(1.0, rowsP[j][xs[j]] / rowsQ[j][xs[j]])
            emit[j][xs[j]] += alive * a
            emit[j] += alive * (1 - a) * R[j]
            alive *= a
        reach[K] += alive
        emit[K] += alive * rowsP[K]
    for j in range(K + 1):
        assert np.allclose(emit[j] / reach[j], rowsP[j], atol=1e-13)
        assert np.allclose(rowsP[j], P[j], atol=1e-6)


def _chisq_positions(oracle, P, Q, T, n, seed, data_seed):
    K = len(Q)
    V = len(P[0])
    rng = np.random.default_rng(data_seed)
    tl = np.stack([logits_of(p) * np.float32(T) for p in P])  # softmax(l/T) = P
    dl = np.stack([logits_of(q) * np.float32(T) for q in Q])
    target = np.broadcast_to(tl, (n, K + 1, V)).copy()
    draft = np.broadcast_to(dl, (n, K, V)).copy()
    probsP = [oracle.row_probs(tl[j], T) for j in range(K + 1)]
    probsQ = [oracle.row_probs(dl[j], T) for j in range(K)]
    x = np.stack([_sample_from(rng, probsQ[j], n) for j in range(K)], axis=1)
    r = oracle.verify(target, draft, x, seed, temperature=T)
    pvals = []
    for j in range(K + 1):
        sel = r["accepted_len"] >= j
        counts = np.bincount(r["tokens"][sel, j], minlength=V)
        exp = probsP[j] * sel.sum()
        keep = exp > 0
        assert counts[~keep].sum() == 0  # masked ids are never emitted
        pvals.append(stats.chisquare(counts[keep], exp[keep]).pvalue)
    accept0 = (r["accepted_len"] >= 1).mean()
    return pvals, accept0, np.minimum(probsP[0], probsQ[0]).sum()


@pytest.mark.slow
@pytest.mark.parametrize("T", [1.0, 0.7])
def test_chisquare_1e6_emitted_tokens_follow_p(oracle, T):
    rng = np.random.default_rng(7)
    V, K = 8, 3
    P = [_rand_dist(rng, V, masked=(j == 2) * 3) for j in range(K + 1)]
    Q = [_rand_dist(rng, V) for j in range(K)]
    pvals, accept0, expect0 = _chisq_positions(oracle, P, Q, T, 1_000_000, seed=12345,
                                              data_seed=99)
    assert min(pvals) > 1e-4, pvals
    # expected acceptance at a position is sum_x min(p, q)
    assert abs(accept0 - expect0) < 5 * np.sqrt(expect0 * (1 - expect0) / 1e6)


def test_chisquare_control_detects_a_planted_error(oracle):
    """Power check of the harness: swapping p and q in the residual (a plausible
    sign mistake) must be rejected by the same chi-square."""
    rng = np.random.default_rng(3)
    V, n = 8, 200_000
    p, q = _rand_dist(rng, V), _rand_dist(rng, V)
    w_bad = oracle.residual(q, p)
    r_bad = w_bad / w_bad.sum()
    out = np.zeros(V)
    for x in range(V):
        a = min(1.0, p[x] / q[x])
        out[x] += q[x] * a
        out += q[x] * (1 - a) * r_bad
    counts = rng.multinomial(n, out)
    assert stats.chisquare(counts, n * p).pvalue < 1e-12


def test_race_frequencies_follow_weights(oracle):
    w = np.array([1.0, 2.0, 0.0, 3.0, 4.0, 0.5, 0.0, 1.5])
    n = 60_000
    ys = np.array([oracle.race(w, 5, pos=i % 7, b=i // 7)[0] for i in range(n)])
    counts = np.bincount(ys, minlength=8)
    assert counts[2] == 0 and counts[6] == 0
    keep = w > 0
    assert stats.chisquare(counts[keep], n * w[keep] / w.sum()).pvalue > 1e-4
    assert oracle.race(np.zeros(8), 5, 0, 0)[0] == -1


def test_identical_models_accept_everything(oracle):
    rng = np.random.default_rng(4)
    B, K, V = 64, 4, 50
    t = rng.standard_normal((B, K + 1, V)).astype(np.float32)
    d = t[:, :K].copy()
    x = rng.integers(0, V, size=(B, K)).astype(np.int32)
    r = oracle.verify(t, d, x, 9)
    assert np.all(r["accepted_len"] == K)  # p/q = 1 > u always
    assert np.array_equal(r["tokens"][:, :K], x)


def test_zero_target_probability_rejects(oracle):
    B, K, V = 8, 3, 16
    t = np.zeros((B, K + 1, V), dtype=np.float32)
    d = np.zeros((B, K, V), dtype=np.float32)
    x = np.full((B, K), 5, dtype=np.int32)
    t[:, 1, 5] = -np.inf  # p(x_1) = 0
    x[3, 0] = V  # out-of-range token: p = q = 0, rejected
    r = oracle.verify(t, d, x, 1)
    assert list(r["accepted_len"]) == [1, 1, 1, 0, 1, 1, 1, 1]
    assert np.all(r["tokens"][np.arange(B) != 3, 1] != 5)


def test_kept_len_samples_target_at_trim_point(oracle):
    rng = np.random.default_rng(8)
    B, K, V = 32, 4, 20
    t = rng.standard_normal((B, K + 1, V)).astype(np.float32)
    d = t[:, :K].copy()  # always accepted
    x = rng.integers(0, V, size=(B, K)).astype(np.int32)
    kept = (np.arange(B) % (K + 1)).astype(np.int32)
    r = oracle.verify(t, d, x, 2, kept_len=kept)
    assert np.array_equal(r["accepted_len"], kept)
    for b in range(B):
        L = kept[b]
        assert np.all(r["tokens"][b, L + 1:] == -1)
        assert np.all(np.isnan(r["t_lse"][b, L + 1:]))  # rows past L never read
        assert np.all(np.isnan(r["d_lse"][b, L:]))


def test_determinism_and_seed_dependence(oracle):
    rng = np.random.default_rng(10)
    B, K, V = 200, 3, 64
    t = (rng.standard_normal((B, K + 1, V)) * 2).astype(np.float32)
    d = (rng.standard_normal((B, K, V)) * 2).astype(np.float32)
    x = rng.integers(0, V, size=(B, K)).astype(np.int32)
    a = oracle.verify(t, d, x, 42, nthreads=1)
    b = oracle.verify(t, d, x, 42, nthreads=5)
    c = oracle.verify(t, d, x, 43)
    assert np.array_equal(a["tokens"], b["tokens"])
    assert not np.array_equal(a["tokens"], c["tokens"])


def test_boundary_flag_near_accept(oracle):
    u0 = oracle.uniform(0, 0, 0, 0, oracle.TAG_ACCEPT)
    V = 4
    q = np.full(V, 0.25)
    p = np.array([0.25 * (u0 + 3e-6), 0, 0, 0])
    p[1:] = (1 - p[0]) / 3
    t = np.stack([logits_of(p), logits_of(p)])[None]
    d = logits_of(q)[None, None]
    r = oracle.verify(t, d, np.zeros((1, 1), dtype=np.int32), 0)
    assert r["boundary"][0] & oracle.NEAR_ACCEPT
    r2 = oracle.verify(t, d, np.ones((1, 1), dtype=np.int32), 0)
    assert not (r2["boundary"][0] & oracle.NEAR_ACCEPT)
