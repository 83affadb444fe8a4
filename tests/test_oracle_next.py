"""Pins of the oracle's IRLS refit, scorer diagnostics, budgeted trimming and
prompt-lookup drafter against things other than itself: an independent
optimiser, finite differences, scikit-learn's metrics, hand-worked cases
and Python's own substring search."""
import math

import numpy as np
import pytest


def _batch(rng, B, K, p_acc=0.6, trim=True):
    """Features, accepted lengths and kept lengths of a synthetic batch."""
    feat = rng.normal(-1.0, 1.2, (B, K))
    acc = np.zeros(B, dtype=np.int32)
    for b in range(B):
        a = 0
        while a < K and rng.random() < p_acc:
            a += 1
        acc[b] = a
    kept = rng.integers(0, K + 1, B).astype(np.int32) if trim else None
    if kept is not None:
        acc = np.minimum(acc, kept)  # verification never accepts past the kept length
    return feat, acc, kept


# ---------------------------------------------------------------------------
# IRLS refit
# ---------------------------------------------------------------------------
def test_irls_converges_to_the_likelihood_optimum(oracle):
    # Undamped Newton rounds on a fixed batch reach the minimiser of the
    # summed log-loss found by an independent quasi-Newton optimiser (scipy),
    # using the oracle's pinned log-loss as the objective.
    from scipy.optimize import minimize
    rng = np.random.default_rng(1)
    B, K = 3000, 4
    feat = rng.normal(-0.5, 1.2, (B, K))
    true = np.array([0.8, 1.5, 1.2, 0.9, 0.6])
    acc = np.zeros(B, dtype=np.int32)
    for b in range(B):  # labels drawn from the logistic model itself
        while acc[b] < K and rng.random() < 1 / (1 + np.exp(-(true[0] * feat[b, acc[b]]
                                                              + true[1 + acc[b]]))):
            acc[b] += 1
    kept = None
    ob = np.r_[1.0, 0.5 - 0.3 * np.arange(K)]
    for _ in range(30):
        st = oracle.IrlsState(K)
        oracle.irls_accumulate(st, feat, acc, kept, ob)
        ob, flags = oracle.irls_solve(st, ob, 0.0)
        assert flags & 1
    res = minimize(lambda th: oracle.av_loss(feat, acc, kept, th)[0], np.zeros(K + 1),
                   method="BFGS", options={"gtol": 1e-11, "maxiter": 2000})
    assert np.allclose(ob, res.x, atol=2e-5), (ob, res.x)


def test_irls_gradient_and_hessian_are_the_loss_derivatives(oracle):
    rng = np.random.default_rng(2)
    B, K = 80, 5
    feat, acc, kept = _batch(rng, B, K)
    ob = np.r_[0.8, rng.normal(0, 0.5, K)]
    st = oracle.IrlsState(K)
    oracle.irls_accumulate(st, feat, acc, kept, ob)
    N = st.cnt[0]

    def total(th):
        m, n = oracle.av_loss(feat, acc, kept, th)
        return m * n

    def grad(th, h=1e-5):
        return np.array([(total(th + h * e) - total(th - h * e)) / (2 * h)
                         for e in np.eye(K + 1)])
    assert N == oracle.av_loss(feat, acc, kept, ob)[1]
    assert np.allclose(st.g, grad(ob), rtol=1e-6, atol=1e-6)
    h = 1e-4
    Hfd = np.array([(grad(ob + h * e) - grad(ob - h * e)) / (2 * h) for e in np.eye(K + 1)])
    assert np.allclose(st.H, Hfd, rtol=1e-4, atol=1e-4)
    # intercepts of different positions never share a label: H is arrow-shaped
    off = st.H[1:, 1:] - np.diag(np.diag(st.H[1:, 1:]))
    assert np.all(off == 0.0)


def test_irls_damping_scales_each_coefficient_by_its_evidence(oracle):
    rng = np.random.default_rng(3)
    B, K = 60, 4
    feat, acc, kept = _batch(rng, B, K)
    ob0 = np.r_[0.7, 0.3, 0.0, -0.3, -0.6]
    steps = {}
    for c in (0.0, 25.0):
        st = oracle.IrlsState(K)
        oracle.irls_accumulate(st, feat, acc, kept, ob0)
        cnt = st.cnt.copy()
        new, _ = oracle.irls_solve(st, ob0, c)
        steps[c] = new - ob0
    assert np.allclose(steps[25.0], steps[0.0] * cnt / (cnt + 25.0), rtol=1e-12, atol=1e-15)
    # a position without labels does not move; huge damping barely moves anything
    st = oracle.IrlsState(K)
    kept0 = np.minimum(kept, 2)
    oracle.irls_accumulate(st, feat, np.minimum(acc, kept0), kept0, ob0)
    assert st.cnt[3] == 0 and st.cnt[4] == 0
    new, _ = oracle.irls_solve(st, ob0, 0.0)
    assert new[3] == ob0[3] and new[4] == ob0[4]


def test_irls_equal_features_hold_the_slope(oracle):
    # Every feature equal: the slope has no curvature of its own left; the
    # intercepts take the closed-form Newton step (ybar - s) / (s (1 - s)).
    B, K = 50, 3
    rng = np.random.default_rng(4)
    feat = np.full((B, K), 0.7)
    _, acc, kept = _batch(rng, B, K)
    ob = np.array([1.0, 0.2, -0.1, -0.5])
    st = oracle.IrlsState(K)
    oracle.irls_accumulate(st, feat, acc, kept, ob)
    new, flags = oracle.irls_solve(st, ob, 0.0)
    assert flags == 3 and new[0] == ob[0]
    for i in range(K):
        ys = [1.0 if i < acc[b] else 0.0 for b in range(B) if i < min(acc[b] + 1, kept[b])]
        if not ys:
            assert new[1 + i] == ob[1 + i]
            continue
        s = 1.0 / (1.0 + math.exp(-(0.7 * ob[0] + ob[1 + i])))
        assert new[1 + i] - ob[1 + i] == pytest.approx((np.mean(ys) - s) / (s * (1 - s)),
                                                       rel=1e-12)


def test_irls_rounds_add_and_reset(oracle):
    rng = np.random.default_rng(5)
    K = 4
    f1, a1, k1 = _batch(rng, 40, K)
    f2, a2, k2 = _batch(rng, 30, K)
    ob = np.r_[0.9, 0.4, 0.1, -0.2, -0.5]
    st = oracle.IrlsState(K)
    oracle.irls_accumulate(st, f1, a1, k1, ob)
    oracle.irls_accumulate(st, f2, a2, k2, ob)
    both = oracle.IrlsState(K)
    oracle.irls_accumulate(both, np.r_[f1, f2], np.r_[a1, a2], np.r_[k1, k2], ob)
    assert np.allclose(st.g, both.g, rtol=1e-13) and np.allclose(st.H, both.H, rtol=1e-13)
    assert np.array_equal(st.cnt, both.cnt)
    oracle.irls_solve(st, ob, 10.0)
    assert not st.g.any() and not st.H.any() and not st.cnt.any()
    # no labels at all: nothing moves
    empty = oracle.IrlsState(K)
    oracle.irls_accumulate(empty, f1, a1, np.zeros(40, dtype=np.int32), ob)
    new, flags = oracle.irls_solve(empty, ob, 10.0)
    assert flags == 0 and np.array_equal(new, ob)


# ---------------------------------------------------------------------------
# Scorer diagnostics
# ---------------------------------------------------------------------------
def _single_position(rng, n, ties=False):
    # K = 1 and every draft kept: the label of sequence b is accepted_len[b]
    f = rng.normal(0, 1.5, (n, 1))
    if ties:
        f = np.round(f * 2) / 2
    y = (rng.random(n) < 1 / (1 + np.exp(-(0.8 * f[:, 0] - 0.2)))).astype(np.int32)
    return f, y, np.ones(n, dtype=np.int32)


@pytest.mark.parametrize("ties", [False, True])
def test_diagnostics_match_scikit_learn(oracle, ties):
    from sklearn.metrics import log_loss, roc_auc_score
    rng = np.random.default_rng(6 + ties)
    f, y, kept = _single_position(rng, 700, ties)
    ob = np.array([0.9, -0.3])
    d = oracle.av_diagnostics(f, y, kept, ob, nbins=10)
    z = 0.9 * f[:, 0] - 0.3
    s = 1 / (1 + np.exp(-z))
    assert d["n"] == 700
    assert d["auc"] == pytest.approx(roc_auc_score(y, z), abs=1e-14)
    assert d["logloss"] == pytest.approx(log_loss(y, s), rel=1e-12)


def test_ece_closed_forms(oracle):
    rng = np.random.default_rng(8)
    f, y, kept = _single_position(rng, 400)
    ob = np.array([0.9, -0.3])
    s = 1 / (1 + np.exp(-(0.9 * f[:, 0] - 0.3)))
    one = oracle.av_diagnostics(f, y, kept, ob, nbins=1)
    assert one["ece"] == pytest.approx(abs(s.mean() - y.mean()), rel=1e-12)
    # hand case: scores 0.2, 0.3 (bin 0 of 2) and 0.8, 0.9 (bin 1); labels 0,1,1,1
    p = np.array([0.2, 0.3, 0.8, 0.9])
    z = np.log(p / (1 - p))
    d = oracle.av_diagnostics(z[:, None], np.array([0, 1, 1, 1], dtype=np.int32),
                              np.ones(4, dtype=np.int32), np.array([1.0, 0.0]), nbins=2)
    # bin 0: |0.25 - 0.5| * 2/4, bin 1: |0.85 - 1| * 2/4
    assert d["ece"] == pytest.approx(0.125 + 0.075, rel=1e-12)
    assert d["auc"] == 1.0


def test_auc_extremes(oracle):
    f = np.zeros((6, 1))
    y = np.array([1, 0, 1, 0, 0, 1], dtype=np.int32)
    d = oracle.av_diagnostics(f, y, np.ones(6, dtype=np.int32), np.array([1.0, 0.0]))
    assert d["auc"] == 0.5                       # every pair tied
    d = oracle.av_diagnostics(f, np.ones(6, dtype=np.int32), np.ones(6, dtype=np.int32),
                              np.array([1.0, 0.0]))
    assert math.isnan(d["auc"])                  # one class only


# ---------------------------------------------------------------------------
# Budgeted trimming
# ---------------------------------------------------------------------------
def test_budget_worked_example(oracle):
    # survivals 0.9, 0.45 | 0.8, 0.72; sorted 0.9, 0.8, 0.72, 0.45;
    # expected tokens 2, 2.9, 3.7, 4.42, 4.87 over costs 1, 1.2, 1.5, 1.9, 2.6:
    # ratios 2, 2.417, 2.467, 2.326, 1.873 -> budget 2: the first draft of each
    conf = np.array([[0.9, 0.5], [0.8, 0.9]], dtype=np.float32)
    r = oracle.av_budget(conf, np.array([1.0, 1.2, 1.5, 1.9, 2.6]))
    assert r["budget"] == 2 and r["kept_len"].tolist() == [1, 1]
    assert r["mask"].tolist() == [[1, 0], [1, 0]]
    est = 2 + np.float32(0.9) + np.float32(0.8)
    assert r["best_ratio"] == pytest.approx(est / 1.5, rel=1e-12)


def test_budget_properties(oracle):
    rng = np.random.default_rng(9)
    B, K = 40, 6
    conf = rng.uniform(0.05, 1.0, (B, K)).astype(np.float32)
    M = B * K
    k = np.arange(M + 1)
    cost = 1.0 + 0.004 * k + 2e-5 * k ** 2
    r = oracle.av_budget(conf, cost)
    surv = np.cumprod(conf.astype(np.float64), axis=1)
    mask = r["mask"].astype(bool)
    assert mask.sum() == r["budget"] == r["kept_len"].sum()
    for b in range(B):  # kept drafts form a prefix of each sequence
        assert mask[b, :r["kept_len"][b]].all() and not mask[b, r["kept_len"][b]:].any()
    if 0 < r["budget"] < M:
        assert surv[mask].min() >= surv[~mask].max() - 1e-6
    # free drafts: every draft kept; prohibitive drafts: none
    assert oracle.av_budget(conf, np.ones(M + 1))["budget"] == M
    assert oracle.av_budget(conf, np.r_[1.0, np.full(M, 1e9)])["budget"] == 0


def test_budget_ties_follow_the_flat_order(oracle):
    conf = np.full((3, 2), 1.0, dtype=np.float32)
    cost = np.array([1.0, 0.5, 0.5, 0.5, 10.0, 10.0, 10.0])  # best: exactly 3 drafts
    r = oracle.av_budget(conf, cost)
    assert r["budget"] == 1 or r["budget"] == 3
    assert r["budget"] == 3 and r["kept_len"].tolist() == [2, 1, 0]


# ---------------------------------------------------------------------------
# Prompt-lookup drafting
# ---------------------------------------------------------------------------
def _pad(rows, S=None):
    S = S or max(len(r) for r in rows)
    ctx = np.full((len(rows), S), -7, dtype=np.int32)
    for i, r in enumerate(rows):
        ctx[i, :len(r)] = r
    return ctx, np.array([len(r) for r in rows], dtype=np.int32)


def test_ngram_hand_cases(oracle):
    ctx, ln = _pad([[1, 2, 3, 4, 1, 2, 3],          # 3-gram at 0 -> 4 1 2
                    [5, 1, 2, 7, 1, 2, 8, 1, 2],    # latest 2-gram at 4 -> 8 1 2
                    [9, 8, 7, 6],                   # nothing repeats
                    [3, 1, 2, 3, 4, 4, 1, 2, 3],    # 3-gram (at 1) beats the later 2-gram
                    [4, 5, 4, 5]])                  # continuation cut at the context end
    r = oracle.ngram_propose(ctx, ln, 2, 3, 3)
    assert r["draft"].tolist() == [[4, 1, 2], [8, 1, 2], [-1, -1, -1], [4, 4, 1], [4, 5, -1]]
    assert r["draft_len"].tolist() == [3, 3, 0, 3, 2]
    assert r["match_pos"].tolist() == [0, 4, -1, 1, 0]
    assert r["match_n"].tolist() == [3, 2, 0, 3, 2]


def test_ngram_matches_python_substring_search(oracle):
    # Tokens over a 3-letter alphabet as characters: the latest earlier
    # occurrence of the length-g suffix is str.rfind over s[:n-1].
    rng = np.random.default_rng(10)
    rows = [rng.integers(0, 3, rng.integers(1, 40)).tolist() for _ in range(300)]
    ctx, ln = _pad(rows, 48)
    n_min, n_max, K = 1, 4, 5
    r = oracle.ngram_propose(ctx, ln, n_min, n_max, K)
    for i, row in enumerate(rows):
        s = "".join(chr(65 + t) for t in row)
        n = len(s)
        want_pos, want_g = -1, 0
        for g in range(n_max, n_min - 1, -1):
            if g >= n:
                continue
            p = s.rfind(s[n - g:], 0, n - 1)
            if p >= 0:
                want_pos, want_g = p, g
                break
        cont = row[want_pos + want_g: want_pos + want_g + K] if want_pos >= 0 else []
        assert r["match_pos"][i] == want_pos and r["match_n"][i] == want_g
        assert r["draft_len"][i] == len(cont)
        assert r["draft"][i].tolist() == cont + [-1] * (K - len(cont))
