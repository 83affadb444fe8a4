"""Pins of the oracle's boundary-case flags: the near-ties where a float32
device computation may legitimately decide the other way, which the parity
tests forgive and which the verifier must keep below 1e-4 of its rows.

  NEAR_ACCEPT     |u_j - p/q| < 1e-5 at an evaluated accept test (page
                  "Speculative Decoding: ...", section "Математика верификации");
  NEAR_RACE       the two largest race keys w/E within 1e-6 relative;
  RESIDUAL_EMPTY  max(0, p - q) vanished, the draw fell back to p;
  NEAR_GATE       |h_j - theta| < 1e-5 at an evaluated FLy gate (page
                  "Training-Free Loosely Speculative Decoding...", part A).

Each flag is pinned by inputs built so that the distance behind it is known
by construction (from the separately pinned Philox uniforms), once just
inside and once well outside its threshold.  The estimator diagnostics' and
the budget's near flags are pinned the same way.
"""
import math

import numpy as np
import pytest

SEED = 11


def _E(oracle, x, pos, b, seed=SEED):
    """E_x = -ln u_x of the race's pinned uniform for id x."""
    return -math.log(oracle.race_uniform(seed, x, pos, b))


# ---------------------------------------------------------------------------
# NEAR_RACE: the relative gap of the two largest keys, k = w / E
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("delta", [1e-7, 1e-3])
@pytest.mark.parametrize("order", ["second_best_first", "best_first", "third_first",
                                   "best_third_second"])
def test_race_gap_of_the_two_largest_keys(oracle, delta, order):
    # Three positive weights with designed keys 1 (third), 1.5 (second) and
    # 1.5 (1 + delta) (best), placed at ids in four orders: a mistake in the
    # second-largest bookkeeping (a best that arrives after the second, a
    # smaller key after both) fails one of them.
    V, pos, b = 12, 3, 5
    keys = {"best": 1.5 * (1 + delta), "second": 1.5, "third": 1.0}
    ids = {"second_best_first": {"second": 2, "best": 6, "third": 9},
           "best_first": {"best": 1, "second": 4, "third": 10},
           "third_first": {"third": 0, "second": 5, "best": 11},
           "best_third_second": {"best": 3, "third": 7, "second": 8}}[order]
    w = np.zeros(V)
    for name, x in ids.items():
        w[x] = keys[name] * _E(oracle, x, pos, b)
    y, gap = oracle.race(w, SEED, pos, b)
    assert y == ids["best"]
    assert gap == pytest.approx(delta / (1 + delta), rel=1e-6)  # (k1 - k2) / k1


def test_race_gap_single_and_no_candidate(oracle):
    w = np.zeros(10)
    w[4] = 0.3
    assert oracle.race(w, SEED, 0, 0) == (4, 1.0)  # no second key: k2 = 0
    y, gap = oracle.race(np.zeros(10), SEED, 0, 0)
    assert y == -1 and math.isnan(gap)


def _bonus_rows(oracle, la, lb, ia=3, ib=9, V=16):
    """K = 1, draft row = target row 0 (the draft is always accepted), so the
    step ends with a draw from p at row 1, whose only finite logits are
    la at id ia and lb at id ib."""
    t = np.full((1, 2, V), -np.inf, dtype=np.float32)
    t[0, 0] = np.linspace(-1, 1, V, dtype=np.float32)
    t[0, 1, ia] = la
    t[0, 1, ib] = lb
    d = t[:, :1].copy()
    return t, d, np.array([[5]], dtype=np.int32)


@pytest.mark.parametrize("delta", [1e-7, 1e-3])
@pytest.mark.parametrize("ia_wins", [True, False])
def test_near_race_flag_end_to_end(oracle, delta, ia_wins):
    # Logits set so that p_a / E_a = (1 + delta) p_b / E_b (or the other way
    # round): the race at row 1 (position 1, sequence 0) is a near-tie when
    # delta = 1e-7 and clear when delta = 1e-3.
    ia, ib = 3, 9
    Ea, Eb = _E(oracle, ia, 1, 0), _E(oracle, ib, 1, 0)
    s = 1.0 if ia_wins else -1.0
    la = np.float32(math.log(Ea / Eb) + s * math.log1p(delta))
    t, d, x = _bonus_rows(oracle, la, 0.0, ia, ib)
    r = oracle.verify(t, d, x, SEED)
    assert r["accepted_len"][0] == 1
    assert r["tokens"][0, 1] == (ia if ia_wins else ib)
    # the float32 logit carries a rounding of at most 2.4e-7 in the key ratio
    assert abs(r["race_gap"][0] - delta / (1 + delta)) < 2.5e-7
    near = bool(r["boundary"][0] & oracle.NEAR_RACE)
    assert near == (delta < 1e-6)


# ---------------------------------------------------------------------------
# RESIDUAL_EMPTY: a rejection where max(0, p - q) is zero everywhere
# ---------------------------------------------------------------------------
def test_residual_empty_falls_back_to_p(oracle):
    # Identical target and draft rows and an out-of-range draft token: the
    # token has p = q = 0 and is rejected, and p - q is exactly 0 at every id,
    # so the replacement is drawn from p itself (never a masked id).
    rng = np.random.default_rng(2)
    B, K, V = 16, 2, 40
    t = rng.standard_normal((B, K + 1, V)).astype(np.float32)
    t[:, :, ::4] = -np.inf
    d = t[:, :K].copy()
    x = np.full((B, K), V + 3, dtype=np.int32)
    r = oracle.verify(t, d, x, SEED)
    assert np.all(r["accepted_len"] == 0)
    assert np.all(r["boundary"] & oracle.RESIDUAL_EMPTY)
    y = r["tokens"][:, 0]
    assert np.all(y % 4 != 0) and np.all((y >= 0) & (y < V))
    # the fallback is the draw from p: the same token as an accepted step's
    # draw at that row would give, i.e. the race over p at (position 0, b)
    for b in range(B):
        p = oracle.row_probs(t[b, 0])
        assert y[b] == oracle.race(p, SEED, 0, b)[0]


def test_no_residual_flag_on_ordinary_rejections(oracle):
    rng = np.random.default_rng(3)
    B, K, V = 64, 3, 50
    t = (rng.standard_normal((B, K + 1, V)) * 2).astype(np.float32)
    d = (rng.standard_normal((B, K, V)) * 2).astype(np.float32)
    x = rng.integers(0, V, size=(B, K)).astype(np.int32)
    r = oracle.verify(t, d, x, SEED)
    assert (r["accepted_len"] < K).any()
    assert not np.any(r["boundary"] & oracle.RESIDUAL_EMPTY)


# ---------------------------------------------------------------------------
# NEAR_ACCEPT: the distance |u - p/q| behind it
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("off", [3e-6, -3e-6, 2e-4])
def test_accept_gap_by_construction(oracle, off):
    # p(x_0)/q(x_0) set to u_0 + off, with u_0 the accept test's pinned uniform
    u0 = oracle.uniform(SEED, 0, 0, 0, oracle.TAG_ACCEPT)
    V = 4
    q = np.full(V, 0.25)
    p = np.array([0.25 * (u0 + off), 0, 0, 0])
    p[1:] = (1 - p[0]) / 3
    with np.errstate(divide="ignore"):
        tl = np.log(p).astype(np.float32)
        dl = np.log(q).astype(np.float32)
    t = np.stack([tl, tl])[None]
    r = oracle.verify(t, dl[None, None], np.zeros((1, 1), dtype=np.int32), SEED)
    # float32 logits move the ratio by at most ~1e-7
    assert abs(r["accept_gap"][0] - abs(off)) < 2e-7
    assert r["accepted_len"][0] == (1 if off > 0 else 0)
    assert bool(r["boundary"][0] & oracle.NEAR_ACCEPT) == (abs(off) < 1e-5)


def test_accept_gap_counts_only_evaluated_tests(oracle):
    # After the first rejection no test is evaluated: a near-tie at a later
    # position is not a boundary case.  Position 0 rejects surely (p(x_0) = 0);
    # position 1's ratio sits 3e-6 above its uniform.
    u1 = oracle.uniform(SEED, 0, 1, 0, oracle.TAG_ACCEPT)
    V = 4
    q = np.full(V, 0.25)
    p1 = np.array([0.25 * (u1 + 3e-6), 0, 0, 0])
    p1[1:] = (1 - p1[0]) / 3
    with np.errstate(divide="ignore"):
        row1 = np.log(p1).astype(np.float32)
    row0 = np.log(np.full(V, 0.25)).astype(np.float32)
    row0[0] = -np.inf
    t = np.stack([row0, row1, row1])[None]
    d = np.log(np.stack([q, q])).astype(np.float32)[None]
    x = np.zeros((1, 2), dtype=np.int32)
    r = oracle.verify(t, d, x, SEED)
    assert r["accepted_len"][0] == 0
    assert not (r["boundary"][0] & oracle.NEAR_ACCEPT)
    u0 = oracle.uniform(SEED, 0, 0, 0, oracle.TAG_ACCEPT)
    assert r["accept_gap"][0] == u0  # |u_0 - 0|: the only test evaluated
    # with position 0 always accepted, position 1's near-tie counts
    t[0, 0] = np.log(q).astype(np.float32)  # p = q at position 0: ratio 1
    r = oracle.verify(t, d, x, SEED)
    assert r["accepted_len"][0] == 2
    assert r["boundary"][0] & oracle.NEAR_ACCEPT
    assert abs(r["accept_gap"][0] - 3e-6) < 2e-7


# ---------------------------------------------------------------------------
# NEAR_GATE: the distance |h - theta| at the gates the scan evaluates
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("off", [5e-6, -5e-6, 1e-3, -1e-3])
def test_near_gate_at_an_evaluated_deviation(oracle, off):
    theta, W = 0.3, 4
    dev = np.array([0, 0, 1, 0, 0, 0, 0, 0])
    h = np.full(8, 0.5)
    h[2] = theta + off
    n, near, gap = oracle.fly_resolve(dev, h, W, theta)
    assert n == (8 if off > 0 else 2)        # 2 + 4 <= 7: the window fits
    assert gap == pytest.approx(abs(off), rel=1e-9)
    assert near == (abs(off) < 1e-5)


def test_near_gate_ignores_gates_never_evaluated(oracle):
    theta, W = 0.3, 2
    # a match at theta is no gate; a deviation after the rejection is never reached
    dev = np.array([0, 1, 0, 1, 0, 0])
    h = np.array([theta, 0.1, 0.5, theta, 0.5, 0.5])
    n, near, gap = oracle.fly_resolve(dev, h, W, theta)
    assert n == 1 and not near and gap == pytest.approx(0.2, rel=1e-12)
    # nor is a deviation inside an accepted deviation's skipped window (the
    # window holds matches only); here position 5 is the next deviation seen
    dev = np.array([1, 0, 0, 0, 0, 1])
    h = np.array([0.6, theta, theta, 0.5, 0.5, theta + 2e-6])
    n, near, gap = oracle.fly_resolve(dev, h, W, theta)
    assert n == 5 and near and gap == pytest.approx(2e-6, rel=1e-6)
    n, near, gap = oracle.fly_resolve(np.zeros(6, dtype=np.int32), h, W, theta)
    assert n == 6 and not near and math.isinf(gap)


@pytest.mark.parametrize("off", [5e-6, 1e-3])
def test_near_gate_flag_end_to_end(oracle, off):
    # a flat target row (high entropy) at position 1 with a deviating draft;
    # theta placed `off` below that row's entropy
    rng = np.random.default_rng(5)
    K, V = 4, 3000
    t = (rng.standard_normal((1, K + 1, V)) * 0.5).astype(np.float32)
    st = oracle.rows_stats(t[0])
    x = st["argmax"][:K].astype(np.int32).copy()[None]
    x[0, 1] = (st["argmax"][1] + 1) % V
    theta = float(st["h"][1]) - off
    r = oracle.verify(t, None, x, 0, oracle.MODE_FLY, theta=theta, window=1)
    assert r["accepted_len"][0] == K
    assert r["gate_gap"][0] == pytest.approx(off, rel=1e-6)
    assert bool(r["boundary"][0] & oracle.NEAR_GATE) == (off < 1e-5)


# ---------------------------------------------------------------------------
# Diagnostics' bin-edge flag and the budget's near-tie flag
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("f,nbins,edge", [(0.0, 10, True), (0.0, 4, True), (0.3, 10, False),
                                          (math.log(0.3 / 0.7), 10, True)])
def test_diagnostics_bin_edge_flag(oracle, f, nbins, edge):
    # s = sigmoid(f) with omega = 1, beta = 0: 0.5 and 0.3 sit on bin edges
    feat = np.array([[f], [2.0]])
    d = oracle.av_diagnostics(feat, np.array([1, 0], dtype=np.int32),
                              np.ones(2, dtype=np.int32), np.array([1.0, 0.0]), nbins=nbins)
    assert d["near_bin_edge"] == edge


@pytest.mark.parametrize("cost1,near,budget", [(1.5, True, 0), (1.4, False, 1)])
def test_budget_near_flag(oracle, cost1, near, budget):
    # survivals 0.5, 0.25; expected tokens 1, 1.5, 1.75 (n_requests 1): with
    # cost 1.5 for one draft the first two ratios tie exactly at 1
    conf = np.array([[0.5, 0.5]], dtype=np.float32)
    r = oracle.av_budget(conf, np.array([1.0, cost1, 2.0]), n_requests=1.0)
    assert r["near"] == near and r["budget"] == budget
