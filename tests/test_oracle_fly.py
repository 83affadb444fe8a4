"""Pins of the oracle's FLy resolver (entropy gate + deferral window).

The resolver is a scan; it is pinned against an independently stated,
non-procedural characterisation of the same rule, exhaustively, and against
hand-built decision tables and the special cases the rule reduces to.

Characterisation: since an accepted deviation's window contains no other
deviation, no deviation is ever skipped by the scan, so the first rejected
position is the first deviation j that is not *admissible*, where admissible
means h_j >= theta, the window j+1..j+W fits inside the draft (j + W <= L-1),
and no position in that window deviates.
"""
import itertools

import numpy as np
import pytest


def first_inadmissible(dev, h, W, theta):
    L = len(dev)
    bad = [j for j in range(L)
           if dev[j] and not (h[j] >= theta and j + W <= L - 1
                              and not any(dev[j + 1:j + W + 1]))]
    return min(bad) if bad else L


@pytest.mark.parametrize("L", range(0, 9))
@pytest.mark.parametrize("W", [0, 1, 2, 4, 8])
def test_exhaustive_against_characterisation(oracle, L, W):
    theta = 0.3
    for dev in itertools.product([0, 1], repeat=L):
        # the gate only matters at deviations: enumerate high/low per deviation
        devpos = [j for j in range(L) if dev[j]]
        for gates in itertools.product([0.1, 0.7], repeat=len(devpos)):
            h = np.full(L, 0.5)
            h[devpos] = gates
            n = oracle.fly_resolve(np.array(dev), h, W, theta)[0]
            assert n == first_inadmissible(dev, list(h), W, theta), (dev, list(h), W)


# Hand-built decision tables from the rule's prose: (deviation pattern, gate
# pattern H = high entropy / L = low, W) -> accepted count, K = 8.
TABLE = [
    ("........", "HHHHHHHH", 4, 8),   # exact match everywhere
    ("..x.....", "LLLLLLLL", 4, 2),   # confident target: reject at once
    ("..x.....", "LLHLLLLL", 4, 8),   # uncertain, clean window of 4: accept
    ("..x..x..", "LLHLLHLL", 4, 2),   # second deviation inside window: retroactive
    ("..x...x.", "LLHLLLHL", 4, 2),   # position 6 is the window's last slot
    ("..x....x", "LLHLLLLH", 4, 7),   # second deviation after window: its window overflows
    ("....x...", "HHHHHHHH", 4, 4),   # 4 + 4 > 7: window cannot be filled
    ("...x....", "HHHHHHHH", 4, 8),   # 3 + 4 = 7: exactly fits
    ("x.......", "HHHHHHHH", 0, 8),   # W = 0: any uncertain deviation accepted
    ("xxxxxxxx", "HHHHHHHH", 0, 8),
    ("xxxxxxxx", "HHHLHHHH", 0, 3),
    (".x......", "HHHHHHHH", 6, 8),   # 1 + 6 = 7 fits
    (".x......", "HHHHHHHH", 7, 1),   # 1 + 7 > 7
]


@pytest.mark.parametrize("devs,gates,W,expect", TABLE)
def test_decision_table(oracle, devs, gates, W, expect):
    dev = np.array([c == "x" for c in devs], dtype=np.int32)
    h = np.array([0.9 if c == "H" else 0.05 for c in gates])
    assert oracle.fly_resolve(dev, h, W, 0.3)[0] == expect


def test_theta_above_one_is_strict_greedy(oracle):
    rng = np.random.default_rng(1)
    for _ in range(500):
        L = int(rng.integers(0, 10))
        dev = rng.integers(0, 2, L)
        h = rng.random(L)  # normalised entropy lies in [0, 1]
        W = int(rng.integers(0, 5))
        first = int(np.argmax(dev)) if dev.any() else L
        assert oracle.fly_resolve(dev, h, W, 1.01)[0] == first


def test_zero_window_nonpositive_theta_accepts_all(oracle):
    rng = np.random.default_rng(2)
    for _ in range(200):
        L = int(rng.integers(0, 10))
        assert oracle.fly_resolve(rng.integers(0, 2, L), rng.random(L), 0, 0.0)[0] == L


def _fly_rows(K, V, peaked, peak_ids, peak=16.0, seed=0):
    rng = np.random.default_rng(seed)
    t = rng.standard_normal((1, K + 1, V)).astype(np.float32)
    for j in range(K + 1):
        if peaked[j]:
            t[0, j, peak_ids[j]] += peak
    return t


def test_end_to_end_fly(oracle):
    K, V = 8, 4096
    peaked = [1, 1, 0, 1, 1, 1, 1, 1, 1]
    ids = [10 * (j + 1) for j in range(K + 1)]
    t = _fly_rows(K, V, peaked, ids)
    st = oracle.rows_stats(t[0])
    am = st["argmax"]
    assert list(am[np.array(peaked) == 1]) == [ids[j] for j in range(K + 1) if peaked[j]]
    # flat rows are high entropy, +16 peaks are low entropy
    assert st["h"][2] > 0.9 and st["h"][0] < 0.1
    x = am[:K].astype(np.int32).copy()
    x[2] = (am[2] + 1) % V  # deviation at a flat (uncertain) row, clean window
    r = oracle.verify(t, None, x[None], 0, oracle.MODE_FLY, theta=0.3, window=4)
    assert r["accepted_len"][0] == K
    assert r["tokens"][0, K] == am[K]  # bonus is the target's top token
    x[5] = (am[5] + 1) % V  # second deviation inside the window: reject at 2
    r = oracle.verify(t, None, x[None], 0, oracle.MODE_FLY, theta=0.3, window=4)
    assert r["accepted_len"][0] == 2
    assert list(r["tokens"][0]) == [x[0], x[1], am[2]] + [-1] * (K - 2)
    x = am[:K].astype(np.int32).copy()
    x[1] = (am[1] + 1) % V  # deviation at a confident row: reject now
    r = oracle.verify(t, None, x[None], 0, oracle.MODE_FLY, theta=0.3, window=4)
    assert r["accepted_len"][0] == 1 and r["tokens"][0, 1] == am[1]
    # FLy needs no draft logits and draws no randomness
    r2 = oracle.verify(t, None, x[None], 999, oracle.MODE_FLY, theta=0.3, window=4)
    assert np.array_equal(r["tokens"], r2["tokens"])
