"""Pins of the oracle's adaptive-verification scorer, trimming rule, label
set and SGD step."""
import math

import numpy as np
import pytest


def test_no_fit_scorer_is_qmax(oracle):
    # omega = 1, beta = 0 turns sigmoid(logit(q_max)) back into q_max: the
    # page's "no fit" baseline of using the draft's own top probability.
    rng = np.random.default_rng(0)
    d = (rng.standard_normal((12, 300)) * 2).astype(np.float32)
    st = oracle.rows_stats(d)
    K = 4
    feat = st["feat"].reshape(3, K)
    conf, mask, kept, _ = oracle.av_score(feat, np.r_[1.0, np.zeros(K)], 0.0)
    assert np.allclose(conf.ravel(), st["qmax"], rtol=1e-12)
    assert np.all(mask == 1) and np.all(kept == K)  # tau <= 0 keeps everything


def test_scorer_parameter_roles(oracle):
    # K + 1 parameters: beta_i shifts position i only; omega scales the feature.
    B, K = 5, 6
    feat = np.linspace(-3, 3, B * K).reshape(B, K)
    ob = np.r_[0.5, np.linspace(0.5, -1.0, K)]
    c, _, _, _ = oracle.av_score(feat, ob, 0.0)
    for i in range(K):
        ob2 = ob.copy()
        ob2[1 + i] += 0.7
        c2, _, _, _ = oracle.av_score(feat, ob2, 0.0)
        changed = np.any(c2 != c, axis=0)
        assert changed[i] and changed.sum() == 1
    z = 0.5 * feat + ob[1:]
    assert np.allclose(np.log(c / (1 - c)), z, atol=1e-12)  # logit(c) is affine


def test_trimming_threshold_and_prefix(oracle):
    # survival = running product; keep while >= tau (a prefix).
    B, K = 4, 5
    # choose feat so conf is known: omega = 0, beta = logit(c_i)
    cs = np.array([0.9, 0.8, 0.5, 0.99, 0.9])
    ob = np.r_[0.0, np.log(cs / (1 - cs))]
    feat = np.zeros((B, K))
    P = np.cumprod(cs)  # 0.9, 0.72, 0.36, 0.3564, 0.32076
    for tau, L in [(0.95, 0), (0.9 - 1e-9, 1), (0.5, 2), (0.36 - 1e-9, 3), (0.33, 4),
                   (0.3, 5), (0.0, 5)]:
        conf, mask, kept, near = oracle.av_score(feat, ob, tau)
        assert np.allclose(conf[0], cs, atol=1e-12)
        assert np.all(kept == L), (tau, kept, P)
        assert np.all(mask[:, :L] == 1) and np.all(mask[:, L:] == 0)
    _, _, _, near = oracle.av_score(feat, ob, P[2] * (1 + 3e-6))
    assert np.all(near & oracle.NEAR_TRIM)


@pytest.mark.parametrize("acc,kept,labels", [
    (2, 5, [1, 1, 0]), (5, 5, [1, 1, 1, 1, 1]), (0, 5, [0]), (0, 0, []),
    (3, 3, [1, 1, 1]), (1, 4, [1, 0])])
def test_label_set(oracle, acc, kept, labels):
    # Only drafts up to and including the first rejection are labelled.
    K = 5
    feat = np.zeros((1, K))
    ob = np.zeros(K + 1)  # prediction 1/2 everywhere
    loss, n = oracle.av_loss(feat, np.array([acc]), np.array([kept]), ob)
    assert n == len(labels)
    if n:
        assert loss == pytest.approx(math.log(2), rel=1e-15)
    new = oracle.av_update(feat, np.array([acc]), np.array([kept]), ob, lr=1.0)
    # with f = 0 only intercepts move: beta_i -= (1/N) (1/2 - y_i)
    expect = np.zeros(K)
    for i, y in enumerate(labels):
        expect[i] = -(0.5 - y) / len(labels)
    assert new[0] == 0.0
    assert np.allclose(new[1:], expect, atol=1e-15)


def test_sgd_step_is_gradient_of_mean_logloss(oracle):
    rng = np.random.default_rng(3)
    B, K = 40, 6
    feat = rng.standard_normal((B, K)) * 1.5 - 1.0
    acc = rng.integers(0, K + 1, B).astype(np.int32)
    kept = np.maximum(acc, rng.integers(0, K + 1, B)).astype(np.int32)
    kept[::7] = acc[::7]  # some sequences accept everything they kept
    ob = np.r_[1.0, 0.5 - 0.3 * np.arange(K)]
    lr = 0.05
    new = oracle.av_update(feat, acc, kept, ob, lr)
    grad = np.zeros(K + 1)
    h = 1e-6
    for k in range(K + 1):
        e = np.zeros(K + 1)
        e[k] = h
        lp, _ = oracle.av_loss(feat, acc, kept, ob + e)
        lm, _ = oracle.av_loss(feat, acc, kept, ob - e)
        grad[k] = (lp - lm) / (2 * h)
    assert np.allclose(new, ob - lr * grad, atol=1e-9)


def test_update_without_labels_is_a_noop(oracle):
    feat = np.ones((3, 4))
    ob = np.r_[0.3, 0.1, 0.2, 0.3, 0.4]
    new = oracle.av_update(feat, np.zeros(3, np.int32), np.zeros(3, np.int32), ob, 0.05)
    assert np.array_equal(new, ob)


def test_logloss_limits(oracle):
    K = 3
    feat = np.full((2, K), 10.0)
    ob = np.r_[5.0, np.zeros(K)]  # sigmoid(50): certain acceptance
    loss, n = oracle.av_loss(feat, np.array([3, 3]), None, ob)
    assert n == 6 and loss < 1e-20
    loss, n = oracle.av_loss(feat, np.array([0, 0]), None, ob)
    assert n == 2 and loss == pytest.approx(50.0, rel=1e-12)  # -log(1 - sigmoid(50))
