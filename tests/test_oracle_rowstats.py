"""Pins of the oracle's per-row statistics: closed forms, special cases and
independent library routines (scipy's logsumexp and entropy)."""
import math

import numpy as np
import pytest
from scipy import special, stats


def bf16_bits(x):
    """Round float32 values to bfloat16 (nearest-even) and return the bits."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def bits_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32)


@pytest.mark.parametrize("V", [2, 8, 1000, 32000])
@pytest.mark.parametrize("c", [0.0, -3.25, 7.5])
def test_uniform_row(oracle, V, c):
    st = oracle.rows_stats(np.full((1, V), c, dtype=np.float32))
    assert st["h"][0] == pytest.approx(1.0, abs=1e-12)
    assert st["lse"][0] == pytest.approx(c + math.log(V), abs=1e-12)
    assert st["qmax"][0] == pytest.approx(1.0 / V, rel=1e-12)
    assert st["feat"][0] == pytest.approx(-math.log(V - 1), abs=1e-12)
    assert st["argmax"][0] == 0  # all tied: lowest id


def test_one_hot_row(oracle):
    row = np.full((1, 4096), -np.inf, dtype=np.float32)
    row[0, 1234] = 2.5
    st = oracle.rows_stats(row)
    assert st["h"][0] == 0.0
    assert st["lse"][0] == 2.5
    assert st["qmax"][0] == 1.0
    assert st["argmax"][0] == 1234
    assert st["feat"][0] == pytest.approx(126 * math.log(2), rel=1e-15)  # clamp


@pytest.mark.parametrize("a,V,alpha,beta", [(1, 10, 3.0, 0.0), (5, 100, 1.0, -2.0),
                                            (3, 32000, 8.0, 0.5), (64, 128256, -1.0, -9.0)])
def test_two_level_row(oracle, a, V, alpha, beta):
    # a entries of alpha, V-a of beta: lse, H, q_max, logit(q_max) in closed form.
    row = np.full((1, V), beta, dtype=np.float32)
    ids = np.linspace(V // 3, V - 1, a).astype(int)
    row[0, ids] = alpha
    Z = a * math.exp(alpha) + (V - a) * math.exp(beta)
    pa, pb = math.exp(alpha) / Z, math.exp(beta) / Z
    H = -(a * pa * math.log(pa) + (V - a) * pb * math.log(pb))
    st = oracle.rows_stats(row)
    assert st["lse"][0] == pytest.approx(math.log(Z), rel=1e-13)
    assert st["H"][0] == pytest.approx(H, rel=1e-11)
    assert st["h"][0] == pytest.approx(H / math.log(V), rel=1e-11)
    assert st["argmax"][0] == (ids.min() if alpha > beta else 0)
    qmax = max(pa, pb)
    assert st["qmax"][0] == pytest.approx(qmax, rel=1e-12)
    assert st["feat"][0] == pytest.approx(math.log(qmax) - math.log1p(-qmax), rel=1e-10, abs=1e-12)


@pytest.mark.parametrize("T", [1.0, 0.7, 2.0])
def test_random_rows_vs_scipy(oracle, T):
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((6, 5003)) * 3).astype(np.float32)
    x[2, ::7] = -np.inf  # masked vocabulary
    st = oracle.rows_stats(x, temperature=T)
    z = x.astype(np.float64) / T
    assert np.allclose(st["lse"], special.logsumexp(z, axis=1), rtol=1e-13, atol=0)
    p = special.softmax(z, axis=1)
    assert np.allclose(st["H"], stats.entropy(p, axis=1), rtol=1e-11)
    assert np.allclose(st["h"], stats.entropy(p, axis=1) / math.log(5003), rtol=1e-11)
    assert np.array_equal(st["argmax"], np.argmax(z, axis=1))
    assert np.allclose(st["qmax"], p.max(axis=1), rtol=1e-12)
    q = p.max(axis=1)
    assert np.allclose(st["feat"], special.logit(q), rtol=1e-9)


def _exact_stats(row, T):
    """lse, H and logit(q_max) of one row in 60-digit decimal arithmetic."""
    import decimal
    D = decimal.Decimal
    ctx = decimal.Context(prec=60)
    z = [ctx.divide(D(float(v)), D(float(T))) for v in row if np.isfinite(v)]
    m = max(z)
    e = [ctx.exp(zi - m) for zi in z]
    s = ctx.add(sum(e, D(0)), D(0))
    r = s - 1  # the maximum contributes exp(0) = 1 (no tie at the top)
    ln_s = ctx.ln(s)
    H = sum((ei / s) * (ln_s - (zi - m)) for ei, zi in zip(e, z))
    return float(m + ln_s), float(H), float(-ctx.ln(r))


@pytest.mark.parametrize("peak,T", [(40.0, 1.0), (30.0, 0.7), (25.0, 1.0), (8.0, 1.0)])
def test_entropy_of_peaked_rows_is_accurate(oracle, peak, T):
    # Near-one-hot rows: H and 1 - q_max are ~1e-13; relative accuracy must hold.
    rng = np.random.default_rng(int(peak))
    x = (rng.standard_normal((1, 997)) * 3).astype(np.float32)
    x[0, 17] += np.float32(peak)
    st = oracle.rows_stats(x, temperature=T)
    lse, H, feat = _exact_stats(x[0], T)
    assert st["lse"][0] == pytest.approx(lse, rel=1e-14)
    assert st["H"][0] == pytest.approx(H, rel=1e-9)
    assert st["feat"][0] == pytest.approx(feat, rel=1e-12)


def test_entropy_closed_form_near_one_hot(oracle):
    # one logit 40, 999 logits 0: r = 999 e^-40, H = log1p(r) + 40 r / (1 + r)
    x = np.zeros((1, 1000), dtype=np.float32)
    x[0, 17] = 40.0
    st = oracle.rows_stats(x)
    r = 999 * math.exp(-40.0)
    assert st["H"][0] == pytest.approx(math.log1p(r) + 40.0 * r / (1 + r), rel=1e-12)
    assert st["feat"][0] == pytest.approx(40.0 - math.log(999), rel=1e-14)
    assert st["lse"][0] == pytest.approx(40.0 + math.log1p(r), rel=1e-15)


def test_bf16_decoding(oracle):
    vals = np.array([1.0, -2.0, 0.5, 3.140625, -np.inf, 100.0], dtype=np.float32)
    bits = bf16_bits(vals)
    assert list(bits[:5]) == [0x3F80, 0xC000, 0x3F00, 0x4049, 0xFF80]
    row = np.zeros((1, 8), dtype=np.uint16)
    row[0, :6] = bits
    st = oracle.rows_stats(row)
    z = np.zeros(8)
    z[:6] = bits_to_f32(bits)
    assert st["lse"][0] == pytest.approx(special.logsumexp(z), rel=1e-14)
    assert st["argmax"][0] == 5


def test_temperature_is_a_rescale(oracle):
    # Stats at T = 0.5 of l equal stats at T = 1 of 2l (exact in float32).
    rng = np.random.default_rng(9)
    x = rng.standard_normal((3, 777)).astype(np.float32)
    a = oracle.rows_stats(x, temperature=0.5)
    b = oracle.rows_stats((2 * x).astype(np.float32), temperature=1.0)
    for k in ("lse", "H", "qmax", "feat"):
        assert np.allclose(a[k], b[k], rtol=1e-14)
    assert np.array_equal(a["argmax"], b["argmax"])


def test_argmax_ties_lowest_id(oracle):
    x = np.zeros((2, 50), dtype=np.float32)
    x[0, [9, 3, 40]] = 5.0
    x[1, [49, 48]] = 1.0
    st = oracle.rows_stats(x)
    assert list(st["argmax"]) == [3, 48]
    # A tie at the top puts the other maximum into 1 - q_max: logit <= 0.
    assert st["feat"][0] < 0


def test_padded_stride(oracle):
    rng = np.random.default_rng(2)
    x = rng.standard_normal((4, 40)).astype(np.float32)
    st_full = oracle.rows_stats(np.ascontiguousarray(x[:, :33]))
    st_pad = oracle.rows_stats(x, V=33)
    for k in ("lse", "H", "qmax", "feat"):
        assert np.array_equal(st_full[k], st_pad[k])
