"""Pins of the oracle's Philox4x32-10 and of the uniform lattice built on it.

Philox is pinned to (1) the published known-answer vectors and (2) rocRAND's
independent host-callable implementation on random keys and counters.
"""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest
from scipy import stats

HERE = os.path.dirname(os.path.abspath(__file__))


def _kat_rows():
    rows = []
    with open(os.path.join(HERE, "golden", "philox4x32_10_kat.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            v = [int(t, 16) for t in line.split()]
            rows.append((v[0:4], v[4:6], v[6:10]))
    return rows


@pytest.mark.parametrize("ctr,key,expect", _kat_rows())
def test_philox_known_answers(oracle, ctr, key, expect):
    assert list(oracle.philox4x32_10(ctr, key)) == expect


@pytest.fixture(scope="module")
def rocrand_dump():
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc) or not os.path.exists("/opt/rocm/include/rocrand"):
        pytest.skip("hipcc / rocRAND headers not available")
    d = tempfile.mkdtemp(prefix="philox_pin_")
    exe = os.path.join(d, "dump")
    subprocess.check_call([hipcc, "-O1", os.path.join(HERE, "helpers", "rocrand_philox_dump.cpp"),
                           "-o", exe], stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    yield exe
    shutil.rmtree(d, ignore_errors=True)


def test_philox_matches_rocrand(oracle, rocrand_dump):
    rng = np.random.default_rng(123)
    cases = rng.integers(0, 2**32, size=(400, 6), dtype=np.uint64)
    cases[:8, 4:] = 0
    cases[8:16, :4] = 0xFFFFFFFF
    lines = []
    for c in cases:
        key = int(c[4]) | (int(c[5]) << 32)
        lines.append("%d %d %d %d %d" % (key, c[0], c[1], c[2], c[3]))
    out = subprocess.run([rocrand_dump], input="\n".join(lines) + "\n", capture_output=True,
                         text=True, check=True).stdout.split("\n")
    for c, o in zip(cases, out):
        got = oracle.philox4x32_10([int(v) for v in c[:4]], [int(c[4]), int(c[5])])
        assert [int(t) for t in o.split()] == list(got)


def test_draw_counter_layout(oracle):
    # Word x&3 of the block at counter (x>>2, pos, b, tag), key = seed halves.
    seed = 0x0123456789ABCDEF
    for x, pos, b, tag in [(0, 0, 0, 1), (5, 3, 7, 2), (131071, 8, 1023, 2), (2, 4, 99, 1)]:
        block = oracle.philox4x32_10([x >> 2, pos, b, tag], [seed & 0xFFFFFFFF, seed >> 32])
        assert oracle.draw_u32(seed, x, pos, b, tag) == int(block[x & 3])


def test_uniform_lattice(oracle):
    # u = (2*(r>>9)+1)/2^24: odd multiples of 2^-24, strictly inside (0, 1).
    us = np.array([oracle.uniform(7, x, 0, 0, 2) for x in range(4096)])
    k = us * 2**24
    assert np.all(k == np.round(k)) and np.all(np.round(k) % 2 == 1)
    assert us.min() > 0 and us.max() < 1
    # The largest and smallest lattice points.
    assert (2 * (0xFFFFFFFF >> 9) + 1) / 2**24 == 1 - 2**-24


def test_uniform_is_uniform(oracle):
    us = np.array([oracle.uniform(11, x, 3, 5, 2) for x in range(200000)])
    assert stats.kstest(us, "uniform").pvalue > 1e-3
    # Different tags / positions / sequences give unrelated streams.
    a = np.array([oracle.uniform(11, x, 3, 5, 1) for x in range(20000)])
    assert abs(np.corrcoef(a, us[:20000])[0, 1]) < 0.03


def test_accept_probability_by_lattice_count():
    # P(u < r) over the lattice equals min(1, r) to within 2^-24 (exact count).
    for r in [0.0, 1e-9, 0.125, 0.3, 0.625, 0.999999, 1.0, 1.5, 7.0]:
        k = np.arange(2**23, dtype=np.float64)
        frac = np.count_nonzero((2 * k + 1) / 2**24 < r) / 2**23
        assert abs(frac - min(1.0, r)) <= 2**-24


def test_race_word_layout(oracle):
    # The race's word for id x: high 16 bits from the screening stream (half
    # x&1 of word (x>>1)&3 of the block at counter (x>>3, pos, b, 3)), low 16
    # bits the high half of the race stream's draw (word x&3 of the block at
    # counter (x>>2, pos, b, 2)); both blocks from the pinned Philox.
    seed = 0x0123456789ABCDEF
    key = [seed & 0xFFFFFFFF, seed >> 32]
    for x, pos, b in [(0, 0, 0), (1, 0, 0), (7, 3, 9), (8, 3, 9), (13, 8, 1023),
                      (131071, 2, 77), (152063, 4, 511)]:
        s = oracle.philox4x32_10([x >> 3, pos, b, oracle.TAG_SCREEN], key)
        r = oracle.philox4x32_10([x >> 2, pos, b, oracle.TAG_RACE], key)
        hi = (int(s[(x >> 1) & 3]) >> (16 * (x & 1))) & 0xFFFF
        assert oracle.race_u32(seed, x, pos, b) == (hi << 16) | (int(r[x & 3]) >> 16)
        k = oracle.race_u32(seed, x, pos, b) >> 9
        assert oracle.race_uniform(seed, x, pos, b) == (2 * k + 1) / 2**24


def test_race_uniform_is_uniform(oracle):
    # Made of two independent streams, the race's uniforms are uniform: a KS
    # test over 200000 ids, leading-one counts with the geometric law the
    # sampler's bound assumes, and no correlation with either stream alone.
    n = 200000
    us = np.array([oracle.race_uniform(5, x, 1, 3) for x in range(n)])
    assert stats.kstest(us, "uniform").pvalue > 1e-3
    words = np.array([oracle.race_u32(5, x, 1, 3) for x in range(n)], dtype=np.uint64)
    ones = np.zeros(n, dtype=np.int64)
    w = words.copy()
    for bit in range(31, -1, -1):  # leading one bits, counted from the top
        still = ones == (31 - bit)
        ones += (still & (((w >> bit) & 1) == 1)).astype(np.int64)
    counts = np.bincount(np.minimum(ones, 8), minlength=9)
    expect = np.array([n * 2.0 ** -(k + 1) for k in range(8)] + [n * 2.0 ** -8])
    assert stats.chisquare(counts, expect).pvalue > 1e-3
    plain = np.array([oracle.uniform(5, x, 1, 3, oracle.TAG_RACE) for x in range(20000)])
    assert abs(np.corrcoef(plain, us[:20000])[0, 1]) < 0.03
    hi = (words >> 16).astype(np.float64)
    lo = (words & 0xFFFF).astype(np.float64)
    assert abs(np.corrcoef(hi, lo)[0, 1]) < 0.01
