"""GPU parity: the HIP library (through its C ABI) against the CPU oracle on
the same seeded inputs.  Small sizes span several tiles and a ragged tail;
the workload sizes are checked on oracle-computed samples and by properties
that hold at any size."""
import os

import numpy as np
import pytest
import torch

import draft_token_verification_vocab_amd as sv
from draft_token_verification_vocab_amd import workloads as W
from oracle import ref
from parity_util import (REL_TOL, assert_close, check_token_layout, compare_decisions, f32,
                         host_logits, oracle_threads)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
NT = oracle_threads()
ALL_NEAR = ref.NEAR_ACCEPT | ref.NEAR_RACE | ref.RESIDUAL_EMPTY | ref.NEAR_GATE | ref.NEAR_TRIM


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "the GPU tests need an MI355X"
    sv.load()
    ref.lib()


def np_(t):
    return t.detach().cpu().numpy()


# ---------------------------------------------------------------------------
# Row statistics
# ---------------------------------------------------------------------------
def _special_rows(V, dtype, stride, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(10, V, generator=g) * 3.0
    x[0, ::5] = -float("inf")                      # masked vocabulary
    x[1, 77 % V] += 30.0                           # very peaked (tiny entropy)
    x[2] = 0.5                                     # uniform: all tied
    x[3, [V - 1, V // 2]] = x[3].max() + 1.0       # two maxima far apart
    x[4] = -float("inf")
    x[4, V - 1] = 1.0                              # one finite entry, at the tail
    x[5] = torch.linspace(-5, 5, V)                # maximum at the last id
    x[6, :min(V, 3)] = 40.0                        # tie at the very front
    xd = torch.full((10, stride), float("nan"))
    xd[:, :V] = x
    return xd.to(dtype)


# lse is compared relative to max(|lse|, 1) (abs_floor = rel): an error d in
# lse is a relative error d in every probability exp(l/T - lse), and lse
# passes through 0, where a purely relative bound would demand more than that.
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("V,stride", [(2, 8), (9, 16), (1003, 1008), (4097, 4104),
                                      (32000, 32000), (128256, 128256), (152064, 152064)])
@pytest.mark.parametrize("T", [1.0, 0.7])
def test_row_stats_parity(dtype, V, stride, T):
    xh = _special_rows(V, dtype, stride, seed=V + int(T * 10))
    x = xh.to(DEV)
    r = sv.row_stats(x, vocab=V, temperature=T, qmax=True, feat=True)
    torch.cuda.synchronize()
    o = ref.rows_stats(host_logits(xh), temperature=f32(T), V=V, nthreads=NT)
    rel = REL_TOL[dtype]
    assert np.array_equal(np_(r["argmax"]), o["argmax"])
    assert_close(np_(r["lse"]), o["lse"], rel, "lse", abs_floor=rel)
    assert_close(np_(r["entropy"]), o["h"], rel, "entropy", abs_floor=1e-12)
    assert_close(np_(r["qmax"]), o["qmax"], rel, "qmax")
    # logit(q_max) passes through 0: relative to max(|feat|, 1)
    assert_close(np_(r["feat"]), o["feat"], rel, "feat", abs_floor=rel)


@pytest.mark.parametrize("T", [1e-4, 0.05, 5.0, 1e4])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_row_stats_extreme_temperatures(dtype, T):
    # both ends of the accepted temperature range: rows scaled by up to 1e4
    # (one-hot to the last ulp) and down to 1e-4 (near uniform)
    for V, stride in ((1003, 1008), (32000, 32000)):
        xh = _special_rows(V, dtype, stride, seed=V + 5)
        r = sv.row_stats(xh.to(DEV), vocab=V, temperature=T, qmax=True, feat=True)
        torch.cuda.synchronize()
        o = ref.rows_stats(host_logits(xh), temperature=f32(T), V=V, nthreads=NT)
        rel = REL_TOL[dtype]
        assert np.array_equal(np_(r["argmax"]), o["argmax"])
        assert_close(np_(r["lse"]), o["lse"], rel, "lse", abs_floor=rel)
        assert_close(np_(r["entropy"]), o["h"], rel, "entropy", abs_floor=1e-12)
        assert_close(np_(r["qmax"]), o["qmax"], rel, "qmax")
        assert_close(np_(r["feat"]), o["feat"], rel, "feat", abs_floor=rel)


def test_row_stats_reproducible_and_ordered_ties():
    x = torch.zeros(5, 40000, device=DEV, dtype=torch.bfloat16)
    x[0, [39999, 12345, 20000]] = 1.0
    x[1, 1] = -1.0
    # a maximum of zero held by -0 and +0: one value, so the lowest id wins
    # whatever its sign (ids held by different threads and chunks)
    x[3] = -1.0
    x[3, [7, 30001]] = torch.tensor([-0.0, 0.0], dtype=torch.bfloat16, device=DEV)
    x[4] = -1.0
    x[4, [5, 17, 39000]] = torch.tensor([0.0, -0.0, -0.0], dtype=torch.bfloat16, device=DEV)
    a = sv.row_stats(x)
    b = sv.row_stats(x)
    assert torch.equal(a["lse"], b["lse"]) and torch.equal(a["entropy"], b["entropy"])
    assert np_(a["argmax"]).tolist() == [12345, 0, 0, 7, 5]
    o = ref.rows_stats(host_logits(x.cpu()), temperature=1.0, V=40000, nthreads=NT)
    assert np.array_equal(np_(a["argmax"]), o["argmax"])


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_row_stats_ties_inside_one_thread(dtype):
    # equal maxima held by one thread: in different chunks of its row and in
    # different vectors of one chunk (thread 5 and thread 9 at the row pass's
    # shapes: 768 threads x 2 vectors of 8 bfloat16, 512 threads x 4 vectors
    # of 4 floats); the lowest id must win
    block, unroll, epv = (768, 2, 8) if dtype == torch.bfloat16 else (512, 4, 4)
    chunk = block * unroll
    V = 3 * chunk * epv + 96  # rows a multiple of 16 bytes
    x = torch.zeros(3, V, dtype=dtype)
    ids = [(5 + it * chunk) * epv + 3 for it in range(3)]       # chunks 0, 1, 2 of thread 5
    x[0, ids[::-1]] = 2.0
    x[1, [(9 + block) * epv + 1, 9 * epv + 1]] = 2.0             # vectors u = 1 and 0
    x[2, [ids[2], (9 + block) * epv + 1]] = 2.0                  # two threads, later chunks
    r = sv.row_stats(x.to(DEV))
    torch.cuda.synchronize()
    assert np_(r["argmax"]).tolist() == [ids[0], 9 * epv + 1, (9 + block) * epv + 1]
    o = ref.rows_stats(host_logits(x), temperature=1.0, V=V, nthreads=NT)
    assert np.array_equal(np_(r["argmax"]), o["argmax"])


def test_read_probe_folds_every_word():
    # the load-only ceiling kernel reads each row's bytes exactly: XOR per row
    g = torch.Generator().manual_seed(3)
    for rows, S, rb in ((7, 2056, 4112), (3, 128256, 256512), (5, 64, 96)):
        xh = torch.randint(-2**15, 2**15, (rows, S), generator=g, dtype=torch.int16)
        got = np_(sv.read_probe(xh.to(DEV), row_bytes=rb)).view(np.uint32)
        words = xh.numpy().view(np.uint32)[:, :rb // 4]
        assert np.array_equal(got, np.bitwise_xor.reduce(words, axis=1))


# ---------------------------------------------------------------------------
# FLy
# ---------------------------------------------------------------------------
def _fly_check(batch, theta=0.3, window=4, kept=None, kept_ref=None, tally="workload"):
    # kept_ref: the oracle's kept lengths, when the library's are meant to be
    # clamped into [0, K] first (the oracle takes only values in range)
    kept_ref = kept if kept_ref is None else kept_ref
    t = batch.target.to(DEV)
    tok = batch.tokens.to(DEV)
    kept_d = None if kept is None else kept.to(DEV)
    r = sv.verify(t, None, tok, seed=0, mode=sv.MODE_FLY, fly_theta=theta, fly_window=window,
                  vocab=batch.V, kept_len=kept_d, stats=True, boundary=True)
    torch.cuda.synchronize()
    o = ref.verify(host_logits(batch.target), None, np_(batch.tokens), 0, ref.MODE_FLY,
                   theta=f32(theta), window=window, V=batch.V,
                   kept_len=None if kept_ref is None else np_(kept_ref), nthreads=NT)
    nm, nb = compare_decisions(np_(r.accepted_len), np_(r.tokens), o, ref.NEAR_GATE, "fly",
                               dev_boundary=np_(r.boundary),
                               kept=None if kept_ref is None else np_(kept_ref), tally=tally)
    rel = REL_TOL[batch.target.dtype]
    assert np.array_equal(np_(r.target_argmax), o["t_argmax"])
    assert_close(np_(r.target_lse), o["t_lse"], rel, "target lse", abs_floor=rel)
    assert_close(np_(r.target_entropy), o["t_h"], rel, "target entropy", abs_floor=1e-12)
    check_token_layout(np_(r.accepted_len), np_(r.tokens), np_(batch.tokens),
                       None if kept_ref is None else np_(kept_ref))
    return r, o, nm, nb


@pytest.mark.parametrize("B,K,V,stride", [(24, 8, 128256, 128256), (16, 4, 5003, 5008),
                                          (8, 1, 1000, 1000)])
def test_fly_parity(B, K, V, stride):
    batch = W.make(2, B=B, K=K, V=V, stride=stride)
    _fly_check(batch)


def test_fly_workspace_contents_do_not_matter():
    # The workspace's contents on entry do not matter: random bytes there, and
    # what a previous call left, must not change the result.
    batch = W.make(2, B=40, K=6, V=3001, stride=3008)
    t, tok = batch.target.to(DEV), batch.tokens.to(DEV)
    B, K = tok.shape
    need = sv.workspace_bytes(B, K, batch.V, stride=3008)
    assert need > 0
    g = torch.Generator(device="cpu").manual_seed(5)
    want = None
    for trial in range(4):
        ws = torch.randint(0, 256, (need,), generator=g, dtype=torch.uint8).to(DEV)
        if trial == 3:
            ws.zero_()
        for rep in range(2):  # the second call finds the first call's words
            r = sv.verify(t, None, tok, seed=0, mode=sv.MODE_FLY, fly_theta=0.3, fly_window=2,
                          vocab=batch.V, workspace=ws)
            torch.cuda.synchronize()
            got = (np_(r.accepted_len).copy(), np_(r.tokens).copy())
            if want is None:
                want = got
                o = ref.verify(host_logits(batch.target), None, np_(batch.tokens), 0, ref.MODE_FLY,
                               theta=f32(0.3), window=2, V=batch.V, nthreads=NT)
                compare_decisions(got[0], got[1], o, ref.NEAR_GATE, "fly")
            assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])


def test_fly_gate_branches():
    # peaks of +16 make confident rows (h ~ 0.03): the reject-now branch
    batch = W.fly(32, 8, 20000, seed=5, peak=16.0)
    r, o, _, _ = _fly_check(batch)
    assert (o["accepted_len"] < 8).any() and (o["accepted_len"] == 8).any()
    # theta > 1 is strict greedy, W = 0 with theta <= 0 accepts everything
    _fly_check(batch, theta=1.5, window=4)
    r, o, _, _ = _fly_check(batch, theta=0.0, window=0)
    assert np.all(o["accepted_len"] == 8)
    kept = torch.randint(0, 9, (32,), generator=torch.Generator().manual_seed(1), dtype=torch.int32)
    _fly_check(batch, kept=kept)


@pytest.mark.parametrize("window", [0, 1, 3, 62, 63, 64, 1 << 20])
def test_fly_max_drafts_and_windows(window):
    # K = 64, the largest draft length: every lane of the resolver's wave holds
    # a position and the stopping row may be row 64.  High match rates make
    # long windows pass; mixed entropies exercise both gate outcomes.
    batch = W.fly(40, 64, 300, seed=11 + window % 7, stride=304, peak=9.0, p_match=0.97)
    kept = torch.randint(0, 65, (40,), generator=torch.Generator().manual_seed(window % 5),
                         dtype=torch.int32)
    kept[:4] = 64
    for theta in (0.2, 0.6):
        _fly_check(batch, theta=theta, window=window)
        _fly_check(batch, theta=theta, window=window, kept=kept)


def test_fly_headline_full_size():
    # the benchmarked FLy workload at its full size, every output checked
    batch = W.make(2)
    r, o, _, _ = _fly_check(batch)
    assert r.accepted_len.shape[0] == 256 and batch.V == 128256


# ---------------------------------------------------------------------------
# Lossless
# ---------------------------------------------------------------------------
def _lossless_check(batch, seed, kept=None, draft_stats_path=False, kept_ref=None,
                    tally="workload"):
    kept_ref = kept if kept_ref is None else kept_ref
    t = batch.target.to(DEV)
    d = batch.draft.to(DEV)
    tok = batch.tokens.to(DEV)
    kept_d = None if kept is None else kept.to(DEV)
    T = batch.temperature
    ds = None
    if draft_stats_path:
        K = tok.shape[1]
        ob = torch.zeros(K + 1, device=DEV)
        _, _, _, ds = sv.av_score(d, tok, ob, 0.0, temperature=T, vocab=batch.V)
    r = sv.verify(t, d, tok, seed=seed, temperature=T, vocab=batch.V, kept_len=kept_d,
                  draft_stats=ds, stats=True, boundary=True)
    torch.cuda.synchronize()
    o = ref.verify(host_logits(batch.target), host_logits(batch.draft), np_(batch.tokens), seed,
                   temperature=f32(T), V=batch.V,
                   kept_len=None if kept_ref is None else np_(kept_ref), nthreads=NT)
    nm, nb = compare_decisions(np_(r.accepted_len), np_(r.tokens), o, ALL_NEAR, "lossless",
                               dev_boundary=np_(r.boundary),
                               kept=None if kept_ref is None else np_(kept_ref), tally=tally)
    rel = REL_TOL[batch.target.dtype]
    assert np.array_equal(np_(r.target_argmax), o["t_argmax"])
    assert_close(np_(r.target_lse), o["t_lse"], rel, "target lse", abs_floor=rel)
    assert_close(np_(r.target_entropy), o["t_h"], rel, "target entropy", abs_floor=1e-12)
    if not draft_stats_path:
        assert_close(np_(r.draft_lse), o["d_lse"], rel, "draft lse", abs_floor=rel)
        assert_close(np_(r.draft_qmax), o["d_qmax"], rel, "draft qmax")
        assert_close(np_(r.draft_feat), o["d_feat"], rel, "draft feat", abs_floor=rel)
    check_token_layout(np_(r.accepted_len), np_(r.tokens), np_(batch.tokens),
                       None if kept_ref is None else np_(kept_ref))
    return r, o, nm, nb


def test_lossless_c0_full_size():
    batch = W.make(0)
    _lossless_check(batch, seed=0)
    for s in range(1, 40):  # more seeds of the same rows: many residual races
        _lossless_check(batch, seed=s)


@pytest.mark.parametrize("cfg", [1, 3])
def test_lossless_workloads_full_size(cfg):
    # the benchmarked lossless workloads at their full sizes, every output
    # checked: B=64 K=5 V=128256, and B=512 K=4 V=152064 at T=0.7
    batch = W.make(cfg, device=DEV)
    _, o, nm, nb = _lossless_check(batch, seed=0)
    assert batch.tokens.shape[0] == W.CONFIGS[cfg]["B"]


@pytest.mark.parametrize("cfg,B,K,V,stride", [(1, 12, 5, 128256, 128256), (3, 12, 4, 152064, 152064),
                                              (1, 16, 3, 7001, 7008), (0, 32, 4, 32000, 32000),
                                              (3, 8, 2, 1003, 1008)])
def test_lossless_parity(cfg, B, K, V, stride):
    batch = W.make(cfg, B=B, K=K, V=V, stride=stride)
    _, o, nm, nb = _lossless_check(batch, seed=7)
    _lossless_check(batch, seed=8, draft_stats_path=True)


@pytest.mark.parametrize("V,stride", [(2, 8), (3, 8), (9, 16), (17, 24)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_lossless_tiny_vocabularies(dtype, V, stride):
    # rows of one or a few vectors, most of them the partial last one: the
    # race's whole trips are empty and only its last trip runs
    batch = W.gaussian(40, 6, V, dtype, 1.0, seed=V, token_seed=1, stride=stride)
    for seed in range(4):
        _lossless_check(batch, seed=seed)


@pytest.mark.parametrize("T", [1e-4, 0.05, 5.0, 1e4])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_lossless_extreme_temperatures(dtype, T):
    # the race's float screening at keys scaled by up to 1e4, and near-uniform
    # rows where every id is a candidate
    batch = W.gaussian(16, 4, 5003, dtype, T, seed=91, token_seed=3, stride=5008)
    for seed in range(3):
        _lossless_check(batch, seed=seed)


def test_lossless_kept_len_and_bad_tokens():
    batch = W.make(1, B=20, K=5, V=3001, stride=3008)
    batch.tokens[3, 1] = 3001       # outside V: rejected
    batch.tokens[4, 0] = -7
    kept = torch.tensor([0, 1, 2, 3, 4, 5] * 3 + [0, 5], dtype=torch.int32)
    r, o, _, _ = _lossless_check(batch, seed=3, kept=kept)
    assert np_(r.accepted_len)[4] == 0


def test_lossless_masked_vocab():
    batch = W.make(1, B=16, K=3, V=4000)
    batch.target[:, :, ::3] = -float("inf")
    batch.draft[:, :, 1::3] = -float("inf")
    r, o, _, _ = _lossless_check(batch, seed=11)
    tok = np_(r.tokens)
    acc = np_(r.accepted_len)
    for b in range(16):  # an emitted replacement / bonus token never has p = 0
        assert tok[b, acc[b]] % 3 != 0


# A short row (two race segments per sequence at these batch sizes) and a
# long one (34 segments): the segment boundaries and the combine's choice
# among many segments both get exercised.
RACE_SHAPES = [(5003, 5008), (70003, 70008)]


@pytest.mark.parametrize("V,stride", RACE_SHAPES)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_lossless_race_without_floor(dtype, V, stride):
    # The draft puts far more mass than the target on the target's top token,
    # so max(0, p - q) is 0 there and the race starts with no floor; the
    # target's last 40% of ids are masked (no residual mass in the last
    # segments) and V leaves a ragged last vector.  The first draft token is
    # that top token, so most sequences reject at position 0.
    B, K = 24, 2
    batch = W.make(1, B=B, K=K, V=V, stride=stride)
    tgt = batch.target.float()
    dft = batch.draft.float()
    tgt[:, :, int(V * 0.6):V] = -float("inf")
    am = tgt[:, :, :V].argmax(-1)
    for b in range(B):
        for j in range(K):
            dft[b, j, am[b, j]] = tgt[b, j, am[b, j]] + 8.0
    batch.target = tgt.to(dtype)
    batch.draft = dft.to(dtype)
    batch.tokens[:, 0] = am[:, 0].to(torch.int32)
    for seed in range(4):
        r, o, _, _ = _lossless_check(batch, seed=seed)
        acc = np_(r.accepted_len)
        tok = np_(r.tokens)
        assert (acc == 0).mean() > 0.5
        for b in range(B):  # a residual token has p > q: never masked, never the top token
            y = tok[b, acc[b]]
            assert 0 <= y < int(V * 0.6)
            if acc[b] == 0:
                assert y != am[b, 0]


@pytest.mark.parametrize("mode", ["lossless", "fly"])
def test_large_vocabulary(mode):
    # V = 2^20 + 3 (ragged, 8x the workloads' largest): row statistics, the
    # race over every id and the FLy resolution, against the oracle
    V = (1 << 20) + 3
    if mode == "lossless":
        batch = W.make(1, B=3, K=2, V=V, stride=V + 5)
        for seed in (0, 1):
            _lossless_check(batch, seed=seed)
    else:
        batch = W.make(2, B=3, K=3, V=V, stride=V + 5)
        _fly_check(batch, theta=0.3, window=1)


def _all_accept_batch(B, K, V, stride, seed, peaks):
    # draft == target, so every verified draft is accepted and the step ends
    # with a draw from p at row L (the bonus row).  Rows: N(0,1) noise far
    # below a few peaks (log-odds within the race's reach of each other).
    g = torch.Generator().manual_seed(seed)
    t = torch.randn(B, K + 1, V, generator=g) - 60.0
    for b in range(B):
        for j in range(K + 1):
            for q, pid in enumerate(peaks(b, j)):
                t[b, j, pid] = 3.0 - 1.5 * q + 0.3 * torch.rand((), generator=g).item()
    tb = torch.full((B, K + 1, stride), float("nan"))
    tb[:, :, :V] = t
    tb = tb.to(torch.bfloat16)
    d = tb[:, :K].clone()
    tok = W.sample_rows(d[:, :, :V], 1.0, torch.Generator().manual_seed(seed + 1))
    return W.Batch(tb, d, tok, V, 1.0)


@pytest.mark.parametrize("V,stride", [(20011, 20016), (70003, 70008)])
@pytest.mark.parametrize("layout", ["spread", "same_thread_two_chunks",
                                    "same_thread_three_chunks", "one_chunk"])
def test_lossless_bonus_candidate_list(layout, V, stride):
    # The row pass lists, for row L, every id a draw from p there could pick;
    # the race then draws over that list.  The peaks sit where the list must
    # take them from: different threads, a thread's max chunk and second chunk
    # (read again), three chunks of one thread (the list is incomplete and the
    # row is raced in full), or one chunk.  bf16 rows: chunk `it` of thread t
    # holds vectors it*1024 + t and it*1024 + 512 + t (8 ids each).
    B, K = 12, 3
    if layout == "spread":
        peaks = lambda b, j: [(97 * b + 13 * j + 1000 * q) % V for q in range(5)]
    elif layout == "same_thread_two_chunks":
        peaks = lambda b, j: [8 * (1024 * 0 + 7) + 1, 8 * (1024 * 2 + 7) + 3, 8 * (512 + 7)]
    elif layout == "same_thread_three_chunks":
        peaks = lambda b, j: [8 * (1024 * 0 + 5), 8 * (1024 * 1 + 5) + 2, 8 * (1024 * 2 + 5) + 7]
    else:
        peaks = lambda b, j: [8 * 9, 8 * 9 + 5, 8 * (512 + 9) + 1]
    batch = _all_accept_batch(B, K, V, stride, 41, peaks)
    for seed in range(6):
        r, o, _, _ = _lossless_check(batch, seed=seed)
        assert (np_(r.accepted_len) == K).all()


def test_lossless_bonus_at_row_64_and_trimmed():
    # the bonus row is row 64 (K = 64, every draft accepted), and with kept
    # lengths the draw from p happens at row L < K
    B, K, V = 4, 64, 3001
    batch = _all_accept_batch(B, K, V, 3008, 7, lambda b, j: [(31 * j + b) % V, (31 * j + 500) % V])
    r, o, _, _ = _lossless_check(batch, seed=2)
    assert (np_(r.accepted_len) == K).all()
    kept = torch.tensor([0, 5, 63, 64], dtype=torch.int32)
    r, o, _, _ = _lossless_check(batch, seed=3, kept=kept)
    assert np_(r.accepted_len).tolist() == [0, 5, 63, 64]


@pytest.mark.parametrize("mode", ["lossless", "fly"])
def test_batch_beyond_grid_y_limit(mode):
    # B = 70000 sequences (more than a grid's 65535 y extent): every launch
    # must index sequences along x
    B, K, V = 70000, 1, 72
    if mode == "lossless":
        batch = W.make(1, B=B, K=K, V=V)
        _lossless_check(batch, seed=9)
    else:
        batch = W.make(2, B=B, K=K, V=V)
        _fly_check(batch, theta=0.3, window=0)


def test_verify_update_batch_beyond_grid_y_limit():
    # spec_verify_update at B = 70000: its last launch has 8751 token-picking
    # workgroups and the update's; results as spec_verify + spec_av_score_update
    B, K, V = 70000, 2, 72
    batch = W.make(1, B=B, K=K, V=V)
    t, d, tok = batch.target.to(DEV), batch.draft.to(DEV), batch.tokens.to(DEV)
    ob_a = torch.tensor(W.av_init(1, K=K), dtype=torch.float32, device=DEV)
    ob_b = ob_a.clone()
    ra, ca, _, _ = sv.verify_update(t, d, tok, ob_a, 0.05, seed=5, score=True)
    out = sv.VerifyResult(torch.empty(B, dtype=torch.int32, device=DEV),
                          torch.empty(B, K + 1, dtype=torch.int32, device=DEV))
    out.draft_stats_out = torch.empty(sv.draft_stats_bytes(B, K), dtype=torch.uint8, device=DEV)
    rb = sv.verify(t, d, tok, seed=5, out=out)
    cb, _, _ = sv.av_score_update(out.draft_stats_out, rb.accepted_len, ob_b, 0.05, B, K)
    torch.cuda.synchronize()
    assert torch.equal(ra.accepted_len, rb.accepted_len) and torch.equal(ra.tokens, rb.tokens)
    assert torch.equal(ca, cb) and torch.equal(ob_a, ob_b)


def test_lossless_deterministic_across_streams():
    batch = W.make(3, B=16, K=4, V=20000)
    t, d, tok = batch.target.to(DEV), batch.draft.to(DEV), batch.tokens.to(DEV)
    a = sv.verify(t, d, tok, seed=5, temperature=0.7)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        b = sv.verify(t, d, tok, seed=5, temperature=0.7)
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(a.tokens, b.tokens) and torch.equal(a.accepted_len, b.accepted_len)
    c = sv.verify(t, d, tok, seed=6, temperature=0.7)
    torch.cuda.synchronize()
    assert not torch.equal(a.tokens, c.tokens)


# ---------------------------------------------------------------------------
# Adaptive verification
# ---------------------------------------------------------------------------
def _av_step(batch, ob_host, tau, lr, seed, prefix=False, fused=False):
    """One GPU step (score, verify, update) and the oracle's step on the same
    inputs and the same starting parameters.  prefix: score with
    spec_av_score_prefix (confidences past each trim point are not read).
    fused: verify and update in one spec_verify_update call."""
    K = batch.tokens.shape[1]
    T = batch.temperature
    t, d, tok = batch.target.to(DEV), batch.draft.to(DEV), batch.tokens.to(DEV)
    ob = torch.tensor(ob_host, dtype=torch.float32, device=DEV)
    conf, mask, kept, ds = sv.av_score(d, tok, ob, tau, temperature=T, vocab=batch.V,
                                       prefix=prefix)
    if fused:
        r, _, _, _ = sv.verify_update(t, d, tok, ob, lr, seed=seed, temperature=T,
                                      vocab=batch.V, kept_len=kept, draft_stats=ds,
                                      boundary=True)
    else:
        r = sv.verify(t, d, tok, seed=seed, temperature=T, vocab=batch.V, kept_len=kept,
                      draft_stats=ds, boundary=True)
        sv.av_update(ds, r.accepted_len, kept, ob, lr, tok.shape[0], K)
    torch.cuda.synchronize()
    dh = host_logits(batch.draft)
    B = dh.shape[0]
    st = ref.rows_stats(dh.reshape(B * K, -1), temperature=f32(T), V=batch.V, nthreads=NT)
    feat = st["feat"].reshape(B, K)
    ob64 = np.asarray(ob_host, dtype=np.float32).astype(np.float64)
    oconf, omask, okept, onear = ref.av_score(feat, ob64, f32(tau))
    o = ref.verify(host_logits(batch.target), dh, np_(batch.tokens), seed, temperature=f32(T),
                   V=batch.V, kept_len=okept, nthreads=NT)
    o["boundary"] |= onear
    rel = REL_TOL[batch.target.dtype]
    if prefix:  # positions up to each first trimmed one were read; the rest are NaN
        read = np.arange(K)[None, :] <= np.minimum(np_(kept), K - 1)[:, None]
        assert np.isnan(np_(conf)[~read]).all()
        oconf = np.where(read, oconf, np.nan)
    assert_close(np_(conf), oconf, rel, "confidence")
    kept_ok = (np_(kept) == okept) | ((onear & ref.NEAR_TRIM) != 0)
    assert kept_ok.all(), "kept_len differs outside the trim boundary set"
    same = np_(kept) == okept
    compare_decisions(np_(r.accepted_len)[same], np_(r.tokens)[same],
                      {k: (v[same] if hasattr(v, "shape") and v.shape[:1] == (B,) else v)
                       for k, v in o.items()}, ALL_NEAR, "av verify",
                      dev_boundary=np_(r.boundary)[same], kept=okept[same])
    new = ref.av_update(feat, o["accepted_len"], okept, ob64, f32(lr))
    return np_(ob), new, o, okept


def test_av_score_update_parity_c1_full_size():
    # the lossless + adaptive-verification workload at its own size: B=64,
    # K=5, V=128256, omega = 1, beta_i = 0.5 - 0.3 i, no trimming, one SGD step
    batch = W.make(1, device=DEV)
    assert batch.tokens.shape == (64, 5)
    ob0 = W.av_init(1)
    got, want, _, okept = _av_step(batch, ob0, tau=0.0, lr=0.05, seed=0)
    assert np.all(okept == 5)
    assert np.allclose(got, want, rtol=0, atol=1e-5), (got, want)


@pytest.mark.parametrize("split", [False, True])
@pytest.mark.parametrize("tau", [0.0, 0.2])
def test_av_step_call_matches_separate_calls(tau, split):
    # AvStepCall with tau <= 0 verifies first (one row pass over target and
    # draft rows, exporting the draft statistics) and scores from them; with
    # tau > 0 it scores, trims and verifies.  Either way, and whether the
    # update shares the verification's last launch (spec_verify_update) or
    # not: bit-identical to the separate calls, over three steps with carried
    # parameters.
    batch = W.make(1, B=20, K=5, V=7001, stride=7008)
    t, d, tok = batch.target.to(DEV), batch.draft.to(DEV), batch.tokens.to(DEV)
    B, K = tok.shape
    ob_a = torch.tensor(W.av_init(1), dtype=torch.float32, device=DEV)
    ob_b = ob_a.clone()
    call = sv.AvStepCall(t, d, tok, ob_a, tau, 0.05, vocab=batch.V, split=split)
    assert call.fused == (tau <= 0.0)
    for step in range(3):
        r_a = call(step)
        conf, mask, kept, ds = sv.av_score(d, tok, ob_b, tau, vocab=batch.V)
        r_b = sv.verify(t, d, tok, seed=step, vocab=batch.V, kept_len=kept, draft_stats=ds)
        sv.av_update(ds, r_b.accepted_len, kept, ob_b, 0.05, B, K)
        torch.cuda.synchronize()
        assert torch.equal(r_a.accepted_len, r_b.accepted_len)
        assert torch.equal(r_a.tokens, r_b.tokens)
        assert torch.equal(call.conf, conf) and torch.equal(call.kept, kept)
        assert torch.equal(call.mask, mask)
        assert torch.equal(call.stats[:24 * B * K], ds[:24 * B * K])
        assert torch.equal(ob_a, ob_b)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B,K,trim", [(300, 7, False), (300, 7, True), (13, 64, False),
                                      (1, 3, True)])
def test_verify_update_matches_separate_calls(B, K, trim, dtype):
    # spec_verify_update against spec_verify followed by spec_av_update (or,
    # untrimmed, spec_av_score_update): the tokens, accepted lengths, boundary
    # bits, scores and coefficients bit for bit.  B not a multiple of the
    # token workgroup's eight sequences; K = 64 fills a wave with positions.
    batch = W.make(1, B=B, K=K, V=3001, stride=3008)
    t, d, tok = batch.target.to(DEV), batch.draft.to(DEV), batch.tokens.to(DEV)
    if dtype == "f32":
        t, d = t.float(), d.float()
    ob0 = torch.tensor(W.av_init(1, K=K), dtype=torch.float32, device=DEV)
    for step in range(2):
        ob_a, ob_b = ob0.clone(), ob0.clone()
        if trim:
            _, _, kept, ds = sv.av_score(d, tok, ob0, 0.2, vocab=batch.V)
            ra, ca, ma, ka = sv.verify_update(t, d, tok, ob_a, 0.05, seed=step, vocab=batch.V,
                                              kept_len=kept, draft_stats=ds, boundary=True)
            rb = sv.verify(t, d, tok, seed=step, vocab=batch.V, kept_len=kept, draft_stats=ds,
                           boundary=True)
            sv.av_update(ds, rb.accepted_len, kept, ob_b, 0.05, B, K)
        else:
            ra, ca, ma, ka = sv.verify_update(t, d, tok, ob_a, 0.05, seed=step, vocab=batch.V,
                                              score=True, boundary=True)
            out = sv.VerifyResult(torch.empty(B, dtype=torch.int32, device=DEV),
                                  torch.empty(B, K + 1, dtype=torch.int32, device=DEV))
            out.boundary = torch.empty(B, dtype=torch.int32, device=DEV)
            out.draft_stats_out = torch.empty(sv.draft_stats_bytes(B, K), dtype=torch.uint8,
                                              device=DEV)
            rb = sv.verify(t, d, tok, seed=step, vocab=batch.V, out=out)
            cb, mb, kb = sv.av_score_update(out.draft_stats_out, rb.accepted_len, ob_b, 0.05,
                                            B, K)
        torch.cuda.synchronize()
        assert torch.equal(ra.accepted_len, rb.accepted_len)
        assert torch.equal(ra.tokens, rb.tokens)
        assert torch.equal(ra.boundary, rb.boundary)
        assert torch.equal(ob_a, ob_b)
        if B > 1:  # labels exist, so the step moved the coefficients
            assert not torch.equal(ob_a, ob0)
        if not trim:
            assert torch.equal(ca, cb) and torch.equal(ma, mb) and torch.equal(ka, kb)
        ob0 = ob_a


def test_verify_update_residual_empty():
    # the residual-empty construction below through spec_verify_update: the
    # fallback race runs in the token workgroup's whole 512 threads; tokens,
    # bits and coefficients as spec_verify and spec_av_score_update give
    rng = np.random.default_rng(2)
    B, K, V = 24, 2, 4000
    t = rng.standard_normal((B, K + 1, V)).astype(np.float32)
    t[:, :, ::4] = -np.inf
    d = t[:, :K].copy()
    x = np.full((B, K), V + 3, dtype=np.int32)
    x[::3, 0] = -1
    tt, dd, xx = (torch.from_numpy(a).to(DEV) for a in (t, d, x))
    ob_a = torch.tensor(W.av_init(1, K=K), dtype=torch.float32, device=DEV)
    ob_b = ob_a.clone()
    ra, ca, _, _ = sv.verify_update(tt, dd, xx, ob_a, 0.05, seed=4, score=True, boundary=True)
    out = sv.VerifyResult(torch.empty(B, dtype=torch.int32, device=DEV),
                          torch.empty(B, K + 1, dtype=torch.int32, device=DEV))
    out.boundary = torch.empty(B, dtype=torch.int32, device=DEV)
    out.draft_stats_out = torch.empty(sv.draft_stats_bytes(B, K), dtype=torch.uint8, device=DEV)
    rb = sv.verify(tt, dd, xx, seed=4, out=out)
    cb, _, _ = sv.av_score_update(out.draft_stats_out, rb.accepted_len, ob_b, 0.05, B, K)
    torch.cuda.synchronize()
    assert np.all(np_(ra.boundary) & sv.RESIDUAL_EMPTY)
    assert torch.equal(ra.tokens, rb.tokens) and torch.equal(ra.boundary, rb.boundary)
    assert torch.equal(ra.accepted_len, rb.accepted_len)
    assert torch.equal(ca, cb) and torch.equal(ob_a, ob_b)


@pytest.mark.parametrize("B,K", [(20, 5), (300, 7), (64, 64)])
def test_av_score_update_matches_score_then_update(B, K):
    # one launch for an untrimmed step's scores and SGD step, against
    # spec_av_score_stats (tau = 0) followed by spec_av_update (kept NULL):
    # bit-identical scores, masks, kept lengths and coefficients.  B*K above
    # the workgroup's 512 threads makes threads score several drafts.
    g = torch.Generator().manual_seed(B * 100 + K)
    ds = torch.zeros(sv.draft_stats_bytes(B, K), dtype=torch.uint8)
    sv.draft_stats_view(ds, B, K)["feat"].copy_(torch.randn(B * K, generator=g) * 1.3 - 1.2)
    ds = ds.to(DEV)
    acc = torch.randint(0, K + 1, (B,), generator=g, dtype=torch.int32).to(DEV)
    ob_a = torch.tensor(W.av_init(1, K=K), dtype=torch.float32, device=DEV)
    ob_b = ob_a.clone()
    for step in range(3):
        c_a, m_a, k_a = sv.av_score_update(ds, acc, ob_a, 0.05, B, K)
        c_b, m_b, k_b = sv.av_score_stats(ds, B, K, ob_b, 0.0)
        sv.av_update(ds, acc, None, ob_b, 0.05, B, K)
        torch.cuda.synchronize()
        assert torch.equal(c_a, c_b) and torch.equal(m_a, m_b) and torch.equal(k_a, k_b)
        assert torch.equal(ob_a, ob_b)
        assert (k_a == K).all() and (m_a == 1).all()


@pytest.mark.parametrize("dtype,tau,K", [("bf16", 0.2, 8), ("f32", 0.35, 5), ("bf16", 0.0, 3),
                                         ("bf16", 0.02, 64), ("f32", 0.9, 4)])
def test_av_score_prefix_matches_full_scoring(dtype, tau, K):
    # spec_av_score_prefix stops reading a sequence's draft rows after its
    # first trimmed position: kept lengths and masks equal spec_av_score's,
    # and so do the confidences and draft statistics of every position up to
    # that first trimmed one, bit for bit; the positions after it are NaN
    B = 48 if K < 64 else 6
    batch = W.gaussian(B, K, 7001, dtype, 1.0, seed=K, token_seed=1, stride=7008)
    d, tok = batch.draft.to(DEV), batch.tokens.to(DEV)
    ob = torch.tensor(W.av_init(4, K=K), dtype=torch.float32, device=DEV)
    c0, m0, k0, s0 = sv.av_score(d, tok, ob, tau, vocab=batch.V)
    c1, m1, k1, s1 = sv.av_score(d, tok, ob, tau, vocab=batch.V, prefix=True)
    torch.cuda.synchronize()
    assert torch.equal(k0, k1) and torch.equal(m0, m1)
    kept = np_(k0)
    if tau > 0:
        assert (kept < K).any()  # some sequences trim
    read = np.arange(K)[None, :] <= np.minimum(kept, K - 1)[:, None]  # rows the prefix read
    v0 = sv.draft_stats_view(s0, B, K)
    v1 = sv.draft_stats_view(s1, B, K)
    pairs = [(c0, c1)] + [(v0[n], v1[n]) for n in ("lse2", "logq2", "qmax", "feat")]
    for a, b in pairs:
        a, b = np_(a).reshape(B, K), np_(b).reshape(B, K)
        assert np.array_equal(a[read].view(np.uint8), b[read].view(np.uint8))
        assert np.isnan(b[~read]).all()


def test_av_step_call_prefix_matches_separate_calls():
    # the step with prefix scoring: same kept lengths, tokens and coefficients
    # as the step with full scoring, over three steps
    batch = W.make(4, B=96, V=6001, stride=6008)
    t, d, tok = batch.target.to(DEV), batch.draft.to(DEV), batch.tokens.to(DEV)
    ob_a = torch.tensor(W.av_init(4), dtype=torch.float32, device=DEV)
    ob_b = ob_a.clone()
    ca = sv.AvStepCall(t, d, tok, ob_a, 0.2, 0.05, vocab=batch.V, prefix=True)
    cb = sv.AvStepCall(t, d, tok, ob_b, 0.2, 0.05, vocab=batch.V)
    for step in range(3):
        ra = ca(step)
        rb = cb(step)
        torch.cuda.synchronize()
        assert torch.equal(ra.accepted_len, rb.accepted_len) and torch.equal(ra.tokens, rb.tokens)
        assert torch.equal(ca.kept, cb.kept) and torch.equal(ob_a, ob_b)


def test_verify_exports_draft_stats():
    # the draft statistics a lossless call computes itself, exported, equal
    # those of spec_av_score bit for bit; scoring from them equals spec_av_score
    batch = W.make(3, B=10, K=4, V=5003, stride=5008)
    t, d, tok = batch.target.to(DEV), batch.draft.to(DEV), batch.tokens.to(DEV)
    B, K = tok.shape
    ob = torch.tensor(W.av_init(1, K=K), dtype=torch.float32, device=DEV)
    out = sv.VerifyResult(torch.empty(B, dtype=torch.int32, device=DEV),
                          torch.empty(B, K + 1, dtype=torch.int32, device=DEV))
    out.draft_stats_out = torch.zeros(sv.draft_stats_bytes(B, K), dtype=torch.uint8, device=DEV)
    sv.verify(t, d, tok, seed=1, temperature=0.7, vocab=batch.V, out=out)
    conf, mask, kept, ds = sv.av_score(d, tok, ob, 0.3, temperature=0.7, vocab=batch.V)
    c2, m2, k2 = sv.av_score_stats(out.draft_stats_out, B, K, ob, 0.3)
    torch.cuda.synchronize()
    assert torch.equal(out.draft_stats_out[:24 * B * K], ds[:24 * B * K])
    assert torch.equal(c2, conf) and torch.equal(m2, mask) and torch.equal(k2, kept)


def test_av_pipeline_twenty_steps_full_size():
    # The adaptive-verification pipeline as configured: B=1024, K=8,
    # V=128256 bf16, tau=0.2, lr=0.05, 20 steps, each with fresh seeded logits
    # and the parameters the previous step left (carried on the GPU side, as
    # the pipeline does; the oracle starts each step from the same values).
    # After every step omega and beta match the oracle's step to 1e-5.  The
    # steps score as the benchmark does, reading draft rows up to each trim
    # point only (even steps) and every draft row (odd steps); the verify and
    # update are one spec_verify_update call in steps 0, 1 mod 4, separate
    # calls otherwise.
    ob = W.av_init(4)
    hist = np.zeros(9, dtype=np.int64)
    for step in range(20):
        batch = W.make(4, device=DEV, step=step)
        assert batch.tokens.shape == (1024, 8)
        got, want, o, okept = _av_step(batch, ob, tau=0.2, lr=0.05, seed=step,
                                       prefix=step % 2 == 0, fused=step % 4 < 2)
        assert np.allclose(got, want, rtol=0, atol=1e-5), (step, got, want)
        hist += np.bincount(okept, minlength=9)
        ob = got.tolist()
        del batch
        torch.cuda.empty_cache()
    print("kept-length histogram over 20 steps:", hist.tolist(), "omega/beta:",
          [round(v, 5) for v in ob])
    assert hist.sum() == 20 * 1024


def test_av_pipeline_c4_recipe_steps():
    ob = W.av_init(4)
    for step in range(3):
        batch = W.make(4, B=24, step=step)
        got, want, o, okept = _av_step(batch, ob, tau=0.2, lr=0.05, seed=step)
        assert np.allclose(got, want, rtol=0, atol=1e-5), (step, got, want)
        ob = got.tolist()  # carry the GPU's parameters forward, as the pipeline does


# ---------------------------------------------------------------------------
# The library's boundary-case log on inputs built to sit on a boundary
# ---------------------------------------------------------------------------
def _check_constructed(t, d, x, seed, T=1.0, kept=None):
    """Lossless call on host float32 logits; returns the library's result and
    the oracle's, compared (flags included)."""
    r = sv.verify(torch.from_numpy(t).to(DEV), torch.from_numpy(d).to(DEV),
                  torch.from_numpy(x).to(DEV), seed=seed, temperature=T, boundary=True,
                  kept_len=None if kept is None else torch.from_numpy(kept).to(DEV))
    torch.cuda.synchronize()
    o = ref.verify(t, d, x, seed, temperature=f32(T), kept_len=kept, nthreads=NT)
    compare_decisions(np_(r.accepted_len), np_(r.tokens), o, ALL_NEAR, "constructed",
                      dev_boundary=np_(r.boundary), kept=kept, tally="constructed")
    return r, o


def test_boundary_residual_empty_on_device():
    # identical target and draft rows and out-of-range draft tokens: rejected
    # at once with p - q = 0 at every id, so the token comes from p itself
    rng = np.random.default_rng(2)
    B, K, V = 24, 2, 4000
    t = rng.standard_normal((B, K + 1, V)).astype(np.float32)
    t[:, :, ::4] = -np.inf
    d = t[:, :K].copy()
    x = np.full((B, K), V + 3, dtype=np.int32)
    x[::3, 0] = -1
    r, o = _check_constructed(t, d, x, seed=4)
    bnd = np_(r.boundary)
    assert np.all(bnd & sv.RESIDUAL_EMPTY) and np.all(o["boundary"] & ref.RESIDUAL_EMPTY)
    y = np_(r.tokens)[:, 0]
    assert np.all(y % 4 != 0) and np.array_equal(y, o["tokens"][:, 0])


def _race_pair_rows(ia, ib, la, lb, V, residual):
    """One sequence, K = 1.  residual=False: position 0 always accepted
    (target = draft row), the draw is from p at row 1, whose only finite
    logits are la at ia and lb at ib.  residual=True: the draft token has
    p = 0 (rejected surely) and the draft row has no mass at ia, ib, so the
    residual race at row 0 runs over those two ids with w = p."""
    t = np.full((1, 2, V), -np.inf, dtype=np.float32)
    d = np.full((1, 1, V), -np.inf, dtype=np.float32)
    if residual:
        t[0, 0, ia], t[0, 0, ib] = la, lb
        d[0, 0, 7:V:5] = 0.0
        x = np.array([[7]], dtype=np.int32)
        t[0, 1, 0] = 0.0
    else:
        t[0, 0] = np.linspace(-1, 1, V, dtype=np.float32)
        d[0, 0] = t[0, 0]
        t[0, 1, ia], t[0, 1, ib] = la, lb
        x = np.array([[5]], dtype=np.int32)
    return t, d, x


@pytest.mark.parametrize("path", ["listed", "raced", "residual"])
@pytest.mark.parametrize("delta", [1e-7, 1e-3])
def test_boundary_near_race_on_device(path, delta):
    # Keys p_a/E_a and p_b/E_b designed delta apart (relative) from the
    # pinned uniforms: a near-tie at 1e-7, clear at 1e-3.  Three race paths:
    # a draw from p over the row pass's candidate list, the same draw on a row
    # too flat to list (the race reads it; 2900 ids sit 22 log2 units
    # below), and a residual race.  V = 4000 float32 ids, the two in
    # different race segments.
    V, seed, ia, ib = 4000, 3, 1234, 3210
    residual = path == "residual"
    pos = 0 if residual else 1
    Ea = -np.log(ref.race_uniform(seed, ia, pos, 0))
    Eb = -np.log(ref.race_uniform(seed, ib, pos, 0))
    la = np.float32(np.log(Ea / Eb) + np.log1p(delta))
    t, d, x = _race_pair_rows(ia, ib, la, 0.0, V, residual)
    if path == "raced":
        t[0, 1, 100:1200] = np.float32(-22 * np.log(2.0))
        t[0, 1, 1300:3100] = np.float32(-22 * np.log(2.0))
    r, o = _check_constructed(t, d, x, seed)
    assert np_(r.accepted_len)[0] == (0 if residual else 1)
    want_near = delta < 1e-6
    assert bool(o["boundary"][0] & ref.NEAR_RACE) == want_near
    assert bool(np_(r.boundary)[0] & sv.NEAR_RACE) == want_near
    if not want_near:
        assert np_(r.tokens)[0, pos] == ia


@pytest.mark.parametrize("off", [3e-6, -3e-6, 2e-4])
def test_boundary_near_accept_on_device(off):
    # p(x_0)/q(x_0) placed `off` from the accept test's uniform
    seed, V = 6, 4096
    u0 = ref.uniform(seed, 0, 0, 0, ref.TAG_ACCEPT)
    q = np.full(V, 1.0 / V)
    p = np.full(V, 0.0)
    p[0] = q[0] * (u0 + off)
    p[1:] = (1 - p[0]) / (V - 1)
    tl = np.log(p).astype(np.float32)
    t = np.stack([tl, tl])[None]
    d = np.log(q).astype(np.float32)[None, None]
    r, o = _check_constructed(t, d, np.zeros((1, 1), dtype=np.int32), seed)
    want = abs(off) < 1e-5
    assert bool(np_(r.boundary)[0] & sv.NEAR_ACCEPT) == want
    assert np_(r.accepted_len)[0] == (1 if off > 0 else 0)


@pytest.mark.parametrize("off", [5e-6, 1e-3])
def test_boundary_near_gate_on_device(off):
    # theta placed `off` below a flat target row's entropy, a deviation there
    rng = np.random.default_rng(5)
    K, V = 4, 30000
    t = (rng.standard_normal((1, K + 1, V)) * 0.5).astype(np.float32)
    st = ref.rows_stats(t[0])
    x = st["argmax"][:K].astype(np.int32).copy()[None]
    x[0, 1] = (st["argmax"][1] + 1) % V
    theta = float(np.float32(st["h"][1] - off))
    r = sv.verify(torch.from_numpy(t).to(DEV), None, torch.from_numpy(x).to(DEV), seed=0,
                  mode=sv.MODE_FLY, fly_theta=theta, fly_window=1, boundary=True)
    torch.cuda.synchronize()
    o = ref.verify(t, None, x, 0, ref.MODE_FLY, theta=theta, window=1, nthreads=NT)
    compare_decisions(np_(r.accepted_len), np_(r.tokens), o, ref.NEAR_GATE, "gate",
                      dev_boundary=np_(r.boundary), tally="constructed")
    assert bool(np_(r.boundary)[0] & sv.NEAR_GATE) == (off < 1e-5)
    assert np_(r.accepted_len)[0] == K


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("path", ["bonus", "residual"])
def test_race_winner_with_saturated_screening_half(dtype, path):
    # Flat weights: the race's winner is the id with the largest word.  For
    # the seed taken that id's high 16 bits (its screening half) are all ones, so its
    # leading ones are known only as "16 or more" until the race stream is
    # drawn: the device must not screen it out.  The draw from p runs at the
    # bonus row (row 0 identical in target and draft: accepted), the residual
    # at row 0 (the draft puts nearly all its mass on the drafted token).
    V = 131072
    pos = 1 if path == "bonus" else 0

    def winner(seed):
        words = np.array([ref.race_u32(seed, x, pos, 0) for x in range(V)], dtype=np.uint64)
        if path == "residual":
            words[7] = 0  # the drafted token has no residual weight
        k = words >> 9  # the lattice index of each id's uniform
        w = int(np.argmax(k))
        unique = np.count_nonzero(k == k[w]) == 1
        return w if unique and int(words[w]) >> 16 == 0xFFFF else None

    # the first seed whose winner has a saturated screening half and no tie
    seed = next(s for s in range(1, 50) if winner(s) is not None)
    win = winner(seed)
    t = np.zeros((1, 2, V), dtype=np.float32)
    d = np.zeros((1, 1, V), dtype=np.float32)
    if path == "residual":
        d[0, 0, 7] = 30.0
    x = np.array([[7]], dtype=np.int32)
    tt = torch.from_numpy(t).to(dtype).to(DEV)
    dd = torch.from_numpy(d).to(dtype).to(DEV)
    r = sv.verify(tt, dd, torch.from_numpy(x).to(DEV), seed=seed, boundary=True)
    torch.cuda.synchronize()
    o = ref.verify(host_logits(tt), host_logits(dd), x, seed, nthreads=NT)
    compare_decisions(np_(r.accepted_len), np_(r.tokens), o, ALL_NEAR, "constructed",
                      dev_boundary=np_(r.boundary), tally="constructed")
    assert np_(r.accepted_len)[0] == pos
    assert o["tokens"][0, pos] == win and np_(r.tokens)[0, pos] == win


def test_low_temperature_race_screening():
    # T = 1e-4 with logits near 10: l*c ~ 1.4e5, where a float carries 1.6e-2
    # of rounding; two ids whose race keys lie 1e-3 apart (within that
    # rounding) must still be ordered as the exact keys order them, on the
    # listed path and on the full race path (a row too flat to list).
    seed, V, T = 8, 6000, 1e-4
    c = 1.0 / np.float32(T)
    for pos_pair in ((11, 4000), (4000, 11)):
        ia, ib = pos_pair
        Ea = -np.log(ref.race_uniform(seed, ia, 1, 0))
        Eb = -np.log(ref.race_uniform(seed, ib, 1, 0))
        # (la - lb)/T = ln(Ea/Eb) + 1e-3
        lb = np.float32(10.0)
        la = np.float32(lb + (np.log(Ea / Eb) + 1e-3) / c)
        t, d, x = _race_pair_rows(ia, ib, la, lb, V, residual=False)
        r, o = _check_constructed(t, d, x, seed, T=T)
        assert (o["boundary"][0] & ref.NEAR_RACE) or np_(r.tokens)[0, 1] == o["tokens"][0, 1]
        # many ids within the race's reach (p about 2^-20 of the two): the
        # row pass cannot list them, so the race reads the row
        t[0, 1, 100:3000] = lb - np.float32(20 * 0.69314718 / c)
        r, o = _check_constructed(t, d, x, seed, T=T)
        assert (o["boundary"][0] & ref.NEAR_RACE) or np_(r.tokens)[0, 1] == o["tokens"][0, 1]


# ---------------------------------------------------------------------------
# Edge cases at the boundary
# ---------------------------------------------------------------------------
def test_empty_batch_is_a_noop():
    t = torch.zeros(0, 5, 64, device=DEV)
    tok = torch.zeros(0, 4, dtype=torch.int32, device=DEV)
    r = sv.verify(t, torch.zeros(0, 4, 64, device=DEV), tok, seed=0)
    assert r.accepted_len.numel() == 0


def test_invalid_arguments_raise():
    t = torch.zeros(2, 3, 64, device=DEV)
    d = torch.zeros(2, 2, 64, device=DEV)
    tok = torch.zeros(2, 2, dtype=torch.int32, device=DEV)
    with pytest.raises(sv.SpecVerifyError):
        sv.verify(t, None, tok, seed=0)                       # lossless needs the draft
    with pytest.raises(sv.SpecVerifyError):
        sv.verify(t, d, tok, seed=0, temperature=0.0)
    with pytest.raises(sv.SpecVerifyError):
        sv.verify(t, d, tok, seed=0, vocab=65)                # V > stride
    with pytest.raises(sv.SpecVerifyError):
        sv.verify(t[:, :, :62].contiguous(), d[:, :, :62].contiguous(), tok, seed=0)  # 248 B rows


def test_binding_rejects_buffers_the_kernels_would_overrun():
    # the library takes raw device pointers: a host tensor, a short buffer or
    # another element type must fail in the binding, before any launch
    B, K, V = 2, 2, 64
    t = torch.zeros(B, K + 1, V, device=DEV)
    d = torch.zeros(B, K, V, device=DEV)
    tok = torch.zeros(B, K, dtype=torch.int32, device=DEV)
    ob = torch.zeros(K + 1, dtype=torch.float32, device=DEV)
    need = sv.workspace_bytes(B, K, V, dtype=sv.DTYPE_F32)
    bad = [
        dict(workspace=torch.empty(need, dtype=torch.uint8)),                  # host memory
        dict(kept_len=torch.zeros(B, dtype=torch.int64, device=DEV)),          # int64
        dict(kept_len=torch.zeros(B - 1, dtype=torch.int32, device=DEV)),      # short
        dict(draft_stats=torch.zeros(sv.draft_stats_bytes(B, K) - 1, dtype=torch.uint8,
                                     device=DEV)),                             # short
        dict(out=sv.VerifyResult(torch.empty(B, dtype=torch.int32, device=DEV),
                                 torch.empty(B, K, dtype=torch.int32, device=DEV))),  # [B, K]
    ]
    for kw in bad:
        with pytest.raises(ValueError):
            sv.verify(t, d, tok, seed=0, **kw)
    with pytest.raises(ValueError):
        sv.verify(t, d, tok.long(), seed=0)
    with pytest.raises(ValueError):
        sv.verify_update(t, d, tok, ob[:K], 0.1)                               # [K] coefficients
    with pytest.raises(ValueError):
        sv.VerifyCall(t, d, tok, draft_stats=torch.zeros(8, dtype=torch.uint8, device=DEV))
    ds = torch.zeros(sv.draft_stats_bytes(B, K), dtype=torch.uint8, device=DEV)
    acc = torch.zeros(B, dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError):
        sv.av_update(ds, acc.long(), None, ob, 0.1, B, K)
    with pytest.raises(ValueError):
        sv.av_update(ds[:-1], acc, None, ob, 0.1, B, K)
    with pytest.raises(ValueError):
        sv.av_score_update(ds, acc, ob.double(), 0.1, B, K)
    st = sv.irls_state(K, DEV)
    with pytest.raises(ValueError):
        sv.irls_accumulate(st[:-1], ds, acc, None, ob, B, K)
    with pytest.raises(ValueError):
        sv.av_diagnostics(ds, acc, None, ob, B, K, out=torch.empty(4, device=DEV))  # float32
    conf = torch.full((B, K), 0.5, device=DEV)
    cost = torch.from_numpy(W.budget_costs(B, K)).to(DEV)
    with pytest.raises(ValueError):
        sv.av_budget(conf, cost.float())
    with pytest.raises(ValueError):
        sv.av_budget(conf, cost[:-1])
    with pytest.raises(ValueError):
        sv.ngram_propose(tok, torch.zeros(B, dtype=torch.int64, device=DEV), 1, 2, 3)
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# Randomised configurations: every option at once, drawn from fixed seeds
# ---------------------------------------------------------------------------
def _random_batch(rng):
    mode = str(rng.choice(["lossless", "fly"]))
    K = int(rng.integers(1, 11)) if rng.random() > 0.1 else 64
    B = int(rng.integers(1, 49)) if K < 64 else int(rng.integers(1, 5))
    V = int(np.exp(rng.uniform(np.log(2), np.log(200000))))
    if B * (2 * K + 1) * V > 3e7:  # keep the oracle's share to a fraction of a second
        V = max(2, int(3e7 / (B * (2 * K + 1))))
    stride = (V + 7) // 8 * 8 + 8 * int(rng.integers(0, 3))
    f32 = bool(rng.random() < 0.5)
    seed = int(rng.integers(0, 1 << 30))
    if mode == "lossless":
        T = float(rng.choice([1.0, 0.7, float(np.exp(rng.uniform(np.log(0.2), np.log(5.0))))]))
        if rng.random() < 0.5:
            batch = W.gaussian(B, K, V, "f32" if f32 else "bf16", T, seed=seed, token_seed=1,
                               stride=stride)
        else:
            batch = W.zipf(B, K, V, T, seed=seed, token_seed=1, stride=stride)
            if f32:
                batch.target, batch.draft = batch.target.float(), batch.draft.float()
    else:
        V = max(V, 5)  # the recipe draws deviations from the top 5
        stride = max(stride, (V + 7) // 8 * 8)
        batch = W.fly(B, K, V, seed=seed, stride=stride)
        if f32:
            batch.target = batch.target.float()
    kept = None
    if rng.random() < 0.4:
        kept = torch.from_numpy(rng.integers(-1, K + 3, B).astype(np.int32))
    return mode, batch, kept, rng


# The randomised tests run 24, 16 and 12 cases by default.
# SPECVERIFY_RANDOM_CASES=N runs the first N configuration cases and
# SPECVERIFY_RANDOM_STEP_CASES=N the first N of each step test; their seeds are
# a per-test base + SPECVERIFY_RANDOM_OFFSET (default 0) + the case number.
RANDOM_CASES = int(os.environ.get("SPECVERIFY_RANDOM_CASES", "24"))
RANDOM_STEP_CASES = os.environ.get("SPECVERIFY_RANDOM_STEP_CASES")
RANDOM_OFFSET = int(os.environ.get("SPECVERIFY_RANDOM_OFFSET", "0"))


@pytest.mark.parametrize("case", range(RANDOM_CASES))
def test_random_configurations(case):
    # mode, recipe, dtype, B, K (up to 64), V (2 to 200000), padded stride,
    # temperature, kept lengths (some outside [0, K]), FLy threshold and window
    mode, batch, kept, rng = _random_batch(np.random.default_rng(9000 + RANDOM_OFFSET + case))
    K = batch.tokens.shape[1]
    kept_ref = None if kept is None else kept.clamp(0, K)  # the library clamps into [0, K]
    if mode == "lossless":
        for seed in range(2):
            _lossless_check(batch, seed=seed, kept=kept, kept_ref=kept_ref)
    else:
        theta = float(rng.uniform(0.0, 1.2))
        window = int(rng.integers(0, K + 2))
        _fly_check(batch, theta=theta, window=window, kept=kept, kept_ref=kept_ref)


@pytest.mark.parametrize("case", range(int(RANDOM_STEP_CASES or 16)))
def test_random_verify_update(case):
    # spec_verify_update on random shapes against the separate calls, bit for
    # bit: untrimmed steps (scores and SGD step from the verify pass's own
    # statistics) and trimmed ones (statistics and kept lengths from
    # spec_av_score), both dtypes, padded strides, random temperatures
    rng = np.random.default_rng(9100 + RANDOM_OFFSET + case)
    K = int(rng.integers(1, 13)) if case % 5 else 64
    B = int(rng.integers(1, 300)) if K < 64 else int(rng.integers(1, 20))
    V = int(np.exp(rng.uniform(np.log(8), np.log(40000))))
    dtype = "bf16" if case % 2 else "f32"
    unit = 8 if dtype == "bf16" else 4
    stride = V + int(rng.integers(0, 3)) * unit
    stride = (stride + unit - 1) // unit * unit
    T = float(np.exp(rng.uniform(np.log(0.5), np.log(2.0))))
    batch = W.gaussian(B, K, V, dtype, T, seed=int(rng.integers(0, 1 << 30)), token_seed=3,
                       stride=stride)
    t, d, tok = batch.target.to(DEV), batch.draft.to(DEV), batch.tokens.to(DEV)
    ob0 = torch.tensor([float(rng.uniform(0.3, 1.5))] + [float(v) for v in
                                                        rng.uniform(-1.0, 1.0, K)],
                       dtype=torch.float32, device=DEV)
    lr = float(rng.uniform(0.01, 0.2))
    ob_a, ob_b = ob0.clone(), ob0.clone()
    if case % 3 == 0:  # untrimmed: scores from the verify pass's statistics
        ra, ca, ma, ka = sv.verify_update(t, d, tok, ob_a, lr, seed=case, temperature=T,
                                          vocab=V, score=True, boundary=True)
        out = sv.VerifyResult(torch.empty(B, dtype=torch.int32, device=DEV),
                              torch.empty(B, K + 1, dtype=torch.int32, device=DEV))
        out.boundary = torch.empty(B, dtype=torch.int32, device=DEV)
        out.draft_stats_out = torch.empty(sv.draft_stats_bytes(B, K), dtype=torch.uint8,
                                          device=DEV)
        rb = sv.verify(t, d, tok, seed=case, temperature=T, vocab=V, out=out)
        cb, mb, kb = sv.av_score_update(out.draft_stats_out, rb.accepted_len, ob_b, lr, B, K)
        torch.cuda.synchronize()
        assert torch.equal(ca, cb) and torch.equal(ma, mb) and torch.equal(ka, kb)
    else:
        tau = float(rng.uniform(0.02, 0.6))
        _, _, kept, ds = sv.av_score(d, tok, ob0, tau, temperature=T, vocab=V,
                                     prefix=case % 2 == 0)
        ra, _, _, _ = sv.verify_update(t, d, tok, ob_a, lr, seed=case, temperature=T, vocab=V,
                                       kept_len=kept, draft_stats=ds, boundary=True)
        rb = sv.verify(t, d, tok, seed=case, temperature=T, vocab=V, kept_len=kept,
                       draft_stats=ds, boundary=True)
        sv.av_update(ds, rb.accepted_len, kept, ob_b, lr, B, K)
        torch.cuda.synchronize()
    assert torch.equal(ra.accepted_len, rb.accepted_len)
    assert torch.equal(ra.tokens, rb.tokens) and torch.equal(ra.boundary, rb.boundary)
    assert torch.equal(ob_a, ob_b)


@pytest.mark.parametrize("case", range(int(RANDOM_STEP_CASES or 12)))
def test_random_av_steps(case):
    # adaptive-verification steps (score, trim at a random tau, verify the kept
    # drafts, SGD update) on random shapes, dtypes and temperatures
    rng = np.random.default_rng(7000 + RANDOM_OFFSET + case)
    K = int(rng.integers(1, 13)) if case % 4 else 64
    B = int(rng.integers(1, 65)) if K < 64 else int(rng.integers(1, 6))
    V = int(np.exp(rng.uniform(np.log(8), np.log(60000))))
    V = max(8, min(V, int(2e7 / (B * (2 * K + 1)))))
    stride = (V + 7) // 8 * 8 + 8 * int(rng.integers(0, 2))
    dtype = "f32" if rng.random() < 0.5 else "bf16"
    T = float(rng.choice([1.0, float(np.exp(rng.uniform(np.log(0.5), np.log(2.0))))]))
    batch = W.gaussian(B, K, V, dtype, T, seed=int(rng.integers(0, 1 << 30)), token_seed=2,
                       stride=stride)
    tau = 0.0 if rng.random() < 0.3 else float(rng.uniform(0.02, 0.6))
    lr = float(rng.uniform(0.01, 0.2))
    ob0 = [float(rng.uniform(0.3, 1.5))] + [float(v) for v in rng.uniform(-1.0, 1.0, K)]
    got, want, _, okept = _av_step(batch, ob0, tau=tau, lr=lr, seed=case, fused=case % 2 == 1)
    assert np.allclose(got, want, rtol=0, atol=1e-5), (got, want)
