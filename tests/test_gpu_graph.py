"""The verification calls allocate nothing and clear no memory with memsets,
so a caller can record them in a HIP graph.  Each test records a call,
replays the graph several times with eager work between the replays, and
checks every replay against an eager call on the same inputs."""
import numpy as np
import pytest
import torch

import draft_token_verification_vocab_amd as sv
from draft_token_verification_vocab_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "the GPU tests need an MI355X"
    sv.load()


def _result(B, K):
    r = sv.VerifyResult(torch.full((B,), -7, dtype=torch.int32, device=DEV),
                        torch.full((B, K + 1), -7, dtype=torch.int32, device=DEV))
    r.target_lse = torch.zeros(B, K + 1, device=DEV)
    r.target_entropy = torch.zeros(B, K + 1, device=DEV)
    r.target_argmax = torch.zeros(B, K + 1, dtype=torch.int32, device=DEV)
    return r


def _same(a, b):
    for k in ("accepted_len", "tokens", "target_lse", "target_entropy", "target_argmax"):
        x, y = getattr(a, k), getattr(b, k)
        assert torch.equal(x, y), k


def _replay_check(call, B, K, workspace, reps=3):
    ref_out = _result(B, K)
    call(ref_out, workspace)            # eager
    torch.cuda.synchronize()
    out = _result(B, K)
    call(out, workspace)                # warm-up on the side stream torch requires
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out, workspace)
    for _ in range(reps):
        for t in (out.accepted_len, out.tokens):
            t.fill_(-7)                 # stale values must be overwritten
        junk = torch.randn(1 << 20, device=DEV).sum()   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _same(out, ref_out)
        assert junk.isfinite()


def test_fly_verify_replays():
    b = W.make(2, B=32)
    t, tok = b.target.to(DEV), b.tokens.to(DEV)
    B, K = tok.shape
    ws = torch.empty(sv.workspace_bytes(B, K, b.V), dtype=torch.uint8, device=DEV)

    def call(out, workspace):
        sv.verify(t, None, tok, seed=0, mode=sv.MODE_FLY, fly_theta=0.3, fly_window=4,
                  workspace=workspace, out=out)
    _replay_check(call, B, K, ws)


def test_lossless_verify_replays():
    b = W.make(3, B=24)
    t, d, tok = b.target.to(DEV), b.draft.to(DEV), b.tokens.to(DEV)
    B, K = tok.shape
    ws = torch.empty(sv.workspace_bytes(B, K, b.V, temperature=0.7), dtype=torch.uint8,
                     device=DEV)

    def call(out, workspace):
        sv.verify(t, d, tok, seed=5, temperature=0.7, workspace=workspace, out=out)
    _replay_check(call, B, K, ws)


def test_av_step_replays():
    # score, trimmed verify and the SGD step, with the parameters reset before
    # each replay so that every replay starts from the same state
    b = W.make(4, B=40, V=5000, stride=5000)
    t, d, tok = b.target.to(DEV), b.draft.to(DEV), b.tokens.to(DEV)
    B, K = tok.shape
    ob0 = torch.tensor(W.av_init(4), dtype=torch.float32, device=DEV)
    ob = ob0.clone()
    ds = torch.empty(sv.load().spec_draft_stats_bytes(B, K), dtype=torch.uint8, device=DEV)
    ws = torch.empty(sv.workspace_bytes(B, K, 5000), dtype=torch.uint8, device=DEV)
    out = _result(B, K)

    def step():
        _, _, kept, _ = sv.av_score(d, tok, ob, 0.2, vocab=5000, draft_stats=ds)
        sv.verify(t, d, tok, seed=1, vocab=5000, kept_len=kept, draft_stats=ds, workspace=ws,
                  out=out)
        sv.av_update(ds, out.accepted_len, kept, ob, 0.05, B, K)
    step()
    torch.cuda.synchronize()
    want_ob, want_acc = ob.clone(), out.accepted_len.clone()
    ob.copy_(ob0)
    step()  # warm-up
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    ob.copy_(ob0)
    with torch.cuda.graph(g):
        step()
    for _ in range(3):
        ob.copy_(ob0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ob, want_ob) and torch.equal(out.accepted_len, want_acc)


def test_av_step_untrimmed_replays():
    # the tau <= 0 step: a verify that exports the draft statistics, then the
    # one-launch score and SGD step, recorded and replayed
    b = W.make(1, B=40, V=5000, stride=5000)
    t, d, tok = b.target.to(DEV), b.draft.to(DEV), b.tokens.to(DEV)
    B, K = tok.shape
    ob0 = torch.tensor(W.av_init(1), dtype=torch.float32, device=DEV)
    ob = ob0.clone()
    ws = torch.empty(sv.workspace_bytes(B, K, 5000), dtype=torch.uint8, device=DEV)
    out = _result(B, K)
    out.draft_stats_out = torch.empty(sv.draft_stats_bytes(B, K), dtype=torch.uint8, device=DEV)
    res = {}

    def step():
        sv.verify(t, d, tok, seed=2, vocab=5000, workspace=ws, out=out)
        res["conf"], _, _ = sv.av_score_update(out.draft_stats_out, out.accepted_len, ob, 0.05,
                                               B, K)
    step()
    torch.cuda.synchronize()
    want_ob, want_acc, want_conf = ob.clone(), out.accepted_len.clone(), res["conf"].clone()
    ob.copy_(ob0)
    step()  # warm-up
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    ob.copy_(ob0)
    with torch.cuda.graph(g):
        step()
    for _ in range(3):
        ob.copy_(ob0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ob, want_ob) and torch.equal(out.accepted_len, want_acc)
        assert torch.equal(res["conf"], want_conf)


@pytest.mark.parametrize("tau", [0.0, 0.2])
def test_av_step_call_replays(tau):
    # AvStepCall, whose verification and update are one spec_verify_update
    # call (the update in the token-picking launch), recorded and replayed.
    # The call binds its stream when it is built, so it is built, warmed up
    # and captured on one side stream.
    b = W.make(1, B=40, V=5000, stride=5000)
    t, d, tok = b.target.to(DEV), b.draft.to(DEV), b.tokens.to(DEV)
    ob0 = torch.tensor(W.av_init(1), dtype=torch.float32, device=DEV)
    ob = ob0.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call = sv.AvStepCall(t, d, tok, ob, tau, 0.05, vocab=5000)
        call(3)
    torch.cuda.synchronize()
    out = call.verify.out
    want_ob, want_acc, want_tok = ob.clone(), out.accepted_len.clone(), out.tokens.clone()
    with torch.cuda.stream(s):
        ob.copy_(ob0)
        call(3)  # warm-up
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call(3)
    for _ in range(3):
        ob.copy_(ob0)
        out.tokens.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ob, want_ob) and torch.equal(out.accepted_len, want_acc)
        assert torch.equal(out.tokens, want_tok)
