"""The acceptance bound on the boundary set.

accepted_len and the emitted tokens must equal the oracle's bit for bit,
except on a logged set of near-ties (an accept test with |u - p/q| < 1e-5,
race keys whose two largest lie within 1e-6 relative; page "Speculative
Decoding: ...", section "Математика верификации", for the accept rule), and
that set must stay below 1e-4 of the rows verified.  Every comparison in the
GPU suite already requires each mismatch to carry both the oracle's flag and
the library's (tests/parity_util.py).  This file measures the set's size:

  * over its own sweep of the workload recipes at their full sizes, many
    seeds each, so that it means something when run alone;
  * over every workload comparison the session made before it (the
    constructed near-tie tests are counted apart: their flags are the point).

Rows are the verified target rows: kept length + 1 per sequence (K + 1
without trimming), the rows a decision is made over.  Flagged sequences are
those the library or the oracle flags.
"""
import numpy as np
import pytest
import torch

import draft_token_verification_vocab_amd as sv
from draft_token_verification_vocab_amd import workloads as W
from oracle import ref
from parity_util import TALLY, compare_decisions, f32, host_logits, oracle_threads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
NT = oracle_threads()
ALL_NEAR = ref.NEAR_ACCEPT | ref.NEAR_RACE | ref.RESIDUAL_EMPTY | ref.NEAR_GATE
BOUND = 1e-4


def _snapshot():
    return dict(TALLY["workload"])


def _diff(a, b):
    return {k: b[k] - a[k] for k in a}


def _lossless(batch, seeds):
    t, d, tok = batch.target.to(DEV), batch.draft.to(DEV), batch.tokens.to(DEV)
    th, dh, xh = host_logits(batch.target), host_logits(batch.draft), batch.tokens.cpu().numpy()
    T = batch.temperature
    for seed in seeds:
        r = sv.verify(t, d, tok, seed=seed, temperature=T, vocab=batch.V, boundary=True)
        torch.cuda.synchronize()
        o = ref.verify(th, dh, xh, seed, temperature=f32(T), V=batch.V, nthreads=NT)
        compare_decisions(r.accepted_len.cpu().numpy(), r.tokens.cpu().numpy(), o, ALL_NEAR,
                          "boundary sweep", dev_boundary=r.boundary.cpu().numpy())


def _fly(batch, theta, window):
    r = sv.verify(batch.target.to(DEV), None, batch.tokens.to(DEV), seed=0, mode=sv.MODE_FLY,
                  fly_theta=theta, fly_window=window, vocab=batch.V, boundary=True)
    torch.cuda.synchronize()
    o = ref.verify(host_logits(batch.target), None, batch.tokens.cpu().numpy(), 0, ref.MODE_FLY,
                   theta=f32(theta), window=window, V=batch.V, nthreads=NT)
    compare_decisions(r.accepted_len.cpu().numpy(), r.tokens.cpu().numpy(), o, ref.NEAR_GATE,
                      "boundary sweep", dev_boundary=r.boundary.cpu().numpy())


def _report(name, t):
    frac = t["flagged"] / max(t["rows"], 1)
    print("%s: %d calls, %d sequences, %d rows, %d flagged (%.2e of rows), %d mismatched"
          % (name, t["calls"], t["sequences"], t["rows"], t["flagged"], frac, t["mismatched"]))
    return frac


def test_boundary_set_below_bound_on_the_workloads():
    before = _snapshot()
    # B=1 K=4 V=32000 float32, T=1: 1000 verification seeds
    _lossless(W.make(0, device=DEV), range(1000))
    # B=64 K=5 V=128256 bf16: 40 seeds
    _lossless(W.make(1, device=DEV), range(40))
    # the FLy headline batch, B=256 K=8 V=128256 bf16, theta=0.3, W=4
    c2 = W.CONFIGS[2]
    _fly(W.make(2, device=DEV), c2["theta"], c2["window"])
    # lossless at the headline shape: 8 seeds
    _lossless(W.gaussian(256, 8, 128256, "bf16", 1.0, seed=77, token_seed=0, device=DEV),
              range(8))
    # B=512 K=4 V=152064 bf16 at T=0.7: 12 seeds
    _lossless(W.make(3, device=DEV), range(12))
    own = _diff(before, _snapshot())
    frac = _report("own sweep", own)
    assert own["rows"] > 50000
    assert own["mismatched"] <= own["flagged"]
    assert frac < BOUND, own


def test_boundary_set_below_bound_over_the_session():
    # every workload comparison of this session (this file's sweep included)
    t = TALLY["workload"]
    frac = _report("session, workloads", t)
    _report("session, constructed near-ties", TALLY["constructed"])
    assert t["rows"] > 0
    assert t["mismatched"] <= t["flagged"]
    assert frac < BOUND, t
