"""Helpers shared by the GPU parity tests: moving tensors to the oracle's
host layout and comparing results under the acceptance rules.

Acceptance rules (tolerances of the verifier's specification):
  * accepted_len and emitted tokens bit-exact, except sequences the oracle
    flags as boundary cases (a near-tie between u_j and p/q within 1e-5, top
    two race keys within 1e-6 relative, an FLy gate within 1e-5 of theta, an
    AV survival product within 1e-5 relative of tau);
  * float statistics within 1e-5 relative for float32 logits and 1e-4
    relative for bfloat16 logits (float32 accumulation).
"""
import os

import numpy as np
import torch

REL_TOL = {torch.float32: 1e-5, torch.bfloat16: 1e-4}


def host_logits(t: torch.Tensor) -> np.ndarray:
    """float32 -> float32 array; bfloat16 -> uint16 bit patterns."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def f32(x) -> float:
    """The float32 value the library receives for a Python float."""
    return float(np.float32(x))


def oracle_threads() -> int:
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else 8
    return max(1, min(n, 16))


def assert_close(got, ref, rel, what, abs_floor=0.0):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    nan_ref = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan_ref), "%s: NaN pattern differs" % what
    g, r = got[~nan_ref], ref[~nan_ref]
    err = np.abs(g - r)
    lim = rel * np.abs(r) + abs_floor
    bad = err > lim
    if bad.any():
        i = int(np.argmax(err - lim))
        raise AssertionError("%s: %d/%d outside rel %.1e (worst got %r ref %r)"
                             % (what, int(bad.sum()), bad.size, rel, g[i], r[i]))


# Boundary bits (the oracle's and the library's share their values).
NEAR_ACCEPT, NEAR_RACE, RESIDUAL_EMPTY, NEAR_GATE = 1, 2, 4, 8

# Session-wide tally of the decisions compared: sequences, verified rows
# (sum over sequences of kept length + 1: the rows a decision is made over),
# boundary-flagged sequences (by the library or the oracle) and mismatched
# sequences.  "workload" counts the workload recipes and random
# configurations; "constructed" counts inputs built to sit on a boundary
# (their flags are the point of the test, not a rate).
TALLY = {k: {"calls": 0, "sequences": 0, "rows": 0, "flagged": 0, "mismatched": 0}
         for k in ("workload", "constructed")}


def _flag_noise(bit, ref):
    """Sequences where the oracle's distance behind `bit` is within float
    noise of its threshold, so that the library's float32 row statistics may
    flag it the other way: |u - p/q| within 1e-6 of 1e-5 (the row pass's
    ratio carries ~1e-7 relative error), |h - theta| within 2e-6 of 1e-5,
    the race gap within [5e-7, 2e-6] (device keys carry ~1e-7 relative
    error).  A vanished residual is only possible after a near-accept
    rejection, so its flag may differ there."""
    if bit == NEAR_ACCEPT:
        return np.abs(ref["accept_gap"] - 1e-5) <= 1e-6
    if bit == NEAR_GATE:
        return np.abs(ref["gate_gap"] - 1e-5) <= 2e-6
    if bit == NEAR_RACE:
        g = ref["race_gap"]
        return np.isnan(g) | ((g >= 5e-7) & (g <= 2e-6))
    if bit == RESIDUAL_EMPTY:
        return (ref["boundary"] & NEAR_ACCEPT) != 0
    return np.zeros(ref["boundary"].shape, dtype=bool)


def compare_decisions(acc_gpu, tok_gpu, ref, allowed_bits, what="", dev_boundary=None,
                      kept=None, tally="workload"):
    """Bit-exact accepted_len and tokens except boundary-flagged sequences.

    ref: the oracle's verify result.  dev_boundary: the library's boundary
    bits for the same sequences (or None).  With them, every mismatched
    sequence must carry a flag on both sides, and the two sides' flags must
    agree except where the oracle's distance behind a flag is within float
    noise of its threshold (_flag_noise).  kept: the kept lengths the call
    verified (None: every draft), for the tally's row count.
    Returns (number of mismatches, number of boundary sequences)."""
    acc_gpu = np.asarray(acc_gpu)
    tok_gpu = np.asarray(tok_gpu)
    mism = (acc_gpu != ref["accepted_len"]) | np.any(tok_gpu != ref["tokens"], axis=1)
    bnd = (ref["boundary"] & allowed_bits) != 0
    bad = mism & ~bnd
    if bad.any():
        b = int(np.flatnonzero(bad)[0])
        raise AssertionError(
            "%s: %d sequences differ outside the boundary set; first b=%d gpu acc=%d tok=%s "
            "ref acc=%d tok=%s boundary=%d gap=%r" % (
                what, int(bad.sum()), b, acc_gpu[b], tok_gpu[b].tolist(),
                ref["accepted_len"][b], ref["tokens"][b].tolist(), ref["boundary"][b],
                ref["race_gap"][b]))
    flagged = bnd
    if dev_boundary is not None:
        dev = np.asarray(dev_boundary).astype(np.uint32)
        dbnd = (dev & allowed_bits) != 0
        unlogged = mism & ~dbnd
        if unlogged.any():
            b = int(np.flatnonzero(unlogged)[0])
            raise AssertionError("%s: %d mismatched sequences carry no library flag; first b=%d "
                                 "oracle boundary=%d" % (what, int(unlogged.sum()), b,
                                                         ref["boundary"][b]))
        same_path = ~mism  # flags of sequences decided alike
        for bit in (NEAR_ACCEPT, NEAR_RACE, RESIDUAL_EMPTY, NEAR_GATE):
            if not (bit & allowed_bits):
                continue
            differ = ((dev & bit) != 0) != ((ref["boundary"] & bit) != 0)
            if bit in (NEAR_RACE, RESIDUAL_EMPTY):
                differ &= same_path  # a different decision races another row
            odd = differ & ~_flag_noise(bit, ref)
            if odd.any():
                b = int(np.flatnonzero(odd)[0])
                raise AssertionError(
                    "%s: boundary bit %d differs from the oracle's at %d sequences; first b=%d "
                    "library=%d oracle=%d accept_gap=%r race_gap=%r gate_gap=%r" % (
                        what, bit, int(odd.sum()), b, dev[b], ref["boundary"][b],
                        ref["accept_gap"][b], ref["race_gap"][b], ref["gate_gap"][b]))
        flagged = bnd | dbnd
    B, K1 = tok_gpu.shape
    L = np.full(B, K1 - 1) if kept is None else np.clip(np.asarray(kept), 0, K1 - 1)
    t = TALLY[tally]
    t["calls"] += 1
    t["sequences"] += B
    t["rows"] += int((L + 1).sum())
    t["flagged"] += int(flagged.sum())
    t["mismatched"] += int(mism.sum())
    return int(mism.sum()), int(bnd.sum())


def check_token_layout(acc, tok, tokens_in, kept=None):
    """Properties that hold at any size: accepted drafts are copied, one
    more token follows, the rest is -1."""
    acc = np.asarray(acc)
    tok = np.asarray(tok)
    tokens_in = np.asarray(tokens_in)
    B, K1 = tok.shape
    K = K1 - 1
    L = np.full(B, K) if kept is None else np.clip(np.asarray(kept), 0, K)
    assert np.all((acc >= 0) & (acc <= L))
    for b in range(B):
        a = acc[b]
        assert np.array_equal(tok[b, :a], tokens_in[b, :a])
        assert tok[b, a] >= 0
        assert np.all(tok[b, a + 1:] == -1)
