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


def compare_decisions(acc_gpu, tok_gpu, ref, allowed_bits, what=""):
    """Bit-exact accepted_len and tokens except boundary-flagged sequences.
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
