"""ctypes wrapper of the CPU oracle (specverify_ref.c).

TEST INFRASTRUCTURE ONLY: imported by the test suite, by the smoke check and by
the benchmark's CPU-baseline leg.  The HIP library never imports this module
and this module never imports the library.

All arrays are host numpy arrays.  Logits are float32 (dtype 0) or bfloat16
bit patterns held in uint16 arrays (dtype 1).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "specverify_ref.c")
_HDR = os.path.join(_HERE, "specverify_ref.h")
LIB_PATH = os.path.join(_HERE, "libspecverify_ref.so")

TAG_ACCEPT = 1
TAG_RACE = 2
TAG_SCREEN = 3
NEAR_ACCEPT = 1
NEAR_RACE = 2
RESIDUAL_EMPTY = 4
NEAR_GATE = 8
NEAR_TRIM = 16
MODE_LOSSLESS = 0
MODE_FLY = 1

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C99, no fast-math, no contraction)."""
    if not force and os.path.exists(LIB_PATH):
        return LIB_PATH
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=gnu99", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
           "-shared", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm", "-lpthread"]
    subprocess.check_call(cmd)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        i64, i32, u32, u64, f64 = (ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32,
                                   ctypes.c_uint64, ctypes.c_double)
        L.ref_philox4x32_10.argtypes = [P, P, P]
        L.ref_philox4x32_10.restype = None
        L.ref_draw_u32.argtypes = [u64, u32, u32, u32, u32]
        L.ref_draw_u32.restype = u32
        L.ref_uniform.argtypes = [u64, u32, u32, u32, u32]
        L.ref_uniform.restype = f64
        L.ref_race_u32.argtypes = [u64, u32, u32, u32]
        L.ref_race_u32.restype = u32
        L.ref_race_uniform.argtypes = [u64, u32, u32, u32]
        L.ref_race_uniform.restype = f64
        L.ref_rows_stats.argtypes = [P, i64, i64, i64, ctypes.c_int, f64, P, P, P, P, P, P, P,
                                     ctypes.c_int]
        L.ref_rows_stats.restype = ctypes.c_int
        L.ref_row_probs.argtypes = [P, i64, ctypes.c_int, f64, P]
        L.ref_row_probs.restype = ctypes.c_int
        L.ref_race.argtypes = [P, i64, u64, u32, u32, P]
        L.ref_race.restype = i64
        L.ref_residual.argtypes = [P, P, i64, P]
        L.ref_residual.restype = None
        L.ref_fly_resolve.argtypes = [ctypes.c_int, ctypes.c_int, f64, P, P, P]
        L.ref_fly_resolve.restype = ctypes.c_int
        L.ref_verify.argtypes = [P, P, P, P, i32, i32, i64, i64, i32, f64, u64, i32, f64, i32,
                                 P, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_int]
        L.ref_verify.restype = ctypes.c_int
        L.ref_av_score.argtypes = [P, i32, i32, P, f64, P, P, P, P]
        L.ref_av_score.restype = None
        L.ref_av_loss.argtypes = [P, P, P, i32, i32, P, P]
        L.ref_av_loss.restype = f64
        L.ref_av_update.argtypes = [P, P, P, i32, i32, f64, P]
        L.ref_irls_accumulate.argtypes = [P, P, P, i32, i32, P, P, P, P]
        L.ref_irls_accumulate.restype = None
        L.ref_irls_solve.argtypes = [i32, f64, P, P, P, P]
        L.ref_irls_solve.restype = ctypes.c_int
        L.ref_av_diagnostics.argtypes = [P, P, P, i32, i32, P, i32, P, P]
        L.ref_av_diagnostics.restype = None
        L.ref_av_budget.argtypes = [P, i32, i32, P, f64, P, P, P, P]
        L.ref_av_budget.restype = i64
        L.ref_ngram_propose.argtypes = [P, P, i32, i64, i32, i32, i32, P, P, P, P]
        L.ref_ngram_propose.restype = None
        L.ref_av_update.restype = None
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _logits(a):
    """Return (contiguous array, dtype code) for float32 or bf16-bits input."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a, 0
    if a.dtype == np.uint16:
        return a, 1
    raise TypeError("oracle logits must be float32 or uint16 (bfloat16 bits), got %s" % a.dtype)


def default_threads() -> int:
    return max(1, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else 1)


# ---------------------------------------------------------------------------
def philox4x32_10(ctr, key):
    c = np.asarray(ctr, dtype=np.uint32).copy()
    k = np.asarray(key, dtype=np.uint32).copy()
    out = np.zeros(4, dtype=np.uint32)
    lib().ref_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def draw_u32(seed, x, pos, b, tag):
    return int(lib().ref_draw_u32(seed, x, pos, b, tag))


def uniform(seed, x, pos, b, tag):
    return float(lib().ref_uniform(seed, x, pos, b, tag))


def race_u32(seed, x, pos, b):
    return int(lib().ref_race_u32(seed, x, pos, b))


def race_uniform(seed, x, pos, b):
    return float(lib().ref_race_uniform(seed, x, pos, b))


def rows_stats(logits2d, temperature=1.0, nthreads=None, V=None):
    """Statistics of every row of a [rows, stride] array (the first V columns)."""
    a, dt = _logits(logits2d)
    rows, stride = a.shape
    V = stride if V is None else V
    out = {k: np.empty(rows, dtype=np.float64) for k in ("m", "lse", "H", "h", "qmax", "feat")}
    out["argmax"] = np.empty(rows, dtype=np.int64)
    rc = lib().ref_rows_stats(_ptr(a), rows, V, stride, dt, float(temperature), _ptr(out["m"]),
                              _ptr(out["lse"]), _ptr(out["H"]), _ptr(out["h"]),
                              _ptr(out["argmax"]), _ptr(out["qmax"]), _ptr(out["feat"]),
                              nthreads or default_threads())
    if rc != 0:
        raise ValueError("ref_rows_stats rejected its arguments")
    return out


def row_probs(row, temperature=1.0):
    a, dt = _logits(row)
    p = np.empty(a.shape[-1], dtype=np.float64)
    if lib().ref_row_probs(_ptr(a), a.shape[-1], dt, float(temperature), _ptr(p)) != 0:
        raise ValueError("ref_row_probs rejected its arguments")
    return p


def race(w, seed, pos, b):
    w = np.ascontiguousarray(w, dtype=np.float64)
    gap = np.zeros(1, dtype=np.float64)
    y = lib().ref_race(_ptr(w), w.shape[0], seed, pos, b, _ptr(gap))
    return int(y), float(gap[0])


def residual(p, q):
    p = np.ascontiguousarray(p, dtype=np.float64)
    q = np.ascontiguousarray(q, dtype=np.float64)
    w = np.empty_like(p)
    lib().ref_residual(_ptr(p), _ptr(q), p.shape[0], _ptr(w))
    return w


def fly_resolve(dev, h, W, theta):
    """Returns (accepted count, near-gate flag, smallest |h - theta| over the
    evaluated gates)."""
    dev = np.ascontiguousarray(dev, dtype=np.int32)
    h = np.ascontiguousarray(h, dtype=np.float64)
    gap = ctypes.c_double(0.0)
    n = lib().ref_fly_resolve(int(dev.shape[0]), int(W), float(theta), _ptr(dev), _ptr(h),
                              ctypes.byref(gap))
    return int(n), bool(gap.value < 1e-5), float(gap.value)


def verify(target, draft, tokens, seed, mode=MODE_LOSSLESS, *, temperature=1.0, theta=0.3,
           window=4, kept_len=None, V=None, nthreads=None):
    """Oracle verification.  target: [B, K+1, stride], draft: [B, K, stride] or None."""
    t, dt = _logits(target)
    B, K1, stride = t.shape
    K = K1 - 1
    V = stride if V is None else V
    d = None
    if draft is not None:
        d, dd = _logits(draft)
        if dd != dt or d.shape != (B, K, stride):
            raise ValueError("draft must match target in dtype, batch and stride")
    tok = np.ascontiguousarray(tokens, dtype=np.int32).reshape(B, K)
    kl = None if kept_len is None else np.ascontiguousarray(kept_len, dtype=np.int32)
    r = {
        "accepted_len": np.zeros(B, dtype=np.int32),
        "tokens": np.zeros((B, K + 1), dtype=np.int32),
        "t_lse": np.zeros((B, K + 1)), "t_h": np.zeros((B, K + 1)),
        "t_argmax": np.zeros((B, K + 1), dtype=np.int64),
        "d_lse": np.zeros((B, K)), "d_qmax": np.zeros((B, K)), "d_feat": np.zeros((B, K)),
        "boundary": np.zeros(B, dtype=np.uint32), "race_gap": np.zeros(B),
        "accept_gap": np.zeros(B), "gate_gap": np.zeros(B),
    }
    rc = lib().ref_verify(_ptr(t), _ptr(d), _ptr(tok), _ptr(kl), B, K, V, stride, dt,
                          float(temperature), int(seed), int(mode), float(theta), int(window),
                          _ptr(r["accepted_len"]), _ptr(r["tokens"]), _ptr(r["t_lse"]),
                          _ptr(r["t_h"]), _ptr(r["t_argmax"]), _ptr(r["d_lse"]),
                          _ptr(r["d_qmax"]), _ptr(r["d_feat"]), _ptr(r["boundary"]),
                          _ptr(r["race_gap"]), _ptr(r["accept_gap"]), _ptr(r["gate_gap"]),
                          nthreads or default_threads())
    if rc != 0:
        raise ValueError("ref_verify rejected its arguments")
    return r


def av_score(feat, omega_beta, tau):
    feat = np.ascontiguousarray(feat, dtype=np.float64)
    B, K = feat.shape
    ob = np.ascontiguousarray(omega_beta, dtype=np.float64)
    if ob.shape != (K + 1,):
        raise ValueError("omega_beta must hold K+1 values")
    conf = np.zeros((B, K))
    mask = np.zeros((B, K), dtype=np.uint8)
    kept = np.zeros(B, dtype=np.int32)
    near = np.zeros(B, dtype=np.uint32)
    lib().ref_av_score(_ptr(feat), B, K, _ptr(ob), float(tau), _ptr(conf), _ptr(mask),
                       _ptr(kept), _ptr(near))
    return conf, mask, kept, near


def av_loss(feat, accepted_len, kept_len, omega_beta):
    feat = np.ascontiguousarray(feat, dtype=np.float64)
    B, K = feat.shape
    acc = np.ascontiguousarray(accepted_len, dtype=np.int32)
    kl = None if kept_len is None else np.ascontiguousarray(kept_len, dtype=np.int32)
    ob = np.ascontiguousarray(omega_beta, dtype=np.float64)
    n = ctypes.c_int64(0)
    v = lib().ref_av_loss(_ptr(feat), _ptr(acc), _ptr(kl), B, K, _ptr(ob), ctypes.byref(n))
    return float(v), int(n.value)


def av_update(feat, accepted_len, kept_len, omega_beta, lr):
    feat = np.ascontiguousarray(feat, dtype=np.float64)
    B, K = feat.shape
    acc = np.ascontiguousarray(accepted_len, dtype=np.int32)
    kl = None if kept_len is None else np.ascontiguousarray(kept_len, dtype=np.int32)
    ob = np.array(omega_beta, dtype=np.float64, copy=True)
    lib().ref_av_update(_ptr(feat), _ptr(acc), _ptr(kl), B, K, float(lr), _ptr(ob))
    return ob


class IrlsState:
    """Round accumulators of the IRLS refit: gradient, dense Hessian and the
    label count behind each coefficient (all zero at the start of a round)."""

    def __init__(self, K):
        self.K = K
        self.g = np.zeros(K + 1)
        self.H = np.zeros((K + 1, K + 1))
        self.cnt = np.zeros(K + 1, dtype=np.int64)


def irls_accumulate(state, feat, accepted_len, kept_len, omega_beta):
    f = np.ascontiguousarray(feat, dtype=np.float64)
    B, K = f.shape
    assert K == state.K
    a = np.ascontiguousarray(accepted_len, dtype=np.int32)
    kl = None if kept_len is None else np.ascontiguousarray(kept_len, dtype=np.int32)
    ob = np.ascontiguousarray(omega_beta, dtype=np.float64)
    lib().ref_irls_accumulate(_ptr(f), _ptr(a), _ptr(kl), B, K, _ptr(ob), _ptr(state.g),
                              _ptr(state.H), _ptr(state.cnt))


def irls_solve(state, omega_beta, c_damp):
    """Solve the round's Newton system and update (a copy of) omega_beta.
    Returns (new omega_beta, flags); the state is reset."""
    ob = np.array(omega_beta, dtype=np.float64)
    flags = lib().ref_irls_solve(state.K, float(c_damp), _ptr(state.g), _ptr(state.H),
                                 _ptr(state.cnt), _ptr(ob))
    return ob, int(flags)


def av_diagnostics(feat, accepted_len, kept_len, omega_beta, nbins=10):
    f = np.ascontiguousarray(feat, dtype=np.float64)
    B, K = f.shape
    a = np.ascontiguousarray(accepted_len, dtype=np.int32)
    kl = None if kept_len is None else np.ascontiguousarray(kept_len, dtype=np.int32)
    ob = np.ascontiguousarray(omega_beta, dtype=np.float64)
    out = np.zeros(4)
    near = ctypes.c_int32(0)
    lib().ref_av_diagnostics(_ptr(f), _ptr(a), _ptr(kl), B, K, _ptr(ob), int(nbins), _ptr(out),
                             ctypes.byref(near))
    return {"auc": out[0], "logloss": out[1], "ece": out[2], "n": int(out[3]),
            "near_bin_edge": bool(near.value)}


def av_budget(conf, cost, n_requests=None):
    c = np.ascontiguousarray(conf, dtype=np.float32)
    B, K = c.shape
    cs = np.ascontiguousarray(cost, dtype=np.float64)
    assert cs.shape == (B * K + 1,)
    kept = np.zeros(B, dtype=np.int32)
    mask = np.zeros((B, K), dtype=np.uint8)
    best = ctypes.c_double(0.0)
    near = ctypes.c_int32(0)
    nr = float(B if n_requests is None else n_requests)
    k = lib().ref_av_budget(_ptr(c), B, K, _ptr(cs), nr, _ptr(kept), _ptr(mask),
                            ctypes.byref(best), ctypes.byref(near))
    return {"budget": int(k), "kept_len": kept, "mask": mask, "best_ratio": best.value,
            "near": bool(near.value)}


def ngram_propose(ctx, lengths, n_min, n_max, K):
    c = np.ascontiguousarray(ctx, dtype=np.int32)
    B, S = c.shape
    ln = np.ascontiguousarray(lengths, dtype=np.int32)
    draft = np.zeros((B, K), dtype=np.int32)
    dl = np.zeros(B, dtype=np.int32)
    mp = np.zeros(B, dtype=np.int32)
    mn = np.zeros(B, dtype=np.int32)
    lib().ref_ngram_propose(_ptr(c), _ptr(ln), B, S, int(n_min), int(n_max), int(K), _ptr(draft),
                            _ptr(dl), _ptr(mp), _ptr(mn))
    return {"draft": draft, "draft_len": dl, "match_pos": mp, "match_n": mn}
