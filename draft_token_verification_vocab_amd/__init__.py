"""Batched speculative-decoding verification over full-vocabulary logits on
AMD MI355X (gfx950).

A thin ctypes binding of the HIP library ``libspecverify.so`` (C ABI in
``include/specverify.h``).  This module only marshals arguments: it checks
shapes, allocates outputs and workspace as torch tensors on the logits'
device and passes raw device pointers plus the current HIP stream.  Every step
of the computation runs in the library's kernels; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

__all__ = [
    "SpecVerifyError", "lib_path", "load", "verify", "av_score", "av_score_stats", "av_update",
    "row_stats",
    "workspace_bytes", "draft_stats_bytes", "MODE_LOSSLESS", "MODE_FLY",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
MODE_LOSSLESS = 0
MODE_FLY = 1
DTYPE_F32 = 0
DTYPE_BF16 = 1
# boundary-case bits of VerifyResult.boundary (see include/specverify.h)
NEAR_ACCEPT = 1
NEAR_RACE = 2
RESIDUAL_EMPTY = 4
NEAR_GATE = 8


class SpecVerifyError(RuntimeError):
    pass


class _Params(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_draft", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("row_stride", ctypes.c_int64), ("temperature", ctypes.c_float),
                ("fly_theta", ctypes.c_float), ("fly_window", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class _VerifyOut(ctypes.Structure):
    _fields_ = [("accepted_len", ctypes.c_void_p), ("tokens", ctypes.c_void_p),
                ("target_lse", ctypes.c_void_p), ("target_entropy", ctypes.c_void_p),
                ("target_argmax", ctypes.c_void_p), ("draft_lse", ctypes.c_void_p),
                ("draft_qmax", ctypes.c_void_p), ("draft_feat", ctypes.c_void_p),
                ("draft_stats_out", ctypes.c_void_p), ("boundary", ctypes.c_void_p)]


# Every symbol the header declares, with its ctypes signature.
_P = ctypes.c_void_p
_SIGNATURES = {
    "spec_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(_Params)]),
    "spec_draft_stats_bytes": (ctypes.c_size_t, [ctypes.c_int32, ctypes.c_int32]),
    "spec_verify": (ctypes.c_int32, [_P, _P, _P, _P, _P, ctypes.c_uint64, ctypes.c_int32,
                                     ctypes.POINTER(_Params), ctypes.POINTER(_VerifyOut), _P,
                                     ctypes.c_size_t, _P]),
    "spec_verify_update": (ctypes.c_int32, [_P, _P, _P, _P, _P, ctypes.c_uint64,
                                            ctypes.POINTER(_Params), ctypes.POINTER(_VerifyOut),
                                            ctypes.c_float, _P, _P, _P, _P, _P, ctypes.c_size_t,
                                            _P]),
    "spec_verify_noalloc": (ctypes.c_int32, [_P, _P, _P, _P, _P, ctypes.c_uint64,
                                             ctypes.c_int32, ctypes.POINTER(_Params),
                                             ctypes.POINTER(_VerifyOut), _P]),
    "spec_av_score": (ctypes.c_int32, [_P, _P, ctypes.POINTER(_Params), _P, ctypes.c_float,
                                       _P, _P, _P, _P, _P]),
    "spec_av_score_prefix": (ctypes.c_int32, [_P, _P, ctypes.POINTER(_Params), _P,
                                              ctypes.c_float, _P, _P, _P, _P, _P]),
    "spec_av_score_stats": (ctypes.c_int32, [_P, ctypes.c_int32, ctypes.c_int32, _P,
                                             ctypes.c_float, _P, _P, _P, _P]),
    "spec_av_update": (ctypes.c_int32, [_P, _P, _P, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_float, _P, _P]),
    "spec_av_score_update": (ctypes.c_int32, [_P, _P, ctypes.c_int32, ctypes.c_int32,
                                              ctypes.c_float, _P, _P, _P, _P, _P]),
    "spec_row_stats": (ctypes.c_int32, [_P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int64,
                                        ctypes.c_int32, ctypes.c_float, _P, _P, _P, _P, _P, _P]),
    "spec_read_probe": (ctypes.c_int32, [_P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                         _P, _P]),
    "spec_irls_state_bytes": (ctypes.c_size_t, [ctypes.c_int32]),
    "spec_irls_reset": (ctypes.c_int32, [_P, ctypes.c_int32, _P]),
    "spec_irls_accumulate": (ctypes.c_int32, [_P, _P, _P, ctypes.c_int32, ctypes.c_int32, _P, _P,
                                              _P]),
    "spec_irls_solve": (ctypes.c_int32, [_P, ctypes.c_int32, ctypes.c_double, _P, _P, _P]),
    "spec_av_diagnostics_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int32, ctypes.c_int32,
                                                              ctypes.c_int32]),
    "spec_av_diagnostics": (ctypes.c_int32, [_P, _P, _P, ctypes.c_int32, ctypes.c_int32, _P,
                                             ctypes.c_int32, _P, _P, ctypes.c_size_t, _P]),
    "spec_av_budget_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int32, ctypes.c_int32]),
    "spec_av_budget": (ctypes.c_int32, [_P, ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_double,
                                        _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "spec_ngram_propose": (ctypes.c_int32, [_P, _P, ctypes.c_int32, ctypes.c_int64,
                                            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, _P,
                                            _P, _P, _P]),
    "spec_status_string": (ctypes.c_char_p, [ctypes.c_int32]),
}

_lib = None


def lib_path() -> str:
    return os.path.join(_HERE, "libspecverify.so")


def load(path: Optional[str] = None):
    """Load the HIP library (raises if it is missing: there is no fallback)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or lib_path()
    if not os.path.exists(p):
        raise SpecVerifyError(
            "%s is missing: build it with `python -m draft_token_verification_vocab_amd.build`"
            % p)
    L = ctypes.CDLL(p)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = L
    return L


def _check(status: int, what: str):
    if status != 0:
        msg = load().spec_status_string(status).decode()
        raise SpecVerifyError("%s failed: %s (status %d)" % (what, msg, status))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float32:
        return DTYPE_F32
    raise TypeError("logits must be bfloat16 or float32, got %s" % t.dtype)


def _need_cuda(t: torch.Tensor, name: str, device=None, dtype=None, shape=None,
               nbytes: Optional[int] = None):
    """Raise unless t is a contiguous GPU tensor (on device, of dtype and
    shape, holding at least nbytes bytes, where given): the library reads and
    writes through raw device pointers, so a host tensor, another GPU's or a
    short buffer would fault the kernel instead of failing here."""
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if device is not None and t.device != torch.device(device):
        raise ValueError("%s must be on %s, not %s" % (name, device, t.device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must be %s, not %s" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, not %s" % (name, tuple(shape), tuple(t.shape)))
    if nbytes is not None and t.numel() * t.element_size() < nbytes:
        raise ValueError("%s must hold at least %d bytes" % (name, nbytes))


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def _check_labels(dev, B, K, draft_stats, accepted_len, kept_len, omega_beta):
    """The estimator's inputs for a batch of B sequences of K drafts on dev."""
    _need_cuda(draft_stats, "draft_stats", dev, nbytes=draft_stats_bytes(B, K))
    if accepted_len is not None:
        _need_cuda(accepted_len, "accepted_len", dev, torch.int32, (B,))
    if kept_len is not None:
        _need_cuda(kept_len, "kept_len", dev, torch.int32, (B,))
    _need_cuda(omega_beta, "omega_beta", dev, torch.float32, (K + 1,))


def _check_inputs(dev, B, K, S, dtype, draft, draft_tokens, kept_len, draft_stats, workspace):
    """The verification inputs besides the target logits, against a batch of
    B sequences of K drafts with row stride S on device dev."""
    if draft is not None:
        _need_cuda(draft, "draft", dev, dtype, (B, K, S))
    _need_cuda(draft_tokens, "draft_tokens", dev, torch.int32, (B, K))
    if kept_len is not None:
        _need_cuda(kept_len, "kept_len", dev, torch.int32, (B,))
    if draft_stats is not None:
        _need_cuda(draft_stats, "draft_stats", dev, nbytes=draft_stats_bytes(B, K))
    if workspace is not None:
        _need_cuda(workspace, "workspace", dev)


def _params(B, K, V, stride, dtype, temperature, theta=0.0, window=0) -> _Params:
    return _Params(int(B), int(K), int(V), int(dtype), int(stride), float(temperature),
                   float(theta), int(window), 0)


def workspace_bytes(B, K, V, dtype=DTYPE_BF16, stride=None, temperature=1.0) -> int:
    p = _params(B, K, V, stride or V, dtype, temperature)
    return int(load().spec_workspace_bytes(ctypes.byref(p)))


def draft_stats_bytes(B, K) -> int:
    return int(load().spec_draft_stats_bytes(int(B), int(K)))


@dataclass
class VerifyResult:
    accepted_len: torch.Tensor            # int32 [B]
    tokens: torch.Tensor                  # int32 [B, K+1]
    target_lse: Optional[torch.Tensor] = None
    target_entropy: Optional[torch.Tensor] = None
    target_argmax: Optional[torch.Tensor] = None
    draft_lse: Optional[torch.Tensor] = None
    draft_qmax: Optional[torch.Tensor] = None
    draft_feat: Optional[torch.Tensor] = None
    # a draft-statistics buffer (draft_stats_bytes) that a lossless call reading
    # the draft rows itself also fills
    draft_stats_out: Optional[torch.Tensor] = None
    # uint32 [B] (as int32): each sequence's boundary-case bits (NEAR_* above)
    boundary: Optional[torch.Tensor] = None

    def check(self, B: int, K: int, device):
        """Raise unless every output given fits a batch of B sequences of K drafts."""
        i32, f32 = torch.int32, torch.float32
        for name, dt, shape in (("accepted_len", i32, (B,)), ("tokens", i32, (B, K + 1)),
                                ("target_lse", f32, (B, K + 1)),
                                ("target_entropy", f32, (B, K + 1)),
                                ("target_argmax", i32, (B, K + 1)), ("draft_lse", f32, (B, K)),
                                ("draft_qmax", f32, (B, K)), ("draft_feat", f32, (B, K)),
                                ("boundary", i32, (B,))):
            t = getattr(self, name)
            if t is not None:
                _need_cuda(t, name, device, dt, shape)
        if self.draft_stats_out is not None:
            _need_cuda(self.draft_stats_out, "draft_stats_out", device,
                       nbytes=draft_stats_bytes(B, K))

    def fields(self):
        """The output pointers in the order of spec_verify_out."""
        return _VerifyOut(*[None if t is None else t.data_ptr() for t in (
            self.accepted_len, self.tokens, self.target_lse, self.target_entropy,
            self.target_argmax, self.draft_lse, self.draft_qmax, self.draft_feat,
            self.draft_stats_out, self.boundary)])


def verify(target: torch.Tensor, draft: Optional[torch.Tensor], draft_tokens: torch.Tensor,
           seed: int, mode: int = MODE_LOSSLESS, *, temperature: float = 1.0,
           fly_theta: float = 0.3, fly_window: int = 4, kept_len: Optional[torch.Tensor] = None,
           draft_stats: Optional[torch.Tensor] = None, vocab: Optional[int] = None,
           stats: bool = False, boundary: bool = False,
           workspace: Optional[torch.Tensor] = None,
           out: Optional[VerifyResult] = None) -> VerifyResult:
    """Verify drafts.  target: [B, K+1, S] and draft: [B, K, S] logits (S >= V
    is the row stride; V defaults to S), draft_tokens: int32 [B, K].
    stats: also return the per-row statistics; boundary: also return each
    sequence's boundary-case bits."""
    _need_cuda(target, "target")
    B, K1, S = target.shape
    K = K1 - 1
    V = S if vocab is None else int(vocab)
    dt = _dtype_code(target)
    dev = target.device
    _check_inputs(dev, B, K, S, target.dtype, draft, draft_tokens, kept_len, draft_stats,
                  workspace)
    p = _params(B, K, V, S, dt, temperature, fly_theta, fly_window)
    L = load()
    if out is None:
        out = VerifyResult(torch.empty(B, dtype=torch.int32, device=dev),
                           torch.empty(B, K + 1, dtype=torch.int32, device=dev))
        if stats:
            out.target_lse = torch.empty(B, K + 1, dtype=torch.float32, device=dev)
            out.target_entropy = torch.empty(B, K + 1, dtype=torch.float32, device=dev)
            out.target_argmax = torch.empty(B, K + 1, dtype=torch.int32, device=dev)
            if mode == MODE_LOSSLESS and draft_stats is None:
                out.draft_lse = torch.empty(B, K, dtype=torch.float32, device=dev)
                out.draft_qmax = torch.empty(B, K, dtype=torch.float32, device=dev)
                out.draft_feat = torch.empty(B, K, dtype=torch.float32, device=dev)
        if boundary:
            out.boundary = torch.empty(B, dtype=torch.int32, device=dev)
    else:
        out.check(B, K, dev)
    o = out.fields()
    need = int(L.spec_workspace_bytes(ctypes.byref(p)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check(L.spec_verify(_ptr(target), _ptr(draft), _ptr(draft_tokens), _ptr(kept_len),
                         _ptr(draft_stats), ctypes.c_uint64(int(seed) & (2**64 - 1)), int(mode),
                         ctypes.byref(p), ctypes.byref(o), _ptr(workspace),
                         _nbytes(workspace), _stream(dev)), "spec_verify")
    return out


def verify_update(target: torch.Tensor, draft: torch.Tensor, draft_tokens: torch.Tensor,
                  omega_beta: torch.Tensor, lr: float, *, seed: int = 0,
                  temperature: float = 1.0, vocab: Optional[int] = None,
                  kept_len: Optional[torch.Tensor] = None,
                  draft_stats: Optional[torch.Tensor] = None, score: bool = False,
                  boundary: bool = False, workspace: Optional[torch.Tensor] = None):
    """spec_verify_update: lossless verification and the estimator's update
    in one call.  score=True (no kept_len, no draft_stats) also returns the
    confidences at the coefficients before the update, as av_score_update.
    Returns (VerifyResult, conf, keep_mask, kept_len_out); the last three are
    None unless score.  omega_beta is updated in place."""
    _need_cuda(target, "target")
    B, K1, S = target.shape
    K = K1 - 1
    V = S if vocab is None else int(vocab)
    dev = target.device
    if draft is None:
        raise ValueError("verify_update is lossless: it needs the draft logits")
    _check_inputs(dev, B, K, S, target.dtype, draft, draft_tokens, kept_len, draft_stats,
                  workspace)
    _need_cuda(omega_beta, "omega_beta", dev, torch.float32, (K + 1,))
    if score and (kept_len is not None or draft_stats is not None):
        raise ValueError("score needs an untrimmed step: no kept_len, no draft_stats")
    p = _params(B, K, V, S, _dtype_code(target), temperature)
    L = load()
    out = VerifyResult(torch.empty(B, dtype=torch.int32, device=dev),
                       torch.empty(B, K + 1, dtype=torch.int32, device=dev))
    if boundary:
        out.boundary = torch.empty(B, dtype=torch.int32, device=dev)
    conf = mask = kept = None
    if score:
        conf = torch.empty(B, K, dtype=torch.float32, device=dev)
        mask = torch.empty(B, K, dtype=torch.uint8, device=dev)
        kept = torch.empty(B, dtype=torch.int32, device=dev)
    o = out.fields()
    need = int(L.spec_workspace_bytes(ctypes.byref(p)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check(L.spec_verify_update(_ptr(target), _ptr(draft), _ptr(draft_tokens), _ptr(kept_len),
                                _ptr(draft_stats), ctypes.c_uint64(int(seed) & (2**64 - 1)),
                                ctypes.byref(p), ctypes.byref(o), float(lr), _ptr(omega_beta),
                                _ptr(conf), _ptr(mask), _ptr(kept), _ptr(workspace),
                                _nbytes(workspace), _stream(dev)), "spec_verify_update")
    return out, conf, mask, kept


class VerifyCall:
    """A verification call with its arguments marshalled once, for loops that
    verify the same buffers again and again (a serving step, a benchmark):
    calling it only sets the seed and enqueues spec_verify on the stream that
    was current at construction.  The tensors must stay alive and in place."""

    def __init__(self, target: torch.Tensor, draft: Optional[torch.Tensor],
                 draft_tokens: torch.Tensor, mode: int = MODE_LOSSLESS, *,
                 temperature: float = 1.0, fly_theta: float = 0.3, fly_window: int = 4,
                 kept_len: Optional[torch.Tensor] = None,
                 draft_stats: Optional[torch.Tensor] = None, vocab: Optional[int] = None,
                 out: Optional[VerifyResult] = None, workspace: Optional[torch.Tensor] = None,
                 boundary: bool = False):
        _need_cuda(target, "target")
        B, K1, S = target.shape
        K = K1 - 1
        V = S if vocab is None else int(vocab)
        dev = target.device
        _check_inputs(dev, B, K, S, target.dtype, draft, draft_tokens, kept_len, draft_stats,
                      workspace)
        self.L = load()
        self.params = _params(B, K, V, S, _dtype_code(target), temperature, fly_theta,
                              fly_window)
        if out is None:
            out = VerifyResult(torch.empty(B, dtype=torch.int32, device=dev),
                               torch.empty(B, K + 1, dtype=torch.int32, device=dev))
        if boundary and out.boundary is None:
            out.boundary = torch.empty(B, dtype=torch.int32, device=dev)
        out.check(B, K, dev)
        self.out = out
        self.vout = out.fields()
        need = int(self.L.spec_workspace_bytes(ctypes.byref(self.params)))
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        self._keep = (target, draft, draft_tokens, kept_len, draft_stats, workspace)
        self.args = [_ptr(target), _ptr(draft), _ptr(draft_tokens), _ptr(kept_len),
                     _ptr(draft_stats), ctypes.c_uint64(0), int(mode), ctypes.byref(self.params),
                     ctypes.byref(self.vout), _ptr(workspace), _nbytes(workspace), _stream(dev)]

    def __call__(self, seed: int = 0) -> VerifyResult:
        self.args[5] = ctypes.c_uint64(int(seed) & (2**64 - 1))
        _check(self.L.spec_verify(*self.args), "spec_verify")
        return self.out


def av_score(draft: torch.Tensor, draft_tokens: torch.Tensor, omega_beta: torch.Tensor,
             tau: float, *, temperature: float = 1.0, vocab: Optional[int] = None,
             draft_stats: Optional[torch.Tensor] = None, prefix: bool = False):
    """Adaptive-verification confidences.  Returns (conf [B,K] float,
    keep_mask [B,K] uint8, kept_len [B] int32, draft_stats buffer).
    prefix: spec_av_score_prefix, which reads each sequence's rows only up to
    its first trimmed position (conf and statistics past it are NaN)."""
    _need_cuda(draft, "draft")
    B, K, S = draft.shape
    V = S if vocab is None else int(vocab)
    dev = draft.device
    _need_cuda(omega_beta, "omega_beta", dev, torch.float32, (K + 1,))
    _need_cuda(draft_tokens, "draft_tokens", dev, torch.int32, (B, K))
    p = _params(B, K, V, S, _dtype_code(draft), temperature)
    L = load()
    conf = torch.empty(B, K, dtype=torch.float32, device=dev)
    mask = torch.empty(B, K, dtype=torch.uint8, device=dev)
    kept = torch.empty(B, dtype=torch.int32, device=dev)
    need = int(L.spec_draft_stats_bytes(B, K))
    if draft_stats is None:
        draft_stats = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    else:
        _need_cuda(draft_stats, "draft_stats", dev, nbytes=need)
    fn = L.spec_av_score_prefix if prefix else L.spec_av_score
    _check(fn(_ptr(draft), _ptr(draft_tokens), ctypes.byref(p), _ptr(omega_beta), float(tau),
              _ptr(conf), _ptr(mask), _ptr(kept), _ptr(draft_stats), _stream(dev)),
           "spec_av_score_prefix" if prefix else "spec_av_score")
    return conf, mask, kept, draft_stats


def av_score_stats(draft_stats: torch.Tensor, B: int, K: int, omega_beta: torch.Tensor,
                   tau: float):
    """Confidences and trimming from an already filled draft-statistics buffer
    (no row is read).  Returns (conf [B,K] float, keep_mask [B,K] uint8,
    kept_len [B] int32)."""
    _need_cuda(draft_stats, "draft_stats")
    dev = draft_stats.device
    _check_labels(dev, B, K, draft_stats, None, None, omega_beta)
    conf = torch.empty(B, K, dtype=torch.float32, device=dev)
    mask = torch.empty(B, K, dtype=torch.uint8, device=dev)
    kept = torch.empty(B, dtype=torch.int32, device=dev)
    _check(load().spec_av_score_stats(_ptr(draft_stats), int(B), int(K), _ptr(omega_beta),
                                      float(tau), _ptr(conf), _ptr(mask), _ptr(kept),
                                      _stream(dev)), "spec_av_score_stats")
    return conf, mask, kept


class AvStepCall:
    """One adaptive-verification step (score and trim, verify, SGD update)
    with its arguments marshalled once and its buffers allocated once: the
    buffers of one batch of draft and target logits, verified again and again
    (a serving loop that refills them in place, a benchmark).  Calling it
    enqueues the step on the stream that was current at construction;
    omega_beta is updated in place.

    With tau > 0: spec_av_score (draft rows), spec_verify on the kept drafts,
    spec_av_update.  prefix=True scores with spec_av_score_prefix instead,
    which stops reading each sequence's draft rows after its first trimmed
    position: the step's results are the same (only kept drafts are verified
    and labelled), conf past the trim point is NaN.  With tau <= 0 nothing can
    be trimmed, so spec_verify reads target and draft rows in one pass and
    exports the draft statistics, and spec_av_score_update scores from them
    and takes the SGD step in one launch: the same results with one row pass
    instead of two.

    The verification and the update are one call, spec_verify_update, whose
    last launch picks the tokens and takes the update side by side; split=True
    makes them the separate calls above instead (the same results)."""

    def __init__(self, target: torch.Tensor, draft: torch.Tensor, draft_tokens: torch.Tensor,
                 omega_beta: torch.Tensor, tau: float, lr: float, *, temperature: float = 1.0,
                 vocab: Optional[int] = None, workspace: Optional[torch.Tensor] = None,
                 boundary: bool = False, prefix: bool = False, split: bool = False):
        _need_cuda(draft, "draft")
        B, K, S = draft.shape
        V = S if vocab is None else int(vocab)
        dev = draft.device
        _need_cuda(target, "target", dev, draft.dtype, (B, K + 1, S))
        _check_inputs(dev, B, K, S, draft.dtype, None, draft_tokens, None, None, workspace)
        _need_cuda(omega_beta, "omega_beta", dev, torch.float32, (K + 1,))
        L = load()
        self.L = L
        self.conf = torch.empty(B, K, dtype=torch.float32, device=dev)
        self.mask = torch.empty(B, K, dtype=torch.uint8, device=dev)
        self.kept = torch.empty(B, dtype=torch.int32, device=dev)
        self.stats = torch.empty(max(int(L.spec_draft_stats_bytes(B, K)), 16), dtype=torch.uint8,
                                 device=dev)
        self.params = _params(B, K, V, S, _dtype_code(draft), temperature)
        self.fused = not (float(tau) > 0.0)
        st = _stream(dev)
        if self.fused:
            out = VerifyResult(torch.empty(B, dtype=torch.int32, device=dev),
                               torch.empty(B, K + 1, dtype=torch.int32, device=dev))
            out.draft_stats_out = self.stats
            self.verify = VerifyCall(target, draft, draft_tokens, temperature=temperature,
                                     vocab=vocab, workspace=workspace, out=out,
                                     boundary=boundary)
            self.score_update_args = (_ptr(self.stats), _ptr(out.accepted_len), int(B), int(K),
                                      float(lr), _ptr(omega_beta), _ptr(self.conf),
                                      _ptr(self.mask), _ptr(self.kept), st)
        else:
            self.score_fn = L.spec_av_score_prefix if prefix else L.spec_av_score
            self.score_args = (_ptr(draft), _ptr(draft_tokens), ctypes.byref(self.params),
                               _ptr(omega_beta), float(tau), _ptr(self.conf), _ptr(self.mask),
                               _ptr(self.kept), _ptr(self.stats), st)
            self.verify = VerifyCall(target, draft, draft_tokens, temperature=temperature,
                                     kept_len=self.kept, draft_stats=self.stats, vocab=vocab,
                                     workspace=workspace, boundary=boundary)
        self.update_args = (_ptr(self.stats), _ptr(self.verify.out.accepted_len),
                            _ptr(self.kept), int(B), int(K), float(lr), _ptr(omega_beta), st)
        self.split = bool(split)
        va = self.verify.args
        if self.fused:  # scores and update from the verify pass's own statistics
            self.vu_args = va[:3] + [None, None, va[5], va[7], va[8], float(lr), _ptr(omega_beta),
                                     _ptr(self.conf), _ptr(self.mask), _ptr(self.kept)] + va[9:]
        else:
            self.vu_args = va[:6] + [va[7], va[8], float(lr), _ptr(omega_beta), None, None,
                                     None] + va[9:]
        self._keep = (target, draft, draft_tokens, omega_beta)

    def __call__(self, seed: int = 0) -> VerifyResult:
        if not self.fused:
            _check(self.score_fn(*self.score_args), "spec_av_score")
        if not self.split:
            self.vu_args[5] = ctypes.c_uint64(int(seed) & (2**64 - 1))
            _check(self.L.spec_verify_update(*self.vu_args), "spec_verify_update")
            return self.verify.out
        r = self.verify(seed)
        if self.fused:
            _check(self.L.spec_av_score_update(*self.score_update_args), "spec_av_score_update")
        else:
            _check(self.L.spec_av_update(*self.update_args), "spec_av_update")
        return r


def draft_stats_view(draft_stats: torch.Tensor, B: int, K: int):
    """Named views of the draft-statistics buffer (lse2, logq2, qmax, feat)."""
    n = B * K
    raw = draft_stats[:24 * n]
    return {"lse2": raw[:8 * n].view(torch.float64), "logq2": raw[8 * n:16 * n].view(torch.float64),
            "qmax": raw[16 * n:20 * n].view(torch.float32),
            "feat": raw[20 * n:24 * n].view(torch.float32)}


def av_score_update(draft_stats: torch.Tensor, accepted_len: torch.Tensor,
                    omega_beta: torch.Tensor, lr: float, B: int, K: int):
    """For an untrimmed step scored after its verification: the confidences
    at the current coefficients (every draft kept), then one SGD step, in one
    launch.  Returns (conf [B,K] float, keep_mask [B,K] uint8, kept_len [B]
    int32); omega_beta is updated in place."""
    _need_cuda(draft_stats, "draft_stats")
    dev = draft_stats.device
    _check_labels(dev, B, K, draft_stats, accepted_len, None, omega_beta)
    conf = torch.empty(B, K, dtype=torch.float32, device=dev)
    mask = torch.empty(B, K, dtype=torch.uint8, device=dev)
    kept = torch.empty(B, dtype=torch.int32, device=dev)
    _check(load().spec_av_score_update(_ptr(draft_stats), _ptr(accepted_len), int(B), int(K),
                                       float(lr), _ptr(omega_beta), _ptr(conf), _ptr(mask),
                                       _ptr(kept), _stream(dev)), "spec_av_score_update")
    return conf, mask, kept


def av_update(draft_stats: torch.Tensor, accepted_len: torch.Tensor,
              kept_len: Optional[torch.Tensor], omega_beta: torch.Tensor, lr: float, B: int,
              K: int) -> torch.Tensor:
    """One SGD step of the estimator; omega_beta (float32 [K+1]) is updated in place."""
    _need_cuda(draft_stats, "draft_stats")
    _check_labels(draft_stats.device, B, K, draft_stats, accepted_len, kept_len, omega_beta)
    _check(load().spec_av_update(_ptr(draft_stats), _ptr(accepted_len), _ptr(kept_len), int(B),
                                 int(K), float(lr), _ptr(omega_beta),
                                 _stream(omega_beta.device)), "spec_av_update")
    return omega_beta


def row_stats(logits: torch.Tensor, *, temperature: float = 1.0, vocab: Optional[int] = None,
              lse: bool = True, entropy: bool = True, argmax: bool = True, qmax: bool = False,
              feat: bool = False) -> dict:
    """Per-row statistics of a [rows, S] logits tensor (first V columns)."""
    _need_cuda(logits, "logits")
    x = logits.reshape(-1, logits.shape[-1])
    rows, S = x.shape
    V = S if vocab is None else int(vocab)
    dev = x.device
    res = {}
    for k, want, dt in (("lse", lse, torch.float32), ("entropy", entropy, torch.float32),
                        ("argmax", argmax, torch.int32), ("qmax", qmax, torch.float32),
                        ("feat", feat, torch.float32)):
        res[k] = torch.empty(rows, dtype=dt, device=dev) if want else None
    _check(load().spec_row_stats(_ptr(x), rows, V, S, _dtype_code(x), float(temperature),
                                 _ptr(res["lse"]), _ptr(res["entropy"]), _ptr(res["argmax"]),
                                 _ptr(res["qmax"]), _ptr(res["feat"]), _stream(dev)),
           "spec_row_stats")
    return {k: v for k, v in res.items() if v is not None}


def read_probe(logits: torch.Tensor, *, row_bytes: Optional[int] = None,
               sink: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Load-only pass over the rows of a [rows, S] tensor with the row pass's
    loads and grid (a bandwidth ceiling for it); returns the XOR of each
    row's 32-bit words (the first row_bytes bytes, default all S)."""
    _need_cuda(logits, "logits")
    x = logits.reshape(-1, logits.shape[-1])
    rows, S = x.shape
    stride_b = S * x.element_size()
    rb = stride_b if row_bytes is None else int(row_bytes)
    if sink is None:
        sink = torch.empty(rows, dtype=torch.int32, device=x.device)
    else:
        _need_cuda(sink, "sink", x.device, torch.int32, (rows,))
    _check(load().spec_read_probe(_ptr(x), rows, rb, stride_b, _ptr(sink), _stream(x.device)),
           "spec_read_probe")
    return sink


def irls_state(K: int, device) -> torch.Tensor:
    """A zeroed Newton-refit state for K draft positions (float64 device tensor)."""
    n = load().spec_irls_state_bytes(int(K))
    if n == 0:
        raise SpecVerifyError("spec_irls_state_bytes: unsupported num_draft %d" % K)
    st = torch.empty(n // 8, dtype=torch.float64, device=device)
    _check(load().spec_irls_reset(_ptr(st), int(K), _stream(st.device)), "spec_irls_reset")
    return st


def irls_accumulate(state: torch.Tensor, draft_stats: torch.Tensor, accepted_len: torch.Tensor,
                    kept_len: Optional[torch.Tensor], omega_beta: torch.Tensor, B: int,
                    K: int) -> torch.Tensor:
    """Add one step's labels to the round's gradient and Hessian."""
    _need_cuda(state, "state", nbytes=load().spec_irls_state_bytes(int(K)))
    _check_labels(state.device, B, K, draft_stats, accepted_len, kept_len, omega_beta)
    _check(load().spec_irls_accumulate(_ptr(draft_stats), _ptr(accepted_len), _ptr(kept_len),
                                       int(B), int(K), _ptr(omega_beta), _ptr(state),
                                       _stream(state.device)), "spec_irls_accumulate")
    return state


def irls_solve(state: torch.Tensor, omega_beta: torch.Tensor, K: int, c_damp: float,
               flags: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Solve the round's Newton system, update omega_beta in place, zero the state."""
    _need_cuda(state, "state", nbytes=load().spec_irls_state_bytes(int(K)))
    _need_cuda(omega_beta, "omega_beta", state.device, torch.float32, (K + 1,))
    if flags is not None:
        _need_cuda(flags, "flags", state.device, torch.int32, nbytes=4)
    _check(load().spec_irls_solve(_ptr(state), int(K), float(c_damp), _ptr(omega_beta),
                                  _ptr(flags), _stream(state.device)), "spec_irls_solve")
    return omega_beta


def av_diagnostics(draft_stats: torch.Tensor, accepted_len: torch.Tensor,
                   kept_len: Optional[torch.Tensor], omega_beta: torch.Tensor, B: int, K: int,
                   nbins: int = 10, out: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """AUC, mean log-loss, ECE and label count of the estimator on one batch
    (float64 device tensor of 4)."""
    _need_cuda(draft_stats, "draft_stats")
    dev = draft_stats.device
    _check_labels(dev, B, K, draft_stats, accepted_len, kept_len, omega_beta)
    if out is None:
        out = torch.empty(4, dtype=torch.float64, device=dev)
    else:
        _need_cuda(out, "out", dev, torch.float64, (4,))
    n = load().spec_av_diagnostics_workspace_bytes(int(B), int(K), int(nbins))
    if workspace is None:
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    else:
        _need_cuda(workspace, "workspace", dev)
    _check(load().spec_av_diagnostics(_ptr(draft_stats), _ptr(accepted_len), _ptr(kept_len),
                                      int(B), int(K), _ptr(omega_beta), int(nbins), _ptr(out),
                                      _ptr(workspace), _nbytes(workspace), _stream(dev)),
           "spec_av_diagnostics")
    return out


def av_budget(conf: torch.Tensor, cost: torch.Tensor, n_requests: Optional[float] = None,
              mask: bool = True, workspace: Optional[torch.Tensor] = None) -> dict:
    """Budgeted trimming of a [B, K] confidence tensor against a float64 cost
    table of B*K+1 entries: kept_len [B], keep mask, budget and best ratio."""
    _need_cuda(conf, "conf", dtype=torch.float32)
    B, K = conf.shape
    dev = conf.device
    _need_cuda(cost, "cost", dev, torch.float64, (B * K + 1,))
    res = {"kept_len": torch.empty(B, dtype=torch.int32, device=dev),
           "mask": torch.empty(B, K, dtype=torch.uint8, device=dev) if mask else None,
           "budget": torch.empty(1, dtype=torch.int64, device=dev),
           "best_ratio": torch.empty(1, dtype=torch.float64, device=dev)}
    nr = float(B if n_requests is None else n_requests)
    if workspace is None:
        n = load().spec_av_budget_workspace_bytes(int(B), int(K))
        workspace = torch.empty(max(n, 16), dtype=torch.uint8, device=dev)
    else:
        _need_cuda(workspace, "workspace", dev)
    _check(load().spec_av_budget(_ptr(conf), int(B), int(K), _ptr(cost), nr,
                                 _ptr(res["kept_len"]), _ptr(res["mask"]), _ptr(res["budget"]),
                                 _ptr(res["best_ratio"]), _ptr(workspace), _nbytes(workspace),
                                 _stream(dev)), "spec_av_budget")
    return res


def ngram_propose(context: torch.Tensor, lengths: torch.Tensor, n_min: int, n_max: int,
                  K: int) -> dict:
    """Prompt-lookup drafts for int32 contexts [B, S] of the given lengths."""
    _need_cuda(context, "context", dtype=torch.int32)
    B, S = context.shape
    dev = context.device
    _need_cuda(lengths, "lengths", dev, torch.int32, (B,))
    res = {"draft": torch.empty(B, K, dtype=torch.int32, device=dev),
           "draft_len": torch.empty(B, dtype=torch.int32, device=dev),
           "match_pos": torch.empty(B, dtype=torch.int32, device=dev),
           "match_n": torch.empty(B, dtype=torch.int32, device=dev)}
    _check(load().spec_ngram_propose(_ptr(context), _ptr(lengths), int(B), int(S), int(n_min),
                                     int(n_max), int(K), _ptr(res["draft"]),
                                     _ptr(res["draft_len"]), _ptr(res["match_pos"]),
                                     _ptr(res["match_n"]), _stream(dev)), "spec_ngram_propose")
    return res
