"""CPU-side checks of the C ABI: the library loads, exports every function the
public header declares, and rejects bad arguments on the host before any GPU
work (so no GPU is needed for these calls)."""
import ctypes
import glob
import os
import re

import pytest
import torch

import draft_token_verification_vocab_amd as sv

# These calls hand the library fake device addresses that host-side
# validation must reject; never let them reach a real GPU.
host_only = pytest.mark.skipif(torch.cuda.is_available(),
                               reason="fake device pointers: host-only validation test")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        for m in re.finditer(r"^[A-Za-z_][\w \t\*]*?\b(spec_\w+)\s*\(", src, flags=re.M):
            names.add(m.group(1))
    return sorted(names)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(sv.lib_path()):
        from draft_token_verification_vocab_amd import build
        build.build()
    return sv.load()


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("spec_verify", "spec_av_score", "spec_av_score_stats", "spec_av_update",
              "spec_av_score_update", "spec_row_stats",
              "spec_workspace_bytes", "spec_draft_stats_bytes", "spec_status_string",
              "spec_read_probe", "spec_irls_state_bytes", "spec_irls_reset",
              "spec_irls_accumulate", "spec_irls_solve", "spec_av_diagnostics",
              "spec_av_diagnostics_workspace_bytes", "spec_av_budget",
              "spec_av_budget_workspace_bytes", "spec_ngram_propose", "spec_verify_update"):
        assert n in names


def test_every_declared_symbol_is_exported(L):
    for n in declared_functions():
        assert hasattr(L, n), n
        assert n in sv._SIGNATURES, "binding lacks a signature for %s" % n


def _params(**kw):
    base = dict(batch=4, num_draft=4, vocab=1024, dtype=1, row_stride=1024, temperature=1.0,
                fly_theta=0.3, fly_window=4, reserved=0)
    base.update(kw)
    return sv._Params(**base)


def test_workspace_query(L):
    p = _params()
    n = L.spec_workspace_bytes(ctypes.byref(p))
    assert n > 0 and n % 256 == 0
    big = _params(batch=1024, num_draft=8, vocab=128256, row_stride=128256)
    assert L.spec_workspace_bytes(ctypes.byref(big)) > n
    assert L.spec_workspace_bytes(ctypes.byref(_params(num_draft=0))) == 0
    assert L.spec_draft_stats_bytes(64, 5) == 24 * 64 * 5


@host_only
@pytest.mark.parametrize("kw,status", [
    (dict(num_draft=0), -1), (dict(num_draft=65), -2), (dict(vocab=1), -1),
    (dict(row_stride=1000), -1), (dict(row_stride=1028), -1), (dict(dtype=7), -1),
    (dict(temperature=0.0), -1), (dict(temperature=float("nan")), -1), (dict(batch=-1), -1),
    (dict(reserved=1), -1),
    # rows are addressed with 32-bit byte offsets: a row must stay below 2 GiB
    (dict(vocab=1 << 29, row_stride=1 << 29, dtype=0), -2),
    (dict(vocab=1 << 30, row_stride=1 << 30, dtype=1), -2)])
def test_verify_rejects_bad_params_on_host(L, kw, status):
    p = _params(**kw)
    out = sv._VerifyOut()
    st = L.spec_verify(ctypes.c_void_p(16), ctypes.c_void_p(16), ctypes.c_void_p(16), None, None,
                       0, 0, ctypes.byref(p), ctypes.byref(out), ctypes.c_void_p(16), 1 << 20,
                       None)
    assert st == status


@host_only
def test_verify_rejects_bad_pointers_and_modes(L):
    p = _params()
    out = sv._VerifyOut(16, 16, None, None, None, None, None, None)
    args = dict(target=16, draft=16, tokens=16)

    def call(mode=0, target=16, draft=16, tokens=16, ws=16, ws_bytes=1 << 30, o=out):
        return L.spec_verify(ctypes.c_void_p(target), ctypes.c_void_p(draft),
                             ctypes.c_void_p(tokens), None, None, 0, mode, ctypes.byref(p),
                             ctypes.byref(o) if o is not None else None, ctypes.c_void_p(ws),
                             ws_bytes, None)
    assert call(mode=5) == -1
    assert call(target=8) == -1                # misaligned logits
    assert call(draft=0) == -1                 # lossless needs draft logits
    assert call(tokens=0) == -1
    assert call(ws=0) == -3                    # no workspace
    assert call(ws_bytes=16) == -3             # workspace too small
    assert call(o=None) == -1
    bad = sv._VerifyOut(0, 16, None, None, None, None, None, None)
    assert call(o=bad) == -1
    fly = _params(fly_window=-1)
    assert L.spec_verify(ctypes.c_void_p(16), None, ctypes.c_void_p(16), None, None, 0, 1,
                         ctypes.byref(fly), ctypes.byref(out), ctypes.c_void_p(16), 1 << 30,
                         None) == -1


@host_only
def test_empty_inputs_are_noops_on_host(L):
    p = _params(batch=0)
    out = sv._VerifyOut()
    assert L.spec_verify(None, None, None, None, None, 0, 0, ctypes.byref(p), ctypes.byref(out),
                         None, 0, None) == 0
    assert L.spec_row_stats(None, 0, 1024, 1024, 1, 1.0, None, None, None, None, None,
                            None) == 0
    assert L.spec_av_update(None, None, None, 0, 4, 0.05, None, None) == 0


@host_only
def test_verify_update_validates_on_host(L):
    p = _params()
    out = sv._VerifyOut(16, 16, None, None, None, None, None, None)
    v16 = ctypes.c_void_p(16)

    def call(kept=None, stats=None, lr=0.05, omega=16, conf=None, pp=p, target=16):
        return L.spec_verify_update(ctypes.c_void_p(target), v16, v16, kept, stats, 0,
                                    ctypes.byref(pp), ctypes.byref(out), lr,
                                    ctypes.c_void_p(omega) if omega else None, conf, None, None,
                                    v16, 1 << 30, None)
    assert call(lr=float("nan")) == -1
    assert call(lr=float("inf")) == -1
    assert call(omega=0) == -1                          # no coefficients to update
    assert call(conf=v16, kept=v16) == -1               # scores need an untrimmed step
    assert call(conf=v16, stats=v16) == -1
    assert call(target=8) == -1                         # spec_verify's own checks
    assert call(pp=_params(num_draft=65)) == -2
    assert call(pp=_params(batch=0), omega=0) == 0      # empty batch: nothing to do


@host_only
def test_other_entry_points_validate(L):
    p = _params()
    assert L.spec_av_score(None, ctypes.c_void_p(16), ctypes.byref(p), ctypes.c_void_p(16), 0.2,
                           None, None, None, ctypes.c_void_p(16), None) == -1
    assert L.spec_av_score(ctypes.c_void_p(16), ctypes.c_void_p(16), ctypes.byref(p),
                           ctypes.c_void_p(16), float("nan"), None, None, None,
                           ctypes.c_void_p(16), None) == -1
    assert L.spec_av_update(ctypes.c_void_p(16), None, None, 4, 4, 0.05, ctypes.c_void_p(16),
                            None) == -1
    assert L.spec_av_update(ctypes.c_void_p(16), ctypes.c_void_p(16), None, 4, 65, 0.05,
                            ctypes.c_void_p(16), None) == -2
    assert L.spec_row_stats(ctypes.c_void_p(16), 4, 1024, 1020, 1, 1.0, None, None, None, None,
                            None, None) == -1
    assert L.spec_row_stats(ctypes.c_void_p(16), -1, 1024, 1024, 1, 1.0, None, None, None, None,
                            None, None) == -1
    assert L.spec_av_score_stats(None, 4, 4, ctypes.c_void_p(16), 0.2, None, None, None,
                                 None) == -1
    assert L.spec_av_score_stats(ctypes.c_void_p(16), 4, 65, ctypes.c_void_p(16), 0.2, None,
                                 None, None, None) == -2
    assert L.spec_av_score_stats(ctypes.c_void_p(16), 0, 4, None, 0.2, None, None, None,
                                 None) == 0
    assert L.spec_av_score_update(None, ctypes.c_void_p(16), 4, 4, 0.05, ctypes.c_void_p(16),
                                  None, None, None, None) == -1
    assert L.spec_av_score_update(ctypes.c_void_p(16), None, 4, 4, 0.05, ctypes.c_void_p(16),
                                  None, None, None, None) == -1
    assert L.spec_av_score_update(ctypes.c_void_p(16), ctypes.c_void_p(16), 4, 65, 0.05,
                                  ctypes.c_void_p(16), None, None, None, None) == -2
    assert L.spec_av_score_update(ctypes.c_void_p(16), ctypes.c_void_p(16), 4, 4,
                                  float("nan"), ctypes.c_void_p(16), None, None, None,
                                  None) == -1
    assert L.spec_av_score_update(None, None, 0, 4, 0.05, None, None, None, None, None) == 0
    assert L.spec_read_probe(ctypes.c_void_p(16), 4, 24, 32, ctypes.c_void_p(16), None) == -1
    assert L.spec_read_probe(ctypes.c_void_p(16), 4, 48, 32, ctypes.c_void_p(16), None) == -1
    assert L.spec_read_probe(ctypes.c_void_p(16), 4, 32, 32, None, None) == -1
    assert L.spec_read_probe(None, 0, 32, 32, None, None) == 0
    assert L.spec_read_probe(ctypes.c_void_p(16), 4, 1 << 31, 1 << 31, ctypes.c_void_p(16),
                             None) == -2
    for s in (0, -1, -2, -3, -4, 99):
        assert isinstance(L.spec_status_string(s), bytes)


def test_next_rows_sizes(L):
    assert L.spec_irls_state_bytes(8) == 8 * (4 * 8 + 3)
    assert L.spec_irls_state_bytes(0) == 0 and L.spec_irls_state_bytes(65) == 0
    assert L.spec_av_diagnostics_workspace_bytes(1024, 8, 10) > 8 * 8192
    assert L.spec_av_diagnostics_workspace_bytes(1024, 8, 65) == 0
    assert L.spec_av_diagnostics_workspace_bytes(8192, 16, 10) == 0  # > 65536 labels
    assert L.spec_av_budget_workspace_bytes(1024, 8) >= 8192 * (2 * 32 + 8)
    assert L.spec_av_budget_workspace_bytes(8193, 8) == 0


@host_only
def test_next_rows_validate_on_host(L):
    P = ctypes.c_void_p
    a = P(16)
    assert L.spec_irls_reset(a, 0, None) == -1
    assert L.spec_irls_reset(a, 65, None) == -2
    assert L.spec_irls_reset(P(12), 4, None) == -1              # not 8-byte aligned
    assert L.spec_irls_accumulate(a, a, None, 4, 65, a, a, None) == -2
    assert L.spec_irls_accumulate(a, None, None, 4, 4, a, a, None) == -1
    assert L.spec_irls_accumulate(None, None, None, 0, 4, None, None, None) == 0
    assert L.spec_irls_solve(a, 4, -1.0, a, None, None) == -1
    assert L.spec_irls_solve(a, 4, float("inf"), a, None, None) == -1
    assert L.spec_irls_solve(a, 4, 1.0, None, None, None) == -1
    assert L.spec_av_diagnostics(a, a, None, 4, 4, a, 0, a, a, 1 << 20, None) == -1
    assert L.spec_av_diagnostics(a, a, None, 4, 4, a, 65, a, a, 1 << 20, None) == -2
    assert L.spec_av_diagnostics(a, a, None, 4, 4, a, 10, a, a, 16, None) == -3
    assert L.spec_av_diagnostics(a, a, None, 4, 4, a, 10, a, None, 1 << 20, None) == -3
    big = 1 << 30
    assert L.spec_av_budget(a, 8193, 8, a, 1.0, a, None, a, None, a, big, None) == -2
    assert L.spec_av_budget(a, 4, 4, P(12), 1.0, a, None, a, None, a, big, None) == -1
    assert L.spec_av_budget(a, 4, 4, a, float("nan"), a, None, a, None, a, big, None) == -1
    assert L.spec_av_budget(a, 0, 4, a, 1.0, a, None, a, None, a, big, None) == -1
    assert L.spec_av_budget(a, 4, 4, a, 1.0, a, None, a, None, a, 16, None) == -3
    assert L.spec_av_budget(a, 4, 4, a, 1.0, a, None, a, None, None, big, None) == -3
    assert L.spec_ngram_propose(a, a, 4, 100, 0, 3, 4, a, a, None, None, None) == -1
    assert L.spec_ngram_propose(a, a, 4, 100, 3, 2, 4, a, a, None, None, None) == -1
    assert L.spec_ngram_propose(a, a, 4, 100, 1, 33, 4, a, a, None, None, None) == -2
    assert L.spec_ngram_propose(a, a, 4, 100, 1, 3, 65, a, a, None, None, None) == -2
    assert L.spec_ngram_propose(a, None, 4, 100, 1, 3, 4, a, a, None, None, None) == -1
    assert L.spec_ngram_propose(None, None, 0, 100, 1, 3, 4, None, None, None, None, None) == 0
