#!/usr/bin/env python3
"""Benchmark of batched speculative-decoding verification on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step is one verification call over one batch of synthetic logits that
already sits in HBM.  The headline workload is FLy loose-greedy verification
of B=256 sequences x K=8 drafts over V=128256 bfloat16 logits (2304 target
rows, 591 MB per call); two input sets alternate so that no call finds its
rows in the 256 MB last-level cache.  Prints one JSON line.

Besides the headline it reports:
  roofline      the streaming row pass (the dominant kernel), launched back to
                back with HIP events on its stream: algorithmic bytes / mean
                launch time against the 8 TB/s HBM peak; `traffic` comes from
                rocprofv3 FETCH_SIZE / WRITE_SIZE counters recorded under
                profiles/ for the same kernel source, else null;
  read_ceiling  the row pass's load-only twin (same grid, loads and shape) on
                the same rows: the bandwidth this access pattern reaches on the
                machine, next to the nominal 8 TB/s;
  cpu_baseline  the CPU oracle timed on a bounded sample of the same workload;
  secondary     the other verification workloads (lossless with adaptive
                verification, lossless at T=0.7 on V=152064, the full
                adaptive-verification pipeline over 20 steps with a freshly
                generated input set per step, lossless at the headline
                shape), each timed the same way, and the estimator's Newton
                refit, diagnostics, budgeted trimming and prompt lookup.
Every verification line also carries `boundary`: the sequences the library
logged as near-ties on its last call per input set, against the verified
rows (kept length + 1 per sequence).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified logits rows/s and achieved HBM GB/s (% peak), V=128256 bf16, 1 GPU"
HBM_PEAK_GBPS = 8000.0
# the row pass's kernel, its launch shape and the helpers it compiles from
ROW_PASS_SOURCES = ["draft_token_verification_vocab_amd/csrc/sv_rowstats.hpp",
                    "draft_token_verification_vocab_amd/csrc/sv_common.hpp",
                    "draft_token_verification_vocab_amd/csrc/sv_philox.hpp"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "row_pass_fly_b256_k8_v128256_bf16.traffic.json")
VALU_FILE = os.path.join(ROOT, "profiles", "row_pass_valu_fly_b256_k8_v128256_bf16.json")


def row_pass_source_hash() -> str:
    """Hash of the row pass's sources with comments and blank space removed
    (an edit to a comment does not change the kernel)."""
    import re
    h = hashlib.sha256()
    for p in ROW_PASS_SOURCES:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"//[^\n]*", "", text)
        text = re.sub(r"\s+", " ", text)
        h.update(text.encode())
    return h.hexdigest()[:16]


# The secondary workloads, in the order run_secondary runs them.
SECONDARY_NAMES = ("lossless_b256_k8_v128256_bf16", "lossless_b1_k4_v32000_f32",
                   "lossless_av_b64_k5_v128256_bf16", "lossless_t0.7_b512_k4_v152064_bf16",
                   "av_pipeline_b1024_k8_v128256_bf16_x20", "next_rows")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # Back-to-back load first slows the clocks for ~10-20 ms and then settles;
    # the defaults time the steady state after that transient (~0.1 s of work).
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--calib-copy", action="store_true",
                    help="first run a plain 1 GiB device copy three times (a known-size "
                         "kernel for calibrating hardware byte counters)")
    ap.add_argument("--only", choices=SECONDARY_NAMES,
                    help="run only this secondary workload, --steps timed steps after "
                         "--warmup untimed ones, and print its line (for per-workload "
                         "kernel traces); no headline, roofline or CPU baseline")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the verification hot path runs on a single MI355X "
              "(multi-GPU sharding is a design note, not built); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import draft_token_verification_vocab_amd as sv
    from draft_token_verification_vocab_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sv.load()
    if args.calib_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.only:
        out = run_secondary(sv, W, dev, torch.cuda.current_stream(dev), args, only=args.only)
        print(json.dumps({"workload": args.only, "steps": args.steps, "warmup": args.warmup,
                          **out[args.only]}), flush=True)
        return

    # ------------------------------------------------------------------ headline
    cfg = W.CONFIGS[2]
    B, K, V = cfg["B"], cfg["K"], cfg["V"]
    log("generating two input sets of %s on the GPU" % cfg["name"])
    sets = [W.make(2, device=dev, step=s) for s in range(2)]
    rows = B * (K + 1)
    row_bytes = V * 2
    bytes_per_step = rows * row_bytes
    ws = torch.empty(sv.workspace_bytes(B, K, V), dtype=torch.uint8, device=dev)
    outs = [sv.VerifyResult(torch.empty(B, dtype=torch.int32, device=dev),
                            torch.empty(B, K + 1, dtype=torch.int32, device=dev),
                            boundary=torch.empty(B, dtype=torch.int32, device=dev))
            for _ in sets]

    def step(i):
        b = sets[i % 2]
        sv.verify(b.target, None, b.tokens, seed=0, mode=sv.MODE_FLY, fly_theta=cfg["theta"],
                  fly_window=cfg["window"], workspace=ws, out=outs[i % 2])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(args.steps):
        step(i)
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    rows_per_s = rows / (ms * 1e-3)
    gbps = bytes_per_step / (ms * 1e-3) / 1e9
    acc_mean = float(torch.cat([o.accepted_len for o in outs]).float().mean().item())
    headline_boundary = _boundary(outs, [rows] * len(outs))
    log("headline: %.1f us/step, %.3g rows/s, %.0f GB/s" % (ms * 1e3, rows_per_s, gbps))

    # ------------------------------------------------------------- roofline
    # The same row-pass kernel and launch shape as the headline's first launch
    # (target rows, entropy + argmax), timed launch by launch on its stream.
    flat = [s.target.view(rows, V) for s in sets]
    st_out = {k: torch.empty(rows, dtype=dt, device=dev) for k, dt in
              (("lse", torch.float32), ("entropy", torch.float32), ("argmax", torch.int32))}
    L = sv.load()
    import ctypes

    def row_launch(i):
        x = flat[i % 2]
        st = L.spec_row_stats(ctypes.c_void_p(x.data_ptr()), rows, V, V, sv.DTYPE_BF16, 1.0,
                              ctypes.c_void_p(st_out["lse"].data_ptr()),
                              ctypes.c_void_p(st_out["entropy"].data_ptr()),
                              ctypes.c_void_p(st_out["argmax"].data_ptr()), None, None,
                              ctypes.c_void_p(stream.cuda_stream))
        assert st == 0

    for i in range(args.warmup):
        row_launch(i)
    n_k = max(args.steps, 20)
    k0 = torch.cuda.Event(enable_timing=True)
    k1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    k0.record(stream)
    for i in range(n_k):
        row_launch(i)
    k1.record(stream)
    torch.cuda.synchronize()
    kms = k0.elapsed_time(k1) / n_k  # back-to-back launches on the launch stream
    achieved = bytes_per_step / (kms * 1e-3) / 1e9

    # Same-shape ceiling: the load-only twin of the row pass (same grid, loads
    # and workgroup shape) over the same rows, timed the same way.
    sink = torch.empty(rows, dtype=torch.int32, device=dev)
    for i in range(args.warmup):
        sv.read_probe(flat[i % 2], sink=sink)
    pev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    pev[0].record(stream)
    for i in range(n_k):
        sv.read_probe(flat[i % 2], sink=sink)
    pev[1].record(stream)
    torch.cuda.synchronize()
    pms = pev[0].elapsed_time(pev[1]) / n_k
    ceiling = {"kernel": "read_probe_kernel<768,2> (load-only twin of the row pass)",
               "kernel_us": round(pms * 1e3, 2),
               "gbps": round(bytes_per_step / (pms * 1e-3) / 1e9, 1),
               "row_pass_frac_of_ceiling": round(pms / kms, 4)}
    log("read ceiling: %.1f us/launch, %.0f GB/s" % (pms * 1e3, ceiling["gbps"]))

    # Spread: the headline step and the row pass again, with an event between
    # consecutive calls.  Each event leaves the queue idle for a few us before
    # the next kernel, so these figures sit above the back-to-back means.
    step_us = _evented(step, args.steps, stream, torch)
    launch_us = _evented(row_launch, n_k, stream, torch)
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("source_hash") == row_pass_source_hash():
            traffic = tr.get("bytes_per_launch")
    valu = None  # VALU counters recorded for the same kernel source
    if os.path.exists(VALU_FILE):
        with open(VALU_FILE) as f:
            va = json.load(f)
        if va.get("source_hash") == row_pass_source_hash():
            valu = {k: va[k] for k in ("valu_insts_per_logit", "valu_busy_frac")}
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                "kernel": "row_stats_kernel<bf16,768,2,entropy>", "kernel_us": round(kms * 1e3, 2),
                "algorithmic_bytes_per_launch": bytes_per_step,
                "evented_launch_us_p10_p50_p90": _pcts(launch_us),
                "valu": valu,
                "source_hash": row_pass_source_hash()}
    log("row pass: %.1f us/launch, %.0f GB/s (%.1f%% of peak)" % (kms * 1e3, achieved,
                                                                  100 * achieved / HBM_PEAK_GBPS))

    # ---------------------------------------------------------- secondary
    secondary = {}
    if not args.no_secondary:
        secondary = run_secondary(sv, W, dev, stream, args)

    # -------------------------------------------------------- cpu baseline
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(sets[0], cfg, args.cpu_seconds)
        if not args.no_secondary:
            log("timing the oracle beside the other workloads")
            cpu["beside"] = oracle_beside(W, cpu["cores"], args.cpu_seconds / 12)

    res = {
        "metric": METRIC, "value": round(rows_per_s, 1), "unit": "rows/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": cfg["name"], "mode": "fly", "B": B, "K": K, "V": V,
                   "logits": "bf16", "theta": cfg["theta"], "window": cfg["window"],
                   "rows_per_step": rows, "bytes_per_step": bytes_per_step,
                   "input_sets": 2},
        "gbps": round(gbps, 1), "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
        "evented_step_us_p10_p50_p90": _pcts(step_us),
        "mean_accepted_len": round(acc_mean, 4),
        "boundary": headline_boundary,
        "roofline": roofline, "read_ceiling": ceiling, "cpu_baseline": cpu,
        "secondary": secondary,
    }
    print(json.dumps(res), flush=True)


def _pcts(xs):
    """p10, p50, p90 of a sorted list (nearest rank)."""
    n = len(xs)
    return [round(xs[min(n - 1, int(q * n))], 2) for q in (0.1, 0.5, 0.9)]


def _evented(fn, n, stream, torch):
    """Sorted per-call durations (us) of n calls with an event between each."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(n):
        fn(i)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    return sorted(ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(n))


def _timeit(fn, n, warm, stream, torch):
    for i in range(warm):
        fn(i)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(n):
        fn(i)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n


def run_secondary(sv, W, dev, stream, args, only=None):
    """Every secondary workload, or only the one named (then timed over
    --steps steps after --warmup)."""
    import torch
    out = {}
    if only is None:
        n, warm = max(5, min(args.steps, 20)), 2
    else:
        n, warm = args.steps, args.warmup

    def want(name):
        return only is None or only == name

    # lossless verification at the headline shape (target + draft rows)
    if want("lossless_b256_k8_v128256_bf16"):
        b0 = W.gaussian(256, 8, 128256, "bf16", 1.0, seed=77, token_seed=0, device=dev)
        b1 = W.gaussian(256, 8, 128256, "bf16", 1.0, seed=78, token_seed=1, device=dev)
        bs = [b0, b1]
        ws = torch.empty(sv.workspace_bytes(256, 8, 128256), dtype=torch.uint8, device=dev)
        calls = [sv.VerifyCall(b.target, b.draft, b.tokens, workspace=ws, boundary=True)
                 for b in bs]
        res = [c.out for c in calls]

        def f(i):
            calls[i % 2](i)
        ms = _timeit(f, n, warm, stream, torch)
        rows = 256 * 17
        byt = rows * 128256 * 2
        out["lossless_b256_k8_v128256_bf16"] = _line(ms, rows, byt, res, [256 * 9] * 2, n)
        del bs, b0, b1

    # lossless, B=1 K=4 V=32000 float32 (latency: a handful of rows)
    c = W.CONFIGS[0]
    if want(c["name"]):
        sets = [W.make(0, device=dev, step=s) for s in range(4)]
        ws0 = torch.empty(sv.workspace_bytes(1, c["K"], c["V"], dtype=sv.DTYPE_F32),
                          dtype=torch.uint8, device=dev)
        calls = [sv.VerifyCall(b.target, b.draft, b.tokens, workspace=ws0, boundary=True)
                 for b in sets]
        res = [cl.out for cl in calls]

        def f0(i):
            calls[i % 4](i)
        # a step of a few microseconds: ten times the steps (when not --only),
        # so that the queue is full and the first calls' launch cost is amortised
        n0 = n if only else 10 * n
        ms = _timeit(f0, n0, warm if only else 10 * warm, stream, torch)
        rows = 2 * c["K"] + 1
        out[c["name"]] = _line(ms, rows, rows * c["V"] * 4, res, [c["K"] + 1] * 4, n0)
        del sets

    # lossless + AV score + one SGD step, B=64 K=5
    c = W.CONFIGS[1]
    if want(c["name"]):
        sets = [W.make(1, device=dev, step=s) for s in range(4)]
        K = c["K"]
        ob = torch.tensor(W.av_init(1), dtype=torch.float32, device=dev)
        ws1 = torch.empty(sv.workspace_bytes(64, K, c["V"]), dtype=torch.uint8, device=dev)
        calls = [sv.AvStepCall(b.target, b.draft, b.tokens, ob, c["av"]["tau"], c["av"]["lr"],
                               workspace=ws1, boundary=True) for b in sets]
        res = [cl.verify.out for cl in calls]

        def f1(i):
            calls[i % 4](0)
        n1 = n if only else 5 * n
        ms = _timeit(f1, n1, warm if only else 5 * warm, stream, torch)
        rows = 64 * (2 * K + 1)
        out[c["name"]] = _line(ms, rows, rows * c["V"] * 2, res, [64 * (K + 1)] * 4, n1)
        del sets

    # lossless at T = 0.7 on V = 152064, B = 512 K = 4
    c = W.CONFIGS[3]
    if want(c["name"]):
        sets = [W.make(3, device=dev, step=s) for s in range(2)]
        ws3 = torch.empty(sv.workspace_bytes(512, 4, c["V"], temperature=0.7),
                          dtype=torch.uint8, device=dev)
        calls = [sv.VerifyCall(b.target, b.draft, b.tokens, temperature=0.7, workspace=ws3,
                               boundary=True) for b in sets]
        res = [cl.out for cl in calls]

        def f3(i):
            calls[i % 2](0)
        ms = _timeit(f3, n, warm, stream, torch)
        rows = 512 * 9
        out[c["name"]] = _line(ms, rows, rows * c["V"] * 2, res, [512 * 5] * 2, n)
        del sets

    # full AV pipeline (score, trimmed verify, update), B=1024 K=8: 20 steps,
    # each on its own freshly generated input set (all 20 resident in HBM,
    # about 89 GB), with the parameters carried from step to step
    c = W.CONFIGS[4]
    if want(c["name"]):
        nsets = c["steps"]
        log("generating %d input sets of %s on the GPU" % (nsets, c["name"]))
        sets = [W.make(4, device=dev, step=s) for s in range(nsets)]
        K = c["K"]
        ob = torch.tensor(W.av_init(4), dtype=torch.float32, device=dev)
        ws4 = torch.empty(sv.workspace_bytes(1024, K, c["V"]), dtype=torch.uint8, device=dev)
        # scoring reads each sequence's draft rows up to its first trimmed
        # position (the rows after it are neither verified nor labelled)
        calls = [sv.AvStepCall(b.target, b.draft, b.tokens, ob, c["av"]["tau"], c["av"]["lr"],
                               workspace=ws4, boundary=True, prefix=True) for b in sets]
        res = [cl.verify.out for cl in calls]

        ran = set()

        def f4(i):
            ran.add(i % nsets)
            calls[i % nsets](i % nsets)
        nsteps = nsets if only is None else n
        ms = _timeit(f4, nsteps, warm, stream, torch)
        # the last step on each input set that ran: its kept lengths; rows
        # read are the draft rows up to each trim point and the target rows
        # 0..kept
        kept_all = torch.stack([calls[i].kept for i in sorted(ran)])
        verified = [int((k + 1).sum().item()) for k in kept_all]
        drafts_read = [int(torch.clamp(k + 1, max=K).sum().item()) for k in kept_all]
        rows = int(round((sum(verified) + sum(drafts_read)) / len(ran)))
        line = _line(ms, rows, rows * c["V"] * 2, [res[i] for i in sorted(ran)], verified,
                     nsteps)
        line["draft_rows_read_per_step"] = round(sum(drafts_read) / len(ran), 1)
        line["draft_rows_per_step"] = 1024 * K
        line["input_sets"] = len(ran)
        line["mean_kept_len"] = round(float(kept_all.float().mean().item()), 4)
        line["kept_len_hist"] = torch.bincount(kept_all.flatten().long(),
                                               minlength=K + 1).tolist()
        line["omega_beta_after"] = [round(v, 5) for v in ob.tolist()]
        out[c["name"]] = line
        del sets, calls, res
    torch.cuda.synchronize()
    if want("next_rows"):
        out["next_rows"] = run_next_rows(sv, W, dev, stream, args)
    return out


def run_next_rows(sv, W, dev, stream, args):
    """The estimator refit, diagnostics, budgeted trimming and prompt lookup
    at the adaptive-verification workload's shape (B=1024, K=8), each call
    timed back to back."""
    import numpy as np
    import torch
    out = {}
    n = max(10, min(args.steps, 50))
    B, K = 1024, 8
    g = torch.Generator(device="cpu").manual_seed(4242)
    feat = (torch.randn(B, K, generator=g) * 1.3 - 1.2).to(dev)
    ds = torch.zeros(sv.draft_stats_bytes(B, K), dtype=torch.uint8, device=dev)
    sv.draft_stats_view(ds, B, K)["feat"].copy_(feat.view(-1))
    kept = torch.randint(0, K + 1, (B,), generator=g, dtype=torch.int32).to(dev)
    acc = torch.minimum(torch.randint(0, K + 1, (B,), generator=g, dtype=torch.int32).to(dev),
                        kept)
    ob = torch.tensor(W.av_init(4), dtype=torch.float32, device=dev)
    st = sv.irls_state(K, dev)

    ms = _timeit(lambda i: sv.irls_accumulate(st, ds, acc, kept, ob, B, K), n, 3, stream, torch)
    out["irls_accumulate_b1024_k8"] = {"us_per_call": round(ms * 1e3, 2)}
    ob2 = ob.clone()
    ms = _timeit(lambda i: sv.irls_solve(st, ob2, K, 10.0), n, 3, stream, torch)
    out["irls_solve_k8"] = {"us_per_call": round(ms * 1e3, 2)}
    ms = _timeit(lambda i: sv.av_update(ds, acc, kept, ob2, 0.05, B, K), n, 3, stream, torch)
    out["sgd_update_b1024_k8"] = {"us_per_call": round(ms * 1e3, 2)}

    dout = torch.empty(4, dtype=torch.float64, device=dev)
    dws = torch.empty(sv.load().spec_av_diagnostics_workspace_bytes(B, K, 10), dtype=torch.uint8,
                      device=dev)
    ms = _timeit(lambda i: sv.av_diagnostics(ds, acc, kept, ob, B, K, 10, out=dout,
                                             workspace=dws), n, 3, stream, torch)
    out["diagnostics_b1024_k8"] = {"us_per_call": round(ms * 1e3, 2),
                                   "labels": int(dout[3].item())}

    for Bb in (1024, 2048):
        conf = torch.rand(Bb, K, generator=g).to(dev) * 0.98 + 0.02
        cost = torch.from_numpy(W.budget_costs(Bb, K)).to(dev)
        bws = torch.empty(sv.load().spec_av_budget_workspace_bytes(Bb, K), dtype=torch.uint8,
                          device=dev)
        res = {}

        def fb(i):
            res["r"] = sv.av_budget(conf, cost, workspace=bws)
        ms = _timeit(fb, n, 3, stream, torch)
        out["budget_b%d_k8" % Bb] = {"us_per_call": round(ms * 1e3, 2),
                                     "budget": int(res["r"]["budget"].item()),
                                     "drafts": Bb * K}

    ctx, lens = W.ngram_contexts(256, 8192, 128256, seed=7, device=dev)
    res = {}

    def fn(i):
        res["r"] = sv.ngram_propose(ctx, lens, 2, 4, 8)
    ms = _timeit(fn, n, 3, stream, torch)
    ctx_bytes = int(lens.sum().item()) * 4
    out["ngram_b256_s8192_n2to4_k8"] = {
        "us_per_call": round(ms * 1e3, 2), "context_bytes": ctx_bytes,
        "gbps_context": round(ctx_bytes / (ms * 1e-3) / 1e9, 1),
        "with_draft": int((res["r"]["draft_len"] > 0).sum().item())}
    torch.cuda.synchronize()
    return out


def _line(ms, rows, byt, res, verified_rows, steps):
    import torch
    acc = torch.cat([r.accepted_len for r in res if r is not None]).float().mean().item()
    return {"us_per_step": round(ms * 1e3, 2), "timed_steps": steps, "rows_per_step": rows,
            "rows_per_s": round(rows / (ms * 1e-3), 1), "gbps": round(byt / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(byt / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "mean_accepted_len": round(acc, 4),
            "boundary": _boundary(res, verified_rows)}


def _boundary(res, verified_rows):
    """The library's boundary-case log over the last call on each input set:
    sequences flagged, sequences, verified target rows (kept length + 1 per
    sequence) and the flagged share of those rows."""
    flagged = sum(int((r.boundary != 0).sum().item()) for r in res)
    seqs = sum(int(r.boundary.numel()) for r in res)
    rows = int(sum(verified_rows))
    return {"flagged": flagged, "sequences": seqs, "verified_rows": rows,
            "frac_of_rows": flagged / max(rows, 1)}


def cpu_baseline(batch, cfg, budget_s):
    """The CPU oracle (never tuned) on a bounded sample of the headline
    workload: the first n sequences, grown (and then repeated) until about
    budget_s seconds of work."""
    import torch
    from oracle import ref
    threads = ref.default_threads()
    tgt = batch.target.cpu().view(torch.int16).numpy().view("uint16")
    tok = batch.tokens.cpu().numpy()
    Btot = batch.target.shape[0]
    n = 4
    while True:  # grow the sample up to the whole batch
        t = time.perf_counter()
        ref.verify(tgt[:n], None, tok[:n], 0, ref.MODE_FLY, theta=cfg["theta"],
                   window=cfg["window"], nthreads=threads)
        dt = time.perf_counter() - t
        if dt >= budget_s or n >= Btot:
            break
        n = min(Btot, max(n * 2, int(n * budget_s / max(dt, 1e-3) * 0.9)))
    reps, total = 1, dt
    while total < budget_s:  # repeat whole passes until the budget is spent
        t = time.perf_counter()
        ref.verify(tgt[:n], None, tok[:n], 0, ref.MODE_FLY, theta=cfg["theta"],
                   window=cfg["window"], nthreads=threads)
        total += time.perf_counter() - t
        reps += 1
    rows = n * (cfg["K"] + 1)
    # one thread on a smaller sample, for scale
    n1 = max(1, min(Btot, n // max(threads, 1)))
    t = time.perf_counter()
    ref.verify(tgt[:n1], None, tok[:n1], 0, ref.MODE_FLY, theta=cfg["theta"],
               window=cfg["window"], nthreads=1)
    dt1 = time.perf_counter() - t
    row_bytes = batch.V * 2
    return {"value": round(rows * reps / total, 1), "unit": "rows/s", "cores": threads,
            "kind": "oracle",
            "sample": "%d of %d sequences (%d target rows) of %s, FLy mode, %d pass(es), %.1f s"
                      % (n, Btot, rows, cfg["name"], reps, total),
            "gbps": round(rows * reps * row_bytes / total / 1e9, 3),
            "single_thread_rows_per_s": round(n1 * (cfg["K"] + 1) / dt1, 1),
            "host_cpu": _cpu_model(), "host_logical_cpus": os.cpu_count()}


def oracle_beside(W, threads, budget_s):
    """The oracle (as it stands) timed beside the other figures of this line:
    one step of each secondary workload on a sample of its sequences
    (generated on the host with the same recipe), scaled to the whole batch,
    and the estimator calls of `secondary.next_rows` at their own shapes.
    Each is repeated for about budget_s seconds."""
    import numpy as np
    import torch
    from oracle import ref

    def host(x):  # bfloat16 logits go to the oracle as their bit patterns
        x = x.contiguous()
        return x.view(torch.int16).numpy().view("uint16") if x.dtype == torch.bfloat16 \
            else x.numpy()

    def step_seconds(make_batch, run, B):
        # at most 32 sequences (generating more on the host would cost more
        # than timing them), repeated until budget_s; seconds per run
        n = min(B, 32)
        b = make_batch(n)
        reps, t0 = 0, time.perf_counter()
        while True:
            run(b)
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= budget_s:
                return n, dt / reps

    def lossless(b):
        return ref.verify(host(b.target), host(b.draft), b.tokens.numpy(), 0,
                          temperature=b.temperature, V=b.V, nthreads=threads)

    def av_step(cfg):
        a = W.CONFIGS[cfg]["av"]
        ob = np.asarray(W.av_init(cfg), dtype=np.float64)

        def run(b):
            Bn, K = b.tokens.shape
            d = host(b.draft)
            st = ref.rows_stats(d.reshape(Bn * K, -1), temperature=b.temperature, V=b.V,
                                nthreads=threads)
            feat = st["feat"].reshape(Bn, K)
            _, _, kept, _ = ref.av_score(feat, ob, a["tau"])
            o = ref.verify(host(b.target), d, b.tokens.numpy(), 0, temperature=b.temperature,
                           V=b.V, kept_len=kept, nthreads=threads)
            ref.av_update(feat, o["accepted_len"], kept, ob, a["lr"])
        return run

    out = {}
    cases = [("lossless_b256_k8_v128256_bf16", 256,
              lambda n: W.gaussian(n, 8, 128256, "bf16", 1.0, seed=77, token_seed=0), lossless)]
    for ci, run in ((0, lossless), (1, av_step(1)), (3, lossless), (4, av_step(4))):
        c = W.CONFIGS[ci]
        cases.append((c["name"], c["B"], lambda n, ci=ci: W.make(ci, B=n), run))
    for name, B, make_batch, run in cases:
        n, dt = step_seconds(make_batch, run, B)
        out[name] = {"sample_sequences": n, "batch_sequences": B,
                     "oracle_us_per_step": round(dt * B / n * 1e6, 1)}

    # the estimator calls at the shapes bench.py times them on the GPU
    B, K = 1024, 8
    rng = np.random.default_rng(4242)
    feat = rng.normal(-1.2, 1.3, (B, K))
    kept = rng.integers(0, K + 1, B).astype(np.int32)
    acc = np.minimum(rng.integers(0, K + 1, B), kept).astype(np.int32)
    ob = np.asarray(W.av_init(4), dtype=np.float64)

    def per_call(fn):
        reps, t0 = 0, time.perf_counter()
        while True:
            fn()
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= budget_s / 4 or reps >= 1000:
                return round(dt / reps * 1e6, 1)
    st = ref.IrlsState(K)
    calls = {"irls_accumulate_b1024_k8": lambda: ref.irls_accumulate(st, feat, acc, kept, ob),
             "irls_solve_k8": lambda: ref.irls_solve(st, ob, 10.0),
             "sgd_update_b1024_k8": lambda: ref.av_update(feat, acc, kept, ob, 0.05),
             "diagnostics_b1024_k8": lambda: ref.av_diagnostics(feat, acc, kept, ob, 10)}
    for Bb in (1024, 2048):
        conf = rng.uniform(0.02, 1.0, (Bb, K)).astype(np.float32)
        cost = W.budget_costs(Bb, K)
        calls["budget_b%d_k8" % Bb] = lambda conf=conf, cost=cost: ref.av_budget(conf, cost)
    ctx, lens = W.ngram_contexts(256, 8192, 128256, seed=7, device="cpu")
    ctx, lens = ctx.numpy(), lens.numpy()
    calls["ngram_b256_s8192_n2to4_k8"] = lambda: ref.ngram_propose(ctx, lens, 2, 4, 8)
    out["next_rows_oracle_us_per_call"] = {k: per_call(f) for k, f in calls.items()}
    return out


def _cpu_model():
    """The host CPU's model name (Linux), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


if __name__ == "__main__":
    main()
