"""Seeded synthetic verification workloads.

This module only *generates inputs*: logits and draft tokens.  It holds none of
the verification arithmetic, and both the HIP library and the CPU oracle are
fed the same tensors it produces.  Draft tokens are drawn from the draft
distribution with torch's own generator (a drafter's job, outside the path
being verified); the verifier's own randomness is the separate Philox stream
keyed by the verification seed.

Recipes (B sequences, K drafts, V vocabulary):
  gaussian  draft logits D ~ 4 N(0,1) over K+1 rows, target = 0.8 D + 2 N(0,1);
            the draft uses rows 0..K-1; tokens ~ softmax(D_j / T).
  fly       target rows i.i.d.: with probability 1/2 "peaked" (N(0,1) plus 12 at
            one uniform id), else "flat" N(0,1); each draft token is the row's
            top token with probability 0.7, else one of its ranks 2..5
            uniformly.  No draft logits.
  zipf      per row a random permutation pi of the ids and
            logit[pi(r)] = -5.5 ln(r+1) + 0.5 N(0,1) for rank r = 0..V-1;
            draft = target + 1.5 N(0,1); tokens ~ softmax(draft_j / T).
bfloat16 inputs are generated in float32 and rounded once (nearest-even).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import torch

CONFIGS = {
    0: dict(name="lossless_b1_k4_v32000_f32", B=1, K=4, V=32000, dtype="f32",
            mode="lossless", temperature=1.0, recipe="gaussian"),
    1: dict(name="lossless_av_b64_k5_v128256_bf16", B=64, K=5, V=128256, dtype="bf16",
            mode="lossless", temperature=1.0, recipe="gaussian",
            av=dict(omega=1.0, beta0=0.5, beta_step=-0.3, lr=0.05, tau=0.0)),
    2: dict(name="fly_b256_k8_v128256_bf16", B=256, K=8, V=128256, dtype="bf16", mode="fly",
            temperature=1.0, theta=0.3, window=4, recipe="fly"),
    3: dict(name="lossless_t0.7_b512_k4_v152064_bf16", B=512, K=4, V=152064, dtype="bf16",
            mode="lossless", temperature=0.7, recipe="zipf"),
    4: dict(name="av_pipeline_b1024_k8_v128256_bf16_x20", B=1024, K=8, V=128256, dtype="bf16",
            mode="lossless", temperature=1.0, recipe="gaussian", steps=20,
            av=dict(omega=1.0, beta0=0.5, beta_step=-0.3, lr=0.05, tau=0.2)),
}


@dataclass
class Batch:
    target: torch.Tensor                 # [B, K+1, S]
    draft: Optional[torch.Tensor]        # [B, K, S] or None
    tokens: torch.Tensor                 # int32 [B, K]
    V: int
    temperature: float
    meta: dict = field(default_factory=dict)


def torch_dtype(name: str):
    return {"bf16": torch.bfloat16, "f32": torch.float32}[name]


def generator(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def data_seed(cfg: int, step: int = 0) -> int:
    return (1000 + cfg) * 1_000_003 + step


def _pad(x: torch.Tensor, stride: int, fill: float) -> torch.Tensor:
    V = x.shape[-1]
    if stride == V:
        return x.contiguous()
    out = torch.full(x.shape[:-1] + (stride,), fill, dtype=x.dtype, device=x.device)
    out[..., :V] = x
    return out


def sample_rows(logits: torch.Tensor, temperature: float, g: torch.Generator,
                chunk: int = 1024) -> torch.Tensor:
    """One categorical draw per row of softmax(logits / T) (torch primitives)."""
    rows = logits.reshape(-1, logits.shape[-1])
    out = torch.empty(rows.shape[0], dtype=torch.int64, device=rows.device)
    for i in range(0, rows.shape[0], chunk):
        pr = torch.softmax(rows[i:i + chunk].float() / temperature, dim=-1)
        out[i:i + chunk] = torch.multinomial(pr, 1, generator=g).squeeze(1)
    return out.reshape(logits.shape[:-1]).to(torch.int32)


def gaussian(B, K, V, dtype="bf16", temperature=1.0, seed=0, token_seed=0, device="cpu",
             stride=None, pad_fill=float("nan")) -> Batch:
    g = generator(seed, device)
    D = torch.randn(B, K + 1, V, generator=g, device=device) * 4.0
    T = 0.8 * D + 2.0 * torch.randn(B, K + 1, V, generator=g, device=device)
    dt = torch_dtype(dtype)
    draft = D[:, :K].to(dt)
    target = T.to(dt)
    del D, T
    tokens = sample_rows(draft, temperature, generator(token_seed, device))
    S = stride or V
    return Batch(_pad(target, S, pad_fill), _pad(draft, S, pad_fill), tokens, V, temperature,
                 dict(recipe="gaussian"))


def fly(B, K, V, seed=0, device="cpu", stride=None, peak=12.0, p_match=0.7,
        pad_fill=float("nan")) -> Batch:
    g = generator(seed, device)
    t = torch.randn(B, K + 1, V, generator=g, device=device)
    peaked = torch.rand(B, K + 1, generator=g, device=device) < 0.5
    ids = torch.randint(0, V, (B, K + 1, 1), generator=g, device=device)
    t.scatter_add_(2, ids, peaked.to(t.dtype).unsqueeze(-1) * peak)
    target = t.to(torch.bfloat16)
    del t
    top5 = torch.topk(target[:, :K].float(), 5, dim=-1).indices
    match = torch.rand(B, K, generator=g, device=device) < p_match
    alt = torch.randint(1, 5, (B, K), generator=g, device=device)
    pick = torch.where(match, torch.zeros_like(alt), alt)
    tokens = top5.gather(-1, pick.unsqueeze(-1)).squeeze(-1).to(torch.int32)
    S = stride or V
    return Batch(_pad(target, S, pad_fill), None, tokens, V, 1.0,
                 dict(recipe="fly", peaked=peaked.cpu()))


def zipf(B, K, V, temperature=0.7, seed=0, token_seed=0, device="cpu", stride=None,
         pad_fill=float("nan")) -> Batch:
    g = generator(seed, device)
    rows = B * (K + 1)
    base = -5.5 * torch.log(torch.arange(V, device=device, dtype=torch.float32) + 1.0)
    perm = torch.argsort(torch.rand(rows, V, generator=g, device=device), dim=1)
    vals = base.unsqueeze(0) + 0.5 * torch.randn(rows, V, generator=g, device=device)
    t = torch.empty(rows, V, device=device)
    t.scatter_(1, perm, vals)
    del perm, vals
    t = t.view(B, K + 1, V)
    d = t[:, :K] + 1.5 * torch.randn(B, K, V, generator=g, device=device)
    target = t.to(torch.bfloat16)
    draft = d.to(torch.bfloat16)
    del t, d
    tokens = sample_rows(draft, temperature, generator(token_seed, device))
    S = stride or V
    return Batch(_pad(target, S, pad_fill), _pad(draft, S, pad_fill), tokens, V, temperature,
                 dict(recipe="zipf"))


def make(cfg: int, device="cpu", B=None, K=None, V=None, stride=None, step=0) -> Batch:
    """Inputs of workload `cfg` (optionally with other B / K / V / stride)."""
    c = CONFIGS[cfg]
    B = B or c["B"]
    K = K or c["K"]
    V = V or c["V"]
    seed = data_seed(cfg, step)
    if c["recipe"] == "gaussian":
        b = gaussian(B, K, V, c["dtype"], c["temperature"], seed, token_seed=step, device=device,
                     stride=stride)
    elif c["recipe"] == "fly":
        b = fly(B, K, V, seed, device, stride)
    else:
        b = zipf(B, K, V, c["temperature"], seed, token_seed=step, device=device, stride=stride)
    b.meta.update(cfg=cfg, name=c["name"], step=step)
    return b


def av_init(cfg: int, K: Optional[int] = None) -> list:
    """Initial (omega, beta_0..beta_{K-1}) of an adaptive-verification workload."""
    a = CONFIGS[cfg]["av"]
    K = K or CONFIGS[cfg]["K"]
    return [a["omega"]] + [a["beta0"] + a["beta_step"] * i for i in range(K)]


def budget_costs(B: int, K: int, per_request: float = 0.01, per_draft: float = 0.002,
                 curve: float = 2.0):
    """Synthetic cost table (ms) of verifying a budget of k = 0..B*K drafts
    in one step, standing in for the measured draft + verify cost tables of
    budgeted trimming: a per-request base, a per-draft slope and a quadratic
    term that reaches `curve` ms at k = B*K.  float64 numpy array."""
    import numpy as np
    M = B * K
    k = np.arange(M + 1, dtype=np.float64)
    return per_request * B + per_draft * k + curve * (k / max(M, 1)) ** 2


def ngram_contexts(B: int, S: int, vocab: int, seed: int = 0, repeat_every: int = 3,
                   device="cpu"):
    """Synthetic token contexts for prompt-lookup drafting: uniform token ids
    over `vocab`, lengths uniform in [S/2, S], and in every `repeat_every`-th
    sequence a span of 2..11 tokens from the first half copied to the end (the
    repetition prompt lookup exploits).  Returns (int32 [B, S], int32 [B])."""
    g = generator(seed, "cpu")
    ctx = torch.randint(0, vocab, (B, S), generator=g, dtype=torch.int32)
    lens = torch.randint(S // 2, S + 1, (B,), generator=g, dtype=torch.int32)
    for b in range(0, B, repeat_every):
        n = int(lens[b])
        src = int(torch.randint(0, n // 2, (1,), generator=g))
        span = int(torch.randint(2, 12, (1,), generator=g))
        ctx[b, n - span:n] = ctx[b, src:src + span].clone()
    return ctx.to(device), lens.to(device)
