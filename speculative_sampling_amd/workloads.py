"""Seeded synthetic inputs for the verify-and-resample step.

This module only draws random logits and per-row parameters; it holds none
of the step's arithmetic (no softmax, no filter, no sampling).  Draft tokens
are drawn afterwards by a sampler the caller supplies (the GPU library with
K = 0, or the oracle in tests), so that they follow the *filtered* draft
distribution of the same configuration.

The shapes follow the workloads of speculative sampling described on the
pages (K = 3..8 draft tokens, vocabularies of roughly 32k to 256k, batch-1
serving up to batched rows); the value distributions are synthetic stand-ins
for model logits:

  worked_example  V=4 fp32, target [0.5, 0.25, 0.15, 0.10], draft
                  [0.3, 0.4, 0.2, 0.1] at every position (roadtointelligence
                  "Speculative Decoding", "Why the output doesn't change").
  iid_normal      target N(0, s_t^2) i.i.d.; draft = target + N(0, s_d^2).
  peaked          target N(0, 4^2) plus +8 on 20 distinct random tokens per
                  (row, position); draft = target + N(0, 0.7^2).
  zipf_ragged     per-row random vocabulary permutation; rank-r logit
                  -1.1 ln r + N(0, 0.5^2); draft = target + N(0, 1); per-row
                  K_b ~ U{1..K_max}; padding rows are NaN; modes cycle
                  plain / top-k / top-p by row.

Logits are formed in fp32 and rounded once to bf16 (round-to-nearest-even)
where the workload is bf16; the draft is the target's fp32 value plus noise,
rounded once.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable, Optional

import torch

PLAIN, TOPK, TOPP, GREEDY = 0, 1, 2, 3
_DT = {"bf16": torch.bfloat16, "f32": torch.float32}


@dataclass
class Workload:
    name: str
    B: int
    K_max: int
    V: int
    dtype: str                       # "bf16" or "f32"
    target: torch.Tensor             # [B][K_max+1][V]
    draft: torch.Tensor              # [B][K_max][V]
    draft_tokens: Optional[torch.Tensor] = None   # [B][K_max] int32
    k_per_row: Optional[torch.Tensor] = None      # [B] int32
    mode: Optional[torch.Tensor] = None           # [B] uint8
    temperature: Optional[torch.Tensor] = None    # [B] float32
    top_k: Optional[torch.Tensor] = None          # [B] int32
    top_p: Optional[torch.Tensor] = None          # [B] float32
    default_mode: int = PLAIN
    default_temperature: float = 1.0
    default_top_k: int = 1
    default_top_p: float = 1.0
    seed: int = 0                    # Philox key of the verify step
    draft_seed: int = 0              # Philox key used to draw the draft tokens
    meta: dict = field(default_factory=dict)

    def algorithmic_bytes(self) -> int:
        """Logit bytes the step must read at least once: sum_b (2 K_b + 1) V esize."""
        es = 2 if self.dtype == "bf16" else 4
        if self.k_per_row is None:
            kb_sum = self.B * self.K_max
        else:
            kb_sum = int(self.k_per_row.to(torch.int64).sum().item())
        return (2 * kb_sum + self.B) * self.V * es

    def row_params(self):
        """Per-row (mode, temperature, top_k, top_p) arrays for the draft rows.

        Draft token d[b][t] is drawn from row t of sequence b's draft with the
        same sampling controls as the sequence, so the per-row parameters are
        repeated K_max times.
        """
        def rep(x):
            return None if x is None else x.repeat_interleave(self.K_max)
        return rep(self.mode), rep(self.temperature), rep(self.top_k), rep(self.top_p)

    def to(self, device) -> "Workload":
        def mv(x):
            return None if x is None else x.to(device)
        return Workload(self.name, self.B, self.K_max, self.V, self.dtype, mv(self.target),
                        mv(self.draft), mv(self.draft_tokens), mv(self.k_per_row), mv(self.mode),
                        mv(self.temperature), mv(self.top_k), mv(self.top_p), self.default_mode,
                        self.default_temperature, self.default_top_k, self.default_top_p,
                        self.seed, self.draft_seed, dict(self.meta))


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _round(x32: torch.Tensor, dtype: str) -> torch.Tensor:
    return x32.to(_DT[dtype])


def bits_u16(t: torch.Tensor):
    """bf16 tensor -> numpy uint16 array of its bit patterns (host copy)."""
    return t.contiguous().view(torch.int16).cpu().numpy().view("uint16")


def host_array(t: torch.Tensor):
    """Logit tensor -> numpy array the oracle reads (uint16 bits or float32)."""
    if t.dtype == torch.bfloat16:
        return bits_u16(t)
    return t.contiguous().cpu().numpy()


def worked_example(B: int, K: int = 4, *, seed: int = 1, draft_seed: int = 1001,
                   device="cpu") -> Workload:
    q = torch.tensor([0.5, 0.25, 0.15, 0.10], dtype=torch.float64)
    p = torch.tensor([0.3, 0.4, 0.2, 0.1], dtype=torch.float64)
    tq = torch.log(q).to(torch.float32).to(device)
    tp = torch.log(p).to(torch.float32).to(device)
    target = tq.expand(B, K + 1, 4).contiguous()
    draft = tp.expand(B, K, 4).contiguous()
    return Workload("worked_example", B, K, 4, "f32", target, draft, default_mode=PLAIN,
                    default_temperature=1.0, seed=seed, draft_seed=draft_seed)


def iid_normal(B: int, K: int, V: int, *, sigma_t: float = 3.0, sigma_d: float = 1.0,
               dtype: str = "bf16", mode: int = PLAIN, temperature: float = 1.0,
               top_k: int = 1, top_p: float = 1.0, seed: int = 0, gen_seed: int = 0,
               draft_seed: Optional[int] = None, device="cpu") -> Workload:
    g = _gen(gen_seed, device)
    t32 = torch.randn(B, K + 1, V, generator=g, device=device) * sigma_t
    d32 = t32[:, :K] + torch.randn(B, K, V, generator=g, device=device) * sigma_d
    return Workload(f"iid_normal_s{sigma_d}", B, K, V, dtype, _round(t32, dtype).contiguous(),
                    _round(d32, dtype).contiguous(), default_mode=mode,
                    default_temperature=temperature, default_top_k=top_k, default_top_p=top_p,
                    seed=seed, draft_seed=(gen_seed + 7919 if draft_seed is None else draft_seed))


def peaked(B: int = 64, K: int = 4, V: int = 128256, *, n_peaks: int = 20, peak: float = 8.0,
           sigma_t: float = 4.0, sigma_d: float = 0.7, dtype: str = "bf16", mode: int = TOPP,
           temperature: float = 0.8, top_p: float = 0.8, top_k: int = 1, seed: int = 0,
           gen_seed: int = 0, draft_seed: Optional[int] = None, device="cpu") -> Workload:
    g = _gen(gen_seed, device)
    t32 = torch.randn(B, K + 1, V, generator=g, device=device) * sigma_t
    # 20 distinct uniformly placed tokens per (row, position): the top-20 of
    # i.i.d. uniform keys is a uniform random 20-subset.
    keys = torch.rand(B, K + 1, V, generator=g, device=device)
    idx = keys.topk(n_peaks, dim=-1).indices
    del keys
    t32.scatter_add_(-1, idx, torch.full(idx.shape, peak, device=device))
    d32 = t32[:, :K] + torch.randn(B, K, V, generator=g, device=device) * sigma_d
    return Workload("peaked", B, K, V, dtype, _round(t32, dtype).contiguous(),
                    _round(d32, dtype).contiguous(), default_mode=mode,
                    default_temperature=temperature, default_top_k=top_k, default_top_p=top_p,
                    seed=seed, draft_seed=(gen_seed + 7919 if draft_seed is None else draft_seed))


def zipf_ragged(B: int = 512, K_max: int = 8, V: int = 256000, *, dtype: str = "bf16",
                slope: float = 1.1, sigma_t: float = 0.5, sigma_d: float = 1.0,
                temperature: float = 0.7, top_k: int = 50, top_p: float = 0.9,
                seed: int = 0, gen_seed: int = 0, draft_seed: Optional[int] = None,
                device="cpu") -> Workload:
    g = _gen(gen_seed, device)
    kpr = torch.randint(1, K_max + 1, (B,), generator=g, device=device, dtype=torch.int64)
    modes = torch.tensor([PLAIN, TOPK, TOPP], dtype=torch.uint8, device=device)[
        torch.arange(B, device=device) % 3]
    dt = _DT[dtype]
    target = torch.empty(B, K_max + 1, V, dtype=dt, device=device)
    draft = torch.empty(B, K_max, V, dtype=dt, device=device)
    base = -slope * torch.log(torch.arange(1, V + 1, device=device, dtype=torch.float32))
    nan = float("nan")
    for b in range(B):
        perm = torch.randperm(V, generator=g, device=device)
        vals = base + torch.randn(K_max + 1, V, generator=g, device=device) * sigma_t
        t32 = torch.empty(K_max + 1, V, device=device)
        t32[:, perm] = vals
        d32 = t32[:K_max] + torch.randn(K_max, V, generator=g, device=device) * sigma_d
        kb = int(kpr[b].item())
        t32[kb + 1:] = nan
        d32[kb:] = nan
        target[b] = t32.to(dt)
        draft[b] = d32.to(dt)
    B_ = B
    return Workload("zipf_ragged", B_, K_max, V, dtype, target, draft,
                    k_per_row=kpr.to(torch.int32), mode=modes,
                    temperature=torch.full((B,), temperature, device=device),
                    top_k=torch.full((B,), top_k, dtype=torch.int32, device=device),
                    top_p=torch.full((B,), top_p, device=device),
                    default_mode=PLAIN, default_temperature=temperature, default_top_k=top_k,
                    default_top_p=top_p, seed=seed,
                    draft_seed=(gen_seed + 7919 if draft_seed is None else draft_seed))


def draw_draft_tokens(w: Workload, sampler: Callable) -> Workload:
    """Fill w.draft_tokens with one draw per draft row from its filtered
    distribution, using `sampler(rows [N][V], mode, temperature, top_k, top_p,
    defaults..., seed)` -> [N] int32 (the GPU library or the oracle).

    Draft rows beyond a sequence's K_b are padding and get token 0.
    """
    if w.K_max == 0:
        w.draft_tokens = torch.zeros(w.B, 0, dtype=torch.int32, device=w.target.device)
        return w
    md, tmp, tk, tp = w.row_params()
    rows = w.draft.reshape(w.B * w.K_max, w.V)
    toks = sampler(rows, md, tmp, tk, tp, w.default_mode, w.default_temperature,
                   w.default_top_k, w.default_top_p, w.draft_seed)
    toks = toks.reshape(w.B, w.K_max).to(torch.int32)
    if w.k_per_row is not None:
        t_idx = torch.arange(w.K_max, device=toks.device).unsqueeze(0)
        pad = t_idx >= w.k_per_row.to(toks.device).unsqueeze(1)
        toks = torch.where(pad, torch.zeros_like(toks), toks)
    w.draft_tokens = toks.contiguous()
    return w


def config(name: str, device="cpu", **kw) -> Workload:
    """The named workloads at their full sizes."""
    if name == "worked_example":
        kw.pop("gen_seed", None)   # its logits are the pages' fixed distributions
        return worked_example(kw.pop("B", 1_000_000), device=device, **kw)
    if name == "latency_b1":
        return iid_normal(kw.pop("B", 1), 4, 32000, sigma_t=3.0, sigma_d=1.0, dtype="bf16",
                          device=device, **kw)
    if name == "nucleus_b64":
        return peaked(64, 4, 128256, device=device, **kw)
    if name in ("plain_b64", "topk50_b64", "greedy_b64"):
        # the nucleus workload's shape and logits with another filter
        mode = {"plain_b64": PLAIN, "topk50_b64": TOPK, "greedy_b64": GREEDY}[name]
        return peaked(64, 4, 128256, mode=mode, top_k=50, device=device, **kw)
    if name.startswith("topk_f32"):
        sigma = float(name.split("_s")[-1]) if "_s" in name else 1.0
        greedy = "greedy" in name
        return iid_normal(256, 8, 32000, sigma_t=3.0, sigma_d=sigma, dtype="f32",
                          mode=GREEDY if greedy else TOPK, temperature=0.7, top_k=40,
                          device=device, **kw)
    if name == "zipf_ragged":
        return zipf_ragged(512, 8, 256000, device=device, **kw)
    raise KeyError(name)


HEADLINE = "nucleus_b64"
