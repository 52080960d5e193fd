"""Seeded synthetic workloads for the KV-cache path.

This module only draws inputs (keys, values, queries) and names the
workload shapes; it holds none of the method's arithmetic.  Both the oracle
side (tests) and the GPU side (tests, bench) take their inputs from here.

Shapes follow the model families the pages mention: a Llama-3.1-8B-shaped
layer (32 query / 8 KV heads, head dim 128) and a Command-R+-104B-shaped
layer (96 / 8, head dim 128), contexts of 32K, 128K and 1M tokens (leviatan.io,
"TurboQuant : 6x moins de cache...", section "Benchmarks de memoire"; the
wis-web.com article's 104B-at-128K example).  Values are N(0,1) with a few
perturbed channels, standing in for the real activations of those models.
"""
from __future__ import annotations

import dataclasses

import torch

# codec names shared by both sides; each side maps them to its own ids
RAW_F32, POLAR, POLAR_QJL, Q8_BLOCK32, POLAR_TREE = "raw_f32", "polar", "polar_qjl", "q8_block32", "polar_tree"


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    ctx: int
    n_q: int
    n_kv: int
    d: int
    dtype: str            # "f32" or "bf16" for K, V (and q before widening)
    k_codec: str
    k_bits: int
    m: int
    v_codec: str
    v_bits: int
    perturb: str          # recipe name, see make_kv
    layers: int = 1       # distinct layer caches a benchmark cycles through
    steps: int = 0        # serving steps (one appended token per sequence each)

    @property
    def group(self) -> int:
        return self.n_q // self.n_kv


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_b1_ctx1k_h8x2", 1, 1024, 8, 2, 128, "f32",
                 POLAR_QJL, 3, 128, POLAR, 3, "k_channels_x10_shared", layers=1),
        Workload("llama8b_b1_ctx32k", 1, 32768, 32, 8, 128, "bf16",
                 POLAR_QJL, 3, 128, POLAR, 2, "pairs_1pct_x8", layers=32),
        Workload("serving_b16_ctx8k", 16, 8192, 32, 8, 128, "bf16",
                 POLAR_QJL, 4, 128, POLAR, 4, "head_scale_u05_2", layers=32, steps=64),
        Workload("cmdr104b_b1_ctx128k", 1, 131072, 96, 8, 128, "bf16",
                 Q8_BLOCK32, 8, 0, POLAR, 2, "k_channels_x10_per_head", layers=64),
        Workload("long_b1_ctx1m", 1, 1048576, 32, 8, 128, "bf16",
                 POLAR_QJL, 3, 128, POLAR, 3, "pairs_2pct_student_t4", layers=4),
    ]
}

ORDER = list(WORKLOADS)


def with_ctx(w: Workload, ctx: int, batch: int | None = None) -> Workload:
    """Same heads, codecs and recipe at another context length (parity cases)."""
    return dataclasses.replace(w, ctx=ctx, batch=w.batch if batch is None else batch,
                               name=f"{w.name}@ctx{ctx}")


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _tdtype(w: Workload):
    return torch.float32 if w.dtype == "f32" else torch.bfloat16


def make_kv(w: Workload, n_tokens: int, seed: int, device="cpu", batch: int | None = None):
    """K and V of shape [batch][n_tokens][n_kv][d] in the workload's dtype.

    Recipes (channel picks are seeded, the same for every token):
      k_channels_x10_shared   4 K channels, the same in every KV head, x10
      pairs_1pct_x8           1% of the (head, channel) pairs x8, K and V
                              drawn independently
      head_scale_u05_2        one scale per KV head ~ U[0.5, 2] on K and V
      k_channels_x10_per_head 4 K channels per KV head x10
      pairs_2pct_student_t4   2% of the (head, channel) pairs replaced by
                              Student-t(4) draws, K and V independently
    """
    B = w.batch if batch is None else batch
    g = _gen(device, seed)
    shape = (B, n_tokens, w.n_kv, w.d)
    k = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    v = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    n_pairs = w.n_kv * w.d
    if w.perturb == "k_channels_x10_shared":
        ch = torch.randperm(w.d, generator=g, device=device)[:4]
        k[..., ch] *= 10.0
    elif w.perturb == "k_channels_x10_per_head":
        for h in range(w.n_kv):
            ch = torch.randperm(w.d, generator=g, device=device)[:4]
            k[:, :, h, ch] *= 10.0
    elif w.perturb == "pairs_1pct_x8":
        for t in (k, v):
            sel = torch.randperm(n_pairs, generator=g, device=device)[: round(0.01 * n_pairs)]
            flat = t.view(B, n_tokens, n_pairs)
            flat[..., sel] *= 8.0
    elif w.perturb == "head_scale_u05_2":
        sc = 0.5 + 1.5 * torch.rand(w.n_kv, generator=g, device=device)
        k *= sc.view(1, 1, -1, 1)
        v *= sc.view(1, 1, -1, 1)
    elif w.perturb == "pairs_2pct_student_t4":
        for t in (k, v):
            sel = torch.randperm(n_pairs, generator=g, device=device)[: round(0.02 * n_pairs)]
            flat = t.view(B, n_tokens, n_pairs)
            z = torch.randn((B, n_tokens, sel.numel()), generator=g, device=device)
            chi = torch.randn((4, B, n_tokens, sel.numel()), generator=g, device=device)
            chi2 = (chi * chi).sum(0)
            flat[..., sel] = z / torch.sqrt(chi2 / 4.0)
    else:
        raise ValueError(w.perturb)
    return k.to(_tdtype(w)), v.to(_tdtype(w))


def make_q(w: Workload, seed: int, device="cpu", batch: int | None = None):
    """One query token per sequence, [batch][n_q][d] fp32.  In bf16
    workloads the query is drawn in bf16 and widened, so both sides see the
    same values."""
    B = w.batch if batch is None else batch
    g = _gen(device, seed)
    q = torch.randn((B, w.n_q, w.d), generator=g, device=device, dtype=torch.float32)
    return q.to(_tdtype(w)).to(torch.float32)


def plant_focus_keys(w: Workload, k: torch.Tensor, q: torch.Tensor, seed: int, every: int = 1024,
                     logit: float = 16.0, n_tokens: int | None = None) -> torch.Tensor:
    """Peaked attention for the decode query q: in every window of `every`
    positions one seeded position per (sequence, KV head) gets the key
    logit * sqrt(d) * qbar / |qbar|^2, qbar the mean query of the head's
    group, so that the group's heads score it near `logit` (natural units)
    while the other keys keep their N(0, 1)-scale scores.  Returns a copy of
    k (same dtype, [batch][n][n_kv][d]) and the planted positions
    [batch][n_kv][n_windows]."""
    B, n, n_kv, d = k.shape
    n = n if n_tokens is None else n_tokens
    g = _gen(k.device, seed)
    qbar = q.to(torch.float32).view(B, n_kv, w.group, d).mean(2)                  # B, n_kv, d
    key = (logit * d ** 0.5) * qbar / (qbar * qbar).sum(-1, keepdim=True)
    n_win = (n + every - 1) // every
    off = torch.randint(0, every, (B, n_kv, n_win), generator=g, device=k.device)
    pos = torch.arange(n_win, device=k.device).view(1, 1, -1) * every + off
    pos = torch.minimum(pos, torch.full_like(pos, n - 1))
    out = k.clone()
    bi = torch.arange(B, device=k.device).view(B, 1, 1).expand_as(pos)
    hi = torch.arange(n_kv, device=k.device).view(1, n_kv, 1).expand_as(pos)
    out[bi, pos, hi] = key.view(B, n_kv, 1, d).expand(B, n_kv, n_win, d).to(k.dtype)
    return out, pos


def widen(x: torch.Tensor) -> torch.Tensor:
    """Exact widening of f32 / bf16 / f16 inputs to fp32."""
    return x.to(torch.float32)
