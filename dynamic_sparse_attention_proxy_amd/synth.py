"""Seeded synthetic prefill inputs shaped like the paper's workloads.

This module holds no arithmetic of the method itself: it only draws Q, K, V
with planted attention structure and applies rotary position embedding, so
that the HIP path and the fp64 oracle are fed the very same bf16 bits.

The paper measures on Llama-3.1-8B and Qwen2.5-7B (ai.info summary,
"Methodology in Plain English"); no weights or datasets are used here.  The
generator takes those models' attention shapes (query/KV head counts, head
dim 128, RoPE base) and replaces activations with Gaussians carrying:
  * an attention sink: keys 0..3 of a group get +8*u and the group's
    sink-dominant query heads get +1.5*u on every row;
  * needles: m key positions p with +6*w_p, and +0.5*w_p on every query of a
    sink-dominant head at positions after p;
  * diffuse heads: queries scaled by 0.3, no additions.

Random draws come from torch generators on the target device; generating on
the GPU and copying to the host gives the oracle the identical bits.
"""

from __future__ import annotations

import math
from dataclasses import dataclass
from typing import List, Optional

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    num_q_heads: int
    num_kv_heads: int
    seq_len: int
    head_dim: int
    seed: int
    rope_theta: float
    sink_frac: float
    needles: int
    diffuse_q_scale: float = 0.3
    sink_k_boost: float = 8.0
    sink_q_boost: float = 1.5
    needle_k_boost: float = 6.0
    needle_q_boost: float = 0.5

    @property
    def num_sink_heads(self) -> int:
        return int(round(self.sink_frac * self.num_q_heads))


# The five prefill workloads: one small single-head case and four
# single-layer shapes up to 512k tokens.
WORKLOADS: List[Workload] = [
    Workload("single-head-4k", 1, 1, 4096, 128, 0, 5e5, 1.0, 4),
    Workload("llama3.1-8b-32k", 32, 8, 32768, 128, 1, 5e5, 0.7, 4),
    Workload("qwen2.5-7b-128k", 28, 4, 131072, 128, 2, 1e6, 0.8, 8),
    Workload("llama3.1-8b-256k", 32, 8, 262144, 128, 3, 5e5, 0.7, 16),
    Workload("llama3.1-8b-512k", 32, 8, 524288, 128, 4, 5e5, 0.7, 32),
]


def workload(idx_or_name) -> Workload:
    if isinstance(idx_or_name, int):
        return WORKLOADS[idx_or_name]
    for w in WORKLOADS:
        if w.name == idx_or_name:
            return w
    raise KeyError(idx_or_name)


def custom(num_q_heads: int, num_kv_heads: int, seq_len: int, seed: int = 0,
           rope_theta: float = 5e5, sink_frac: float = 0.7, needles: int = 4,
           head_dim: int = 128) -> Workload:
    return Workload(f"custom-{num_q_heads}x{num_kv_heads}-{seq_len}", num_q_heads, num_kv_heads,
                    seq_len, head_dim, seed, rope_theta, sink_frac, needles)


def _unit(x: torch.Tensor) -> torch.Tensor:
    return x / x.norm(dim=-1, keepdim=True)


def _rope_tables(n: int, d: int, theta: float, device):
    half = d // 2
    inv = theta ** (-torch.arange(half, dtype=torch.float64, device=device) * 2.0 / d)
    ang = torch.arange(n, dtype=torch.float64, device=device)[:, None] * inv[None, :]
    return torch.cos(ang), torch.sin(ang)


def _rope(x: torch.Tensor, cos: torch.Tensor, sin: torch.Tensor) -> torch.Tensor:
    """Rotate-half RoPE (pairs (k, k + d/2)) in float64."""
    half = x.shape[-1] // 2
    x1, x2 = x[..., :half], x[..., half:]
    return torch.cat([x1 * cos - x2 * sin, x2 * cos + x1 * sin], dim=-1)


@dataclass
class Inputs:
    q: torch.Tensor  # [Hq][n][d] bf16
    k: torch.Tensor  # [Hkv][n][d] bf16
    v: torch.Tensor  # [Hkv][n][d] bf16
    workload: Workload
    sink_heads: List[int]
    needle_pos: dict  # kv group -> sorted list of needle key positions


def make_inputs(w: Workload, device="cpu", seq_len: Optional[int] = None) -> Inputs:
    """Draw one workload's Q, K, V (bf16, post-RoPE) on `device`.

    Order of draws from one generator seeded with w.seed: Q per query head,
    K per KV head, V per KV head, then per KV group holding a sink-dominant
    head: the sink direction u, the needle positions (uniform without
    replacement in [128, n-128)) and one unit direction per needle.
    """
    n = w.seq_len if seq_len is None else seq_len
    d = w.head_dim
    Hq, Hkv = w.num_q_heads, w.num_kv_heads
    qpg = Hq // Hkv
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed)

    q = torch.empty((Hq, n, d), dtype=torch.bfloat16, device=dev)
    k = torch.empty((Hkv, n, d), dtype=torch.bfloat16, device=dev)
    v = torch.empty((Hkv, n, d), dtype=torch.bfloat16, device=dev)
    qraw = [torch.randn((n, d), generator=gen, device=dev, dtype=torch.float32) for _ in range(Hq)]
    kraw = [torch.randn((n, d), generator=gen, device=dev, dtype=torch.float32) for _ in range(Hkv)]
    for g in range(Hkv):
        v[g] = torch.randn((n, d), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)

    sink_heads = list(range(w.num_sink_heads))
    needle_pos = {}
    cos, sin = _rope_tables(n, d, w.rope_theta, dev)
    for g in range(Hkv):
        heads = [g * qpg + t for t in range(qpg)]
        sinky = [h for h in heads if h in sink_heads]
        kg = kraw[g]
        if sinky:
            u = _unit(torch.randn((d,), generator=gen, device=dev, dtype=torch.float32))
            m = min(w.needles, n - 256)  # needles live in [128, n - 128)
            pos = torch.randperm(max(n - 256, 1), generator=gen, device=dev)[:m] + 128
            pos, _ = torch.sort(pos)
            wdir = _unit(torch.randn((m, d), generator=gen, device=dev, dtype=torch.float32))
            needle_pos[g] = [int(p) for p in pos.cpu()]
            kg[0:4] += w.sink_k_boost * u
            kg[pos] += w.needle_k_boost * wdir
            # needle p reaches every query row after p: a running sum of
            # directions started at row p + 1 (p < n - 128 keeps it in range)
            add = torch.zeros((n, d), device=dev, dtype=torch.float32)
            add.index_add_(0, pos + 1, wdir)
            qadd = torch.cumsum(add, dim=0) * w.needle_q_boost + w.sink_q_boost * u
            for h in sinky:
                qraw[h] += qadd
            del add, qadd
        for h in heads:
            if h not in sink_heads:
                qraw[h] *= w.diffuse_q_scale
            q[h] = _rope(qraw[h].double(), cos, sin).to(torch.bfloat16)
            qraw[h] = None
        k[g] = _rope(kg.double(), cos, sin).to(torch.bfloat16)
        kraw[g] = None
    return Inputs(q, k, v, w, sink_heads, needle_pos)


# ---------------------------------------------------------------------------
# Graded-structure family for the routing-agreement measurement.
# ---------------------------------------------------------------------------

ROUTING_FAMILY_SINK_STEP = 2.5   # query coupling to the sink direction, per grid step
ROUTING_FAMILY_LOCAL_STEP = 0.35 # query coupling to the local direction, per grid step


def make_routing_family(seq_len: int = 32768, num_q_heads: int = 32, num_kv_heads: int = 8, seed: int = 5,
                        rope_theta: float = 5e5, sink_k_boost: float = 8.0, local_norm: float = 12.0,
                        device="cpu") -> Inputs:
    """Heads whose sink and recency structure is graded, so that routing
    signals cross their thresholds (Llama-3.1-8B attention shape).

    Q, K, V are iid N(0,1) from one generator seeded with `seed` (Q per query
    head, K per KV head, V per KV head, then per KV group: the sink direction
    u and the local direction c).  Per KV group g:
      * u is a random unit vector on the four lowest-frequency rotary pairs,
        which barely rotate over the sequence, so a sink coupling keeps its
        strength at every distance; keys 0..3 get + sink_k_boost * u;
      * c is a random vector of norm local_norm on the sixteen
        highest-frequency rotary pairs; every key gets + c, and after RoPE a
        query carrying c scores keys at small offsets highest (a recency
        window), the product decaying within about a hundred positions.
    Query head h = g * qpg + t gets + beta_h * u + lambda_h * c on every row,
    beta_h = 2.5 * (h mod 8) and lambda_h = 0.35 * (h div 8 mod 4): 32 heads
    span an 8 x 4 grid from structureless to sink- and recency-dominated.
    RoPE is applied after the additions, as in make_inputs.
    """
    n, d = seq_len, 128
    Hq, Hkv = num_q_heads, num_kv_heads
    qpg = Hq // Hkv
    half = d // 2
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    q = torch.empty((Hq, n, d), dtype=torch.bfloat16, device=dev)
    k = torch.empty((Hkv, n, d), dtype=torch.bfloat16, device=dev)
    v = torch.empty((Hkv, n, d), dtype=torch.bfloat16, device=dev)
    qraw = [torch.randn((n, d), generator=gen, device=dev, dtype=torch.float32) for _ in range(Hq)]
    kraw = [torch.randn((n, d), generator=gen, device=dev, dtype=torch.float32) for _ in range(Hkv)]
    for g in range(Hkv):
        v[g] = torch.randn((n, d), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    low = torch.tensor([p for p in range(half - 4, half)] + [p + half for p in range(half - 4, half)], device=dev)
    high = torch.tensor(list(range(16)) + [p + half for p in range(16)], device=dev)
    cos, sin = _rope_tables(n, d, rope_theta, dev)
    sink_heads = []
    for g in range(Hkv):
        u = torch.zeros(d, device=dev, dtype=torch.float32)
        u[low] = torch.randn((low.numel(),), generator=gen, device=dev, dtype=torch.float32)
        u = _unit(u)
        c = torch.zeros(d, device=dev, dtype=torch.float32)
        c[high] = torch.randn((high.numel(),), generator=gen, device=dev, dtype=torch.float32)
        c = local_norm * _unit(c)
        kg = kraw[g]
        kg[0:4] += sink_k_boost * u
        kg += c
        for t in range(qpg):
            h = g * qpg + t
            beta = ROUTING_FAMILY_SINK_STEP * (h % 8)
            lam = ROUTING_FAMILY_LOCAL_STEP * ((h // 8) % 4)
            if beta > 0:
                sink_heads.append(h)
            qraw[h] += beta * u + lam * c
            q[h] = _rope(qraw[h].double(), cos, sin).to(torch.bfloat16)
            qraw[h] = None
        k[g] = _rope(kg.double(), cos, sin).to(torch.bfloat16)
        kraw[g] = None
    w = Workload(f"routing-family-{Hq}x{Hkv}-{n}", Hq, Hkv, n, d, seed, rope_theta, 0.0, 0)
    return Inputs(q, k, v, w, sink_heads, {})
