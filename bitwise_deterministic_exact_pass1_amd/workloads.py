"""Seeded synthetic inputs for the attention and cross-entropy workloads.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic.  The GPU tests, the CPU oracle's tests and the benchmark
all take their inputs from here, so both sides always see identical bytes.

Every tensor is drawn on the CPU from ``torch.Generator('cpu').manual_seed``
in the order listed, as f32 N(0,1), then rounded to bf16 (round to nearest
even) where the workload is bf16.  No public dataset is involved: the pages
measure on synthetic N(0,1) data, and the long non-causal shape is the
production boundary of the vortex exact-attention contract page ("Canonical
Boundary": 37810 tokens, 56 heads, head dim 128, interleaved QKV rows of 21504
bf16 with Q/K/V at offsets 0/7168/14336).
"""
from __future__ import annotations

import math

import torch


def _gen(seed: int) -> torch.Generator:
    return torch.Generator(device="cpu").manual_seed(seed)


def default_scale(D: int) -> float:
    """RN64(1/RN64(sqrt(D))): 1/sqrt(D) evaluated in binary64 on the host."""
    return 1.0 / math.sqrt(D)


def attn_inputs(seed: int, B: int, Hq: int, Hkv: int, Sq: int, Skv: int, D: int,
                dtype: torch.dtype = torch.bfloat16, std: float = 1.0):
    """Q [B,Hq,Sq,D], K and V [B,Hkv,Skv,D]; N(0, std^2) drawn in that order."""
    g = _gen(seed)
    q = torch.randn(B, Hq, Sq, D, generator=g) * std
    k = torch.randn(B, Hkv, Skv, D, generator=g) * std
    v = torch.randn(B, Hkv, Skv, D, generator=g) * std
    return q.to(dtype), k.to(dtype), v.to(dtype)


# ---------------------------------------------------------------- named workloads

ATTN_WORKLOADS = {
    # name: (seed, B, Hq, Hkv, S, D, dtype, causal, scale)
    "tiny_mha_f32": (1, 1, 2, 2, 128, 64, torch.float32, False, 0.125),
    "gqa_causal_bf16": (2, 2, 8, 2, 1024, 128, torch.bfloat16, True, None),
    "cp_share_bf16": (3, 1, 32, 8, 8192, 128, torch.bfloat16, True, None),
    "cp_share_d256_bf16": (6, 1, 32, 8, 2048, 256, torch.bfloat16, True, None),
}


def attn_workload(name: str):
    """Returns dict(q, k, v, causal, scale, desc) for a named dense BHSD workload."""
    seed, B, Hq, Hkv, S, D, dtype, causal, scale = ATTN_WORKLOADS[name]
    q, k, v = attn_inputs(seed, B, Hq, Hkv, S, S, D, dtype)
    return dict(q=q, k=k, v=v, causal=causal, scale=default_scale(D) if scale is None else scale,
                desc=f"B={B} Hq={Hq} Hkv={Hkv} S={S} D={D} {str(dtype).split('.')[-1]} "
                     f"{'causal' if causal else 'non-causal'}")


LONG_S, LONG_H, LONG_D, LONG_ROW = 37810, 56, 128, 21504


def long_nhd_buffer(seed: int = 5, S: int = LONG_S) -> torch.Tensor:
    """One interleaved QKV buffer [S, 21504] bf16, N(0,1)."""
    g = _gen(seed)
    return torch.randn(S, LONG_ROW, generator=g).to(torch.bfloat16)


def long_nhd_views(buf: torch.Tensor):
    """Q, K, V as [1, H, S, D] views of the interleaved buffer.

    Element (b, h, s, d) of Q sits at s*21504 + h*128 + d; K and V add 7168 and
    14336.  Strides (B, H, S, D) = (S*21504, 128, 21504, 1)."""
    S = buf.shape[0]
    sB, sH, sS = S * LONG_ROW, LONG_D, LONG_ROW
    views = []
    for off in (0, LONG_H * LONG_D, 2 * LONG_H * LONG_D):
        views.append(torch.as_strided(buf, (1, LONG_H, S, LONG_D), (sB, sH, sS, 1), buf.storage_offset() + off))
    return tuple(views)


def ce_inputs(seed: int = 4, N: int = 4096, V: int = 128256, dtype: torch.dtype = torch.bfloat16,
              std: float = 2.0, boost: float = 4.0):
    """logits [N, V] = std*N(0,1) with the target logit of each row raised by
    `boost`; targets uniform in [0, V).  Drawn: logits, then targets."""
    g = _gen(seed)
    x = torch.randn(N, V, generator=g) * std
    t = torch.randint(0, V, (N,), generator=g, dtype=torch.int64)
    x[torch.arange(N), t] += boost
    return x.to(dtype), t


def kv_split_ranges(splits):
    """[(lo, hi), ...] for consecutive shard lengths."""
    out, lo = [], 0
    for n in splits:
        out.append((lo, lo + n))
        lo += n
    return out


def shard_order(seed: int, n: int):
    """A seeded permutation of range(n) (the order shards are composed in)."""
    return torch.randperm(n, generator=_gen(seed)).tolist()
