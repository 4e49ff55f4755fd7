"""Float32 contrast: the conventional combines the exact path replaces.

The det-attn page motivates the method with the usual float32 online-softmax
combine of KV-shard partials (running max, rescaled sums and outputs): merging
the same shards starting from a different shard gives different bits.  The
det-cross-entropy page makes the same point for a float32 logsumexp combined
over vocabulary splits, where some tokens' losses flip with the split count.
These helpers compute those conventional results with plain torch float32
operations so that the bench and the tests can set them beside the exact path,
which gives one set of bits for every order and split.  They are measurement
aids, not part of the path.
"""
from __future__ import annotations

import hashlib
from typing import List, Sequence, Tuple

import torch


def digest(t: torch.Tensor) -> str:
    """Short sha256 of a tensor's bytes (its bits, not its values)."""
    return hashlib.sha256(t.detach().contiguous().cpu().numpy().tobytes()).hexdigest()[:16]


def rotations(n: int) -> List[List[int]]:
    """The n cyclic merge orders r, r+1, ..., r+n-1 (mod n)."""
    return [[(r + a) % n for a in range(n)] for r in range(n)]


def f32_attn_partials(Q, K, V, splits: Sequence[int], causal: bool, scale: float):
    """Per KV shard, float32 (m, l, o): the max of the scaled scores, the sum of
    exp(s - m) and the normalized output sum(p v) / l (zeros for a row that sees
    no key of the shard)."""
    B, Hq, Sq, D = Q.shape
    g = Hq // K.shape[1]
    q = Q.float()
    k = K.float().repeat_interleave(g, dim=1)
    v = V.float().repeat_interleave(g, dim=1)
    rows = torch.arange(Sq, device=Q.device)[:, None]
    parts, lo = [], 0
    for n in splits:
        hi = lo + n
        s = torch.matmul(q, k[:, :, lo:hi].transpose(-1, -2).contiguous()) * scale
        if causal:
            s = s.masked_fill(torch.arange(lo, hi, device=Q.device)[None, :] > rows, float("-inf"))
        m = s.amax(-1, keepdim=True)
        p = torch.exp(s - torch.where(torch.isinf(m), torch.zeros_like(m), m))
        l = p.sum(-1, keepdim=True)
        o = torch.matmul(p, v[:, :, lo:hi].contiguous()) / torch.where(l > 0, l, torch.ones_like(l))
        parts.append((m, l, o))
        lo = hi
    return parts


def f32_attn_combine(parts, order: Sequence[int]) -> torch.Tensor:
    """Merge the partials pairwise in `order` with the online-softmax rescale."""
    m, l, o = parts[order[0]]
    for a in order[1:]:
        mb, lb, ob = parts[a]
        mn = torch.maximum(m, mb)
        ref = torch.where(torch.isinf(mn), torch.zeros_like(mn), mn)
        la, lb = l * torch.exp(m - ref), lb * torch.exp(mb - ref)
        ln = la + lb
        o = (o * la + ob * lb) / torch.where(ln > 0, ln, torch.ones_like(ln))
        m, l = mn, ln
    return o


def f32_ce_loss(X: torch.Tensor, T: torch.Tensor, nsplit: int) -> torch.Tensor:
    """Per-token float32 loss from a logsumexp combined over `nsplit` equal
    vocabulary splits: per split its max and sum of exp(x - max), merged by
    rescaling to the global max."""
    N, V = X.shape
    bounds = [V * a // nsplit for a in range(nsplit + 1)]
    ms, ss = [], []
    for lo, hi in zip(bounds[:-1], bounds[1:]):
        x = X[:, lo:hi].float()
        m = x.amax(1)
        ss.append(torch.exp(x - m[:, None]).sum(1))
        ms.append(m)
        del x
    M = torch.stack(ms).amax(0)
    S = torch.zeros_like(M)
    for m, s in zip(ms, ss):
        S = S + s * torch.exp(m - M)
    lse = M + torch.log(S)
    return lse - X.gather(1, T[:, None]).squeeze(1).float()


def attention_contrast(attention, Q, K, V, splits: Sequence[int], causal: bool, scale: float) -> dict:
    """Rotations of the shard merge order: distinct output digests of the float32
    combine and of det_attn_sharded, the largest float32 spread between
    rotations, and the float32 error against the exact output."""
    parts = f32_attn_partials(Q, K, V, splits, causal, scale)
    f32 = [f32_attn_combine(parts, r) for r in rotations(len(splits))]
    det = [attention.det_attn_sharded(Q, K, V, list(splits), causal, scale, order=r) for r in rotations(len(splits))]
    exact = det[0]
    spread = max(float((a - f32[0]).abs().max()) for a in f32)
    return {"splits": list(splits), "orders": len(f32),
            "f32_distinct_digests": len({digest(a) for a in f32}),
            "f32_max_spread": spread,
            "f32_max_abs_err_vs_exact": max(float((a - exact).abs().max()) for a in f32),
            "det_distinct_digests": len({digest(a) for a in det})}


def ce_contrast(cross_entropy, X: torch.Tensor, T: torch.Tensor, splits=(1, 2, 4, 8)) -> dict:
    """Tokens whose float32 loss bits differ from the one-split loss, per split
    count, beside the exact path's vocabulary-split losses (rowmax, digit sums
    and finalize per split)."""
    base = f32_ce_loss(X, T, 1)
    loss, m, _ = cross_entropy.forward(X, T)
    N, V = X.shape
    f32_flips, det_flips = {}, {}
    for n in splits:
        f = f32_ce_loss(X, T, n)
        f32_flips[n] = int((f.view(torch.int32) != base.view(torch.int32)).sum())
        bounds = [V * a // n for a in range(n + 1)]
        gm = torch.stack([cross_entropy.rowmax(X, lo, hi) for lo, hi in zip(bounds[:-1], bounds[1:])]).amax(0)
        den = None
        for lo, hi in zip(bounds[:-1], bounds[1:]):
            den = cross_entropy.denom_digits(X, gm, lo, hi, out=den)
        l2, _ = cross_entropy.finalize(den, X, T, gm)
        det_flips[n] = int((l2.view(torch.int32) != loss.view(torch.int32)).sum())
    return {"tokens": N, "f32_flipped_losses": f32_flips, "det_flipped_losses": det_flips}
