"""Deterministic cross-entropy on MI355X (torch front end).

Names follow the det-cross-entropy page's API table: ``cross_entropy``
(autograd), ``forward``, ``rowmax``, ``denom_digits``, ``finalize``.  The loss
and its gradient are fixed functions of the logits: the vocabulary sum is an
exact long-accumulator sum, so vocabulary shards compose by an elementwise max
of the row maxima and an int64 add of the denominator digits.
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch

from ._lib import DEN_DIGITS, DET_BF16, DET_F32, check, lib

REDUCTIONS = {"none": 0, "mean": 1, "sum": 2}


def _logits(x: torch.Tensor) -> Tuple[int, int, int, int]:
    if x.dim() != 2 or not x.is_cuda:
        raise ValueError("logits are a CUDA tensor [N, V]")
    if x.shape[1] > 1 and x.stride(1) != 1:
        raise ValueError("logits rows must be contiguous")
    if x.dtype == torch.float32:
        code = DET_F32
    elif x.dtype == torch.bfloat16:
        code = DET_BF16
    else:
        raise TypeError(f"logits must be float32 or bfloat16, got {x.dtype}")
    N, V = x.shape
    return code, N, V, max(x.stride(0), V) if N > 1 else V


def _stream(x: torch.Tensor) -> int:
    return torch.cuda.current_stream(x.device).cuda_stream


def _targets(t: torch.Tensor, N: int) -> torch.Tensor:
    t = t.reshape(-1)
    if t.dtype != torch.int64 or t.numel() != N:
        raise ValueError("targets must be int64 [N]")
    return t.contiguous()


def rowmax(logits: torch.Tensor, v_lo: int = 0, v_hi: Optional[int] = None) -> torch.Tensor:
    """Per-token max over vocabulary columns [v_lo, v_hi): f32 [N]."""
    code, N, V, ld = _logits(logits)
    v_hi = V if v_hi is None else v_hi
    if not 0 <= v_lo <= v_hi <= V:
        raise ValueError("vocab range outside the logits")
    out = torch.empty(N, dtype=torch.float32, device=logits.device)
    check(lib().det_ce_rowmax(logits.data_ptr(), code, N, ld, v_lo, v_hi, out.data_ptr(), _stream(logits)))
    return out


def denom_digits(logits: torch.Tensor, global_rowmax: torch.Tensor, v_lo: int = 0, v_hi: Optional[int] = None,
                 out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Exact denominator digits of columns [v_lo, v_hi): canonical int64 [9, N].
    With `out` the range is added into it in place."""
    code, N, V, ld = _logits(logits)
    v_hi = V if v_hi is None else v_hi
    if not 0 <= v_lo <= v_hi <= V:
        raise ValueError("vocab range outside the logits")
    m = global_rowmax.contiguous()
    if m.dtype != torch.float32 or m.numel() != N:
        raise ValueError("rowmax must be float32 [N]")
    add_into = out is not None
    if out is None:
        out = torch.empty((DEN_DIGITS, N), dtype=torch.int64, device=logits.device)
    elif out.dtype != torch.int64 or tuple(out.shape) != (DEN_DIGITS, N) or not out.is_contiguous():
        raise ValueError("out must be contiguous int64 [9, N]")
    check(lib().det_ce_denom_digits(logits.data_ptr(), code, N, ld, m.data_ptr(), v_lo, v_hi, out.data_ptr(),
                                    int(add_into), _stream(logits)))
    return out


def finalize(den_digits: torch.Tensor, logits: torch.Tensor, targets: torch.Tensor,
             global_rowmax: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """(loss f32 [N], denom f64 [N]) from composed digits."""
    code, N, V, ld = _logits(logits)
    t = _targets(targets, N)
    m = global_rowmax.contiguous()
    d = den_digits.contiguous()
    if d.dtype != torch.int64 or tuple(d.shape) != (DEN_DIGITS, N):
        raise ValueError("den_digits must be int64 [9, N]")
    loss = torch.empty(N, dtype=torch.float32, device=logits.device)
    denom = torch.empty(N, dtype=torch.float64, device=logits.device)
    check(lib().det_ce_finalize(d.data_ptr(), logits.data_ptr(), code, N, V, ld, t.data_ptr(), m.data_ptr(),
                                loss.data_ptr(), denom.data_ptr(), _stream(logits)))
    return loss, denom


def forward(logits: torch.Tensor, targets: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Fused (loss f32 [N], rowmax f32 [N], denom f64 [N]) over the whole vocabulary."""
    code, N, V, ld = _logits(logits)
    t = _targets(targets, N)
    loss = torch.empty(N, dtype=torch.float32, device=logits.device)
    m = torch.empty(N, dtype=torch.float32, device=logits.device)
    denom = torch.empty(N, dtype=torch.float64, device=logits.device)
    check(lib().det_ce_forward(logits.data_ptr(), code, N, V, ld, t.data_ptr(), loss.data_ptr(), m.data_ptr(),
                               denom.data_ptr(), None, 0, _stream(logits)))
    return loss, m, denom


def reduce(loss: torch.Tensor, reduction: str) -> torch.Tensor:
    """none: the losses; sum/mean: RN32 of the exact sum (divided by N in fp64 for mean)."""
    code = REDUCTIONS[reduction]
    l = loss.contiguous()
    N = l.numel()
    out = torch.empty(N if code == 0 else 1, dtype=torch.float32, device=loss.device)
    check(lib().det_ce_reduce(l.data_ptr(), N, code, out.data_ptr(), None, 0, _stream(loss)))
    return out if code == 0 else out.reshape(())


def backward(logits: torch.Tensor, targets: torch.Tensor, rowmax_: torch.Tensor, denom: torch.Tensor,
             grad_loss: torch.Tensor, reduction: str, v0: int = 0) -> torch.Tensor:
    """dLogits f32 [N, V]: (softmax - onehot) times the upstream gradient.
    For a vocabulary shard, `logits` holds columns [v0, v0 + V) of the
    vocabulary (e.g. a column slice), `targets` are whole-vocabulary indices
    and rowmax_ / denom are the composed global values; the result is that
    shard's columns of the whole gradient, bit for bit."""
    code, N, V, ld = _logits(logits)
    t = _targets(targets, N)
    g = grad_loss.reshape(-1).to(torch.float32).contiguous()
    grad = torch.empty((N, V), dtype=torch.float32, device=logits.device)
    check(lib().det_ce_backward(logits.data_ptr(), code, N, V, ld, int(v0), t.data_ptr(),
                                rowmax_.contiguous().data_ptr(), denom.contiguous().data_ptr(), g.data_ptr(),
                                REDUCTIONS[reduction], grad.data_ptr(), V, _stream(logits)))
    return grad


class _DetCrossEntropy(torch.autograd.Function):
    @staticmethod
    def forward(ctx, logits, targets, reduction):
        loss, m, denom = forward(logits, targets)
        ctx.save_for_backward(logits, targets, m, denom)
        ctx.reduction = reduction
        return reduce(loss, reduction)

    @staticmethod
    def backward(ctx, grad_out):
        logits, targets, m, denom = ctx.saved_tensors
        g = backward(logits, targets, m, denom, grad_out, ctx.reduction)
        return g.to(logits.dtype), None, None


def cross_entropy(logits: torch.Tensor, targets: torch.Tensor, reduction: str = "mean") -> torch.Tensor:
    """Deterministic autograd cross-entropy (reduction 'mean', 'sum' or 'none')."""
    if reduction not in REDUCTIONS:
        raise ValueError("reduction must be 'mean', 'sum' or 'none'")
    return _DetCrossEntropy.apply(logits, targets, reduction)
