"""Shard-invariant exact softmax attention on MI355X (torch front end).

The names follow the det-attn page's API table: ``det_attn``, ``rowmax``,
``accumulate``, ``finalize``, ``det_attn_sharded``; composition of shards is
``combine_rowmax`` (elementwise max) and ``combine_digits`` (int64 add, then
carry to canonical form).  Everything runs in the HIP library; this module
only builds descriptors, passes torch's current stream and allocates the
workspace the library asks for.

Q is [B, Hq, Sq, D]; K and V are [B, Hkv, Skv, D] with Hq % Hkv == 0; all
float32 or all bfloat16 CUDA tensors whose last dimension is contiguous (any
other strides, e.g. views into an interleaved QKV projection, are fine).
"""
from __future__ import annotations

import ctypes as C
import math
from typing import Optional, Sequence, Tuple

import torch

from ._lib import DEN_DIGITS, NUM_DIGITS, DET_BF16, DET_F32, Out, Tensor, check, lib


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return DET_F32
    if t.dtype == torch.bfloat16:
        return DET_BF16
    raise TypeError(f"expected float32 or bfloat16, got {t.dtype}")


def _desc(t: torch.Tensor) -> Tensor:
    if t.dim() != 4:
        raise ValueError("attention operands are [B, H, S, D]")
    if not t.is_cuda:
        raise ValueError("attention operands must be on the GPU")
    if t.shape[3] > 1 and t.stride(3) != 1:
        raise ValueError("the head dimension must be contiguous")
    B, H, S, D = t.shape
    return Tensor(t.data_ptr(), _dtype_code(t), B, H, S, D, t.stride(0), t.stride(1), t.stride(2))


def _out(o: torch.Tensor) -> Out:
    return Out(o.data_ptr(), o.stride(0), o.stride(1), o.stride(2))


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _workspace(nbytes: int, device) -> Tuple[torch.Tensor, int]:
    ws = torch.empty(max(int(nbytes), 256) + 256, dtype=torch.uint8, device=device)
    addr = ws.data_ptr()
    aligned = (addr + 255) & ~255
    return ws, aligned


def default_scale(D: int) -> float:
    """RN64(1 / RN64(sqrt(D))), evaluated on the host in binary64."""
    return 1.0 / math.sqrt(D)


def det_attn(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, causal: bool = False,
             scale: Optional[float] = None) -> torch.Tensor:
    """Fused deterministic attention, f32 output [B, Hq, Sq, D]."""
    scale = default_scale(Q.shape[3]) if scale is None else float(scale)
    q, k, v = _desc(Q), _desc(K), _desc(V)
    out = torch.empty(Q.shape, dtype=torch.float32, device=Q.device)
    L = lib()
    nbytes = L.det_attn_workspace_size(C.byref(q), C.byref(k), C.byref(v), int(causal))
    ws, addr = _workspace(nbytes, Q.device)
    check(L.det_attn(C.byref(q), C.byref(k), C.byref(v), int(causal), scale, C.byref(_out(out)), addr, nbytes,
                     _stream(Q)))
    return out


def det_attn_with_stats(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, causal: bool = False,
                        scale: Optional[float] = None):
    """det_attn plus each row's max (f32 [B, Hq, Sq]) and RN64(DEN) (f64
    [B, Hq, Sq]), the two values the gradients need."""
    scale = default_scale(Q.shape[3]) if scale is None else float(scale)
    q, k, v = _desc(Q), _desc(K), _desc(V)
    out = torch.empty(Q.shape, dtype=torch.float32, device=Q.device)
    m = torch.empty(Q.shape[:3], dtype=torch.float32, device=Q.device)
    den = torch.empty(Q.shape[:3], dtype=torch.float64, device=Q.device)
    L = lib()
    nbytes = L.det_attn_workspace_size(C.byref(q), C.byref(k), C.byref(v), int(causal))
    ws, addr = _workspace(nbytes, Q.device)
    check(L.det_attn_stats(C.byref(q), C.byref(k), C.byref(v), int(causal), scale, C.byref(_out(out)),
                           m.data_ptr(), den.data_ptr(), addr, nbytes, _stream(Q)))
    return out, m, den


def det_attn_backward(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, O: torch.Tensor, dO: torch.Tensor,
                      rowmax: torch.Tensor, den64: torch.Tensor, causal: bool = False,
                      scale: Optional[float] = None):
    """(dQ, dK, dV) as float32 tensors shaped like Q, K, V: exact sums over
    the sequence axes (the rule stated in include/det_attn.h).  O and dO are
    the float32 forward output and its gradient; rowmax and den64 come from
    det_attn_with_stats."""
    scale = default_scale(Q.shape[3]) if scale is None else float(scale)
    if O.dtype != torch.float32 or dO.dtype != torch.float32:
        raise TypeError("O and dO must be float32")
    for t, dt in ((rowmax, torch.float32), (den64, torch.float64)):
        if t.dtype != dt or not t.is_contiguous() or tuple(t.shape) != tuple(Q.shape[:3]):
            raise ValueError("rowmax / den64 must be contiguous [B, Hq, Sq] float32 / float64")
    q, k, v, o, g = _desc(Q), _desc(K), _desc(V), _desc(O), _desc(dO)
    dq = torch.empty(Q.shape, dtype=torch.float32, device=Q.device)
    dk = torch.empty(K.shape, dtype=torch.float32, device=Q.device)
    dv = torch.empty(V.shape, dtype=torch.float32, device=Q.device)
    L = lib()
    nbytes = L.det_attn_backward_workspace_size(C.byref(q), C.byref(k), C.byref(v), int(causal))
    ws, addr = _workspace(nbytes, Q.device)
    check(L.det_attn_backward(C.byref(q), C.byref(k), C.byref(v), C.byref(o), C.byref(g), rowmax.data_ptr(),
                              den64.data_ptr(), int(causal), scale, C.byref(_out(dq)), C.byref(_out(dk)),
                              C.byref(_out(dv)), addr, nbytes, _stream(Q)))
    return dq, dk, dv


class _DetAttnFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, Q, K, V, causal, scale):
        out, m, den = det_attn_with_stats(Q, K, V, causal, scale)
        ctx.save_for_backward(Q, K, V, out, m, den)
        ctx.causal, ctx.scale = causal, scale
        return out

    @staticmethod
    def backward(ctx, dO):
        Q, K, V, out, m, den = ctx.saved_tensors
        dq, dk, dv = det_attn_backward(Q, K, V, out, dO.float(), m, den, ctx.causal, ctx.scale)
        return dq.to(Q.dtype), dk.to(K.dtype), dv.to(V.dtype), None, None


def det_attn_autograd(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, causal: bool = False,
                      scale: Optional[float] = None) -> torch.Tensor:
    """det_attn with gradients through det_attn_backward (cast to the input
    dtypes, round to nearest)."""
    scale = default_scale(Q.shape[3]) if scale is None else float(scale)
    return _DetAttnFunction.apply(Q, K, V, causal, scale)


def rowmax(Q: torch.Tensor, K: torch.Tensor, kv_lo: int = 0, kv_hi: Optional[int] = None, causal: bool = False,
           scale: Optional[float] = None, q_lo: int = 0, q_hi: Optional[int] = None,
           out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Per-query max score over keys [kv_lo, kv_hi): f32 [B, Hq, Sq].  Only
    query rows [q_lo, q_hi) are computed; the other rows of `out` (a new
    tensor filled with -inf when not given) are left as they are."""
    kv_hi = K.shape[2] if kv_hi is None else kv_hi
    q_hi = Q.shape[2] if q_hi is None else q_hi
    scale = default_scale(Q.shape[3]) if scale is None else float(scale)
    q, k = _desc(Q), _desc(K)
    if out is None:
        out = torch.full(Q.shape[:3], float("-inf"), dtype=torch.float32, device=Q.device)
    elif out.dtype != torch.float32 or not out.is_contiguous() or tuple(out.shape) != tuple(Q.shape[:3]):
        raise ValueError("out must be contiguous float32 [B, Hq, Sq]")
    L = lib()
    nbytes = L.det_attn_rowmax_workspace_size(C.byref(q), C.byref(k), q_lo, q_hi, kv_lo, kv_hi)
    ws, addr = _workspace(nbytes, Q.device)
    check(L.det_attn_rowmax(C.byref(q), C.byref(k), q_lo, q_hi, kv_lo, kv_hi, int(causal), scale, out.data_ptr(),
                            addr, nbytes, _stream(Q)))
    return out


def accumulate(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, rowmax: torch.Tensor, kv_lo: int = 0,
               kv_hi: Optional[int] = None, causal: bool = False, scale: Optional[float] = None,
               num: Optional[torch.Tensor] = None, den: Optional[torch.Tensor] = None, q_lo: int = 0,
               q_hi: Optional[int] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Exact digits of keys [kv_lo, kv_hi) against `rowmax` (normally the
    composed global max), for query rows [q_lo, q_hi).  Returns canonical
    (NUM int64 [14,B,Hq,Sq,D], DEN int64 [9,B,Hq,Sq]).  When `num`/`den` are
    given the shard is added into their rows [q_lo, q_hi) in place; new arrays
    start at zero."""
    kv_hi = K.shape[2] if kv_hi is None else kv_hi
    q_hi = Q.shape[2] if q_hi is None else q_hi
    scale = default_scale(Q.shape[3]) if scale is None else float(scale)
    B, Hq, Sq, D = Q.shape
    add_into = num is not None
    if add_into != (den is not None):
        raise ValueError("pass both num and den, or neither")
    if not add_into:
        num = torch.zeros((NUM_DIGITS, B, Hq, Sq, D), dtype=torch.int64, device=Q.device)
        den = torch.zeros((DEN_DIGITS, B, Hq, Sq), dtype=torch.int64, device=Q.device)
    _check_digits(num, den, (B, Hq, Sq, D))
    rm = rowmax.contiguous()
    if rm.dtype != torch.float32 or rm.numel() != B * Hq * Sq:
        raise ValueError("rowmax must be float32 [B, Hq, Sq]")
    q, k, v = _desc(Q), _desc(K), _desc(V)
    L = lib()
    nbytes = L.det_attn_accumulate_workspace_size(C.byref(q), C.byref(k), C.byref(v), q_lo, q_hi, kv_lo, kv_hi)
    ws, addr = _workspace(nbytes, Q.device)
    check(L.det_attn_accumulate(C.byref(q), C.byref(k), C.byref(v), rm.data_ptr(), q_lo, q_hi, kv_lo, kv_hi,
                                int(causal), scale, num.data_ptr(), den.data_ptr(), int(add_into), addr, nbytes,
                                _stream(Q)))
    return num, den


def _check_digits(num: torch.Tensor, den: torch.Tensor, shape) -> None:
    B, Hq, Sq, D = shape
    if num.dtype != torch.int64 or not num.is_contiguous() or tuple(num.shape) != (NUM_DIGITS, B, Hq, Sq, D):
        raise ValueError("num must be contiguous int64 [14, B, Hq, Sq, D]")
    if den.dtype != torch.int64 or not den.is_contiguous() or tuple(den.shape) != (DEN_DIGITS, B, Hq, Sq):
        raise ValueError("den must be contiguous int64 [9, B, Hq, Sq]")


def combine_rowmax(acc: torch.Tensor, part: torch.Tensor) -> torch.Tensor:
    """acc <- totalOrder max(acc, part), in place."""
    if acc.shape != part.shape or acc.dtype != torch.float32 or part.dtype != torch.float32:
        raise ValueError("rowmax arrays must be float32 of one shape")
    if not (acc.is_contiguous() and part.is_contiguous()):
        raise ValueError("rowmax arrays must be contiguous")
    check(lib().det_rowmax_combine(acc.data_ptr(), part.data_ptr(), acc.numel(), _stream(acc)))
    return acc


def combine_digits(acc: torch.Tensor, part: torch.Tensor) -> torch.Tensor:
    """acc <- canonical(acc + part), in place (digit-major planes, 14 or 9 digits)."""
    if acc.shape != part.shape or acc.dtype != torch.int64 or part.dtype != torch.int64:
        raise ValueError("digit arrays must be int64 of one shape")
    if not (acc.is_contiguous() and part.is_contiguous()):
        raise ValueError("digit arrays must be contiguous")
    K = acc.shape[0]
    check(lib().det_digits_combine(acc.data_ptr(), part.data_ptr(), acc.numel() // K, K, _stream(acc)))
    return acc


def normalize_digits(acc: torch.Tensor) -> torch.Tensor:
    """acc <- canonical(acc), in place (digit-major planes, 14 or 9 digits):
    the same exact values, e.g. after a caller-side int64 add of digit arrays."""
    if acc.dtype != torch.int64 or not acc.is_contiguous():
        raise ValueError("digit arrays must be contiguous int64")
    K = acc.shape[0]
    check(lib().det_digits_normalize(acc.data_ptr(), acc.numel() // K, K, _stream(acc)))
    return acc


def finalize(num: torch.Tensor, den: torch.Tensor, shape: Optional[Sequence[int]] = None) -> torch.Tensor:
    """out = RN32(RN64(NUM) / RN64(DEN)) as f32 [B, Hq, Sq, D]."""
    shape = tuple(num.shape[1:]) if shape is None else tuple(shape)
    _check_digits(num, den, shape)
    B, Hq, Sq, D = shape
    out = torch.empty(shape, dtype=torch.float32, device=num.device)
    check(lib().det_attn_finalize(num.data_ptr(), den.data_ptr(), B, Hq, Sq, D, C.byref(_out(out)),
                                  _stream(num)))
    return out


def det_attn_sharded(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, kv_splits: Sequence[int],
                     causal: bool = False, scale: Optional[float] = None,
                     order: Optional[Sequence[int]] = None) -> torch.Tensor:
    """KV-shard composition inside the library (per-shard rowmax composed by
    max, per-shard digits composed by int64 add in `order`, then finalize);
    bit-identical to det_attn for every split and order."""
    scale = default_scale(Q.shape[3]) if scale is None else float(scale)
    q, k, v = _desc(Q), _desc(K), _desc(V)
    n = len(kv_splits)
    splits = (C.c_int64 * n)(*[int(x) for x in kv_splits])
    order_arr = None if order is None else (C.c_int32 * n)(*[int(x) for x in order])
    out = torch.empty(Q.shape, dtype=torch.float32, device=Q.device)
    L = lib()
    nbytes = L.det_attn_sharded_workspace_size(C.byref(q), C.byref(k), C.byref(v), splits, n, int(causal))
    ws, addr = _workspace(nbytes, Q.device)
    check(L.det_attn_sharded(C.byref(q), C.byref(k), C.byref(v), splits, n, order_arr, int(causal), scale,
                             C.byref(_out(out)), addr, nbytes, _stream(Q)))
    return out


def det_attn_composed(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, kv_splits: Sequence[int],
                      causal: bool = False, scale: Optional[float] = None,
                      order: Optional[Sequence[int]] = None) -> torch.Tensor:
    """The same composition driven from Python through the primitives
    (rowmax -> combine_rowmax, accumulate -> combine_digits, finalize), the way
    a context-parallel caller would run it across devices."""
    scale = default_scale(Q.shape[3]) if scale is None else float(scale)
    bounds, lo = [], 0
    for n in kv_splits:
        bounds.append((lo, lo + int(n)))
        lo += int(n)
    order = list(range(len(bounds))) if order is None else list(order)
    m = None
    for s in order:
        part = rowmax(Q, K, bounds[s][0], bounds[s][1], causal, scale)
        m = part if m is None else combine_rowmax(m, part)
    num = den = None
    for s in order:
        n_, d_ = accumulate(Q, K, V, m, bounds[s][0], bounds[s][1], causal, scale)
        if num is None:
            num, den = n_, d_
        else:
            combine_digits(num, n_)
            combine_digits(den, d_)
    return finalize(num, den)
