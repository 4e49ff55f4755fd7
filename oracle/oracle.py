"""Python front end of the CPU oracle (TEST INFRASTRUCTURE ONLY).

Loads ``libdet_oracle.so`` (built from ``det_oracle.c`` with gcc) through
ctypes.  Only the test suite, the smoke check and the benchmark's CPU-baseline
leg may import this module; the GPU library never does.

The arithmetic lives in the C file; this module only marshals torch/numpy
arrays.  What the oracle computes is stated at the top of ``det_oracle.h``:
the det-attn page ("Method") for attention and the det-cross-entropy page
("Method") for the vocabulary-axis reduction.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "det_oracle.c")
_LIB = os.path.join(_HERE, "libdet_oracle.so")

NUM_DIGITS, NUM_ELO = 14, -298
DEN_DIGITS, DEN_ELO = 9, -149


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain C, OpenMP over independent rows)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-shared",
                               "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _Tensor(C.Structure):
    _fields_ = [("data", C.c_void_p), ("dtype", C.c_int32), ("B", C.c_int64), ("H", C.c_int64),
                ("S", C.c_int64), ("D", C.c_int64), ("sB", C.c_int64), ("sH", C.c_int64), ("sS", C.c_int64)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = C.CDLL(build())
        P, I64, I32, D = C.c_void_p, C.c_int64, C.c_int32, C.c_double
        T = C.POINTER(_Tensor)
        sig = {
            "ora_version": (I32, []),
            "ora_threads": (I32, []),
            "ora_exp_det": (D, [D]),
            "ora_log_det": (D, [D]),
            "ora_score": (C.c_float, [P, P, I64, D]),
            "ora_attn_rowmax_rows": (I32, [T, T, I64, P, I64, I64, I32, D, P]),
            "ora_attn_accumulate_rows": (I32, [T, T, T, I64, P, P, I64, I64, I32, D, P, P]),
            "ora_attn_finalize": (None, [P, P, I64, I64, P]),
            "ora_attn_backward": (I32, [T, T, T, T, I32, D, P, P, P]),
            "ora_digits_combine": (I32, [P, P, I64, I32, I32]),
            "ora_digits_to_double": (None, [P, I64, I32, I32, P]),
            "ora_double_to_digits": (I32, [P, I64, I32, I32, P]),
            "ora_ce_rowmax": (None, [P, I32, I64, I64, I64, I64, P]),
            "ora_ce_denom_digits": (None, [P, I32, I64, I64, P, I64, I64, P]),
            "ora_ce_finalize": (None, [P, P, I32, I64, I64, P, P, P, P]),
            "ora_ce_reduce": (None, [P, I64, I32, P]),
            "ora_ce_backward": (None, [P, I32, I64, I64, I64, P, P, P, P, I32, P, I64]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(_lib, name)
            fn.restype = res
            fn.argtypes = args
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _host_ptr(t: torch.Tensor):
    """(address of element 0, dtype code) for a CPU f32/bf16 tensor."""
    if t.device.type != "cpu":
        raise ValueError("oracle inputs must be CPU tensors")
    if t.dtype == torch.float32:
        return t.data_ptr(), 0
    if t.dtype == torch.bfloat16:
        return t.data_ptr(), 1
    raise ValueError("oracle inputs must be float32 or bfloat16")


def _tensor(t: torch.Tensor, keep: list) -> _Tensor:
    """Describe a [B,H,S,D] tensor with unit D stride (any other strides)."""
    if t.dim() != 4:
        raise ValueError("attention operands are [B, H, S, D]")
    if t.shape[3] > 1 and t.stride(3) != 1:
        raise ValueError("D stride must be 1")
    keep.append(t)
    ptr, code = _host_ptr(t)
    B, H, S, D = t.shape
    return _Tensor(ptr, code, B, H, S, D, t.stride(0), t.stride(1), t.stride(2))


def all_rows(B: int, H: int, S: int) -> np.ndarray:
    """Every (b, h, i) triplet in row-major order."""
    g = np.indices((B, H, S)).reshape(3, -1).T
    return np.ascontiguousarray(g, dtype=np.int64)


def default_scale(D: int) -> float:
    """RN64(1 / RN64(sqrt(D))), computed on the host."""
    return 1.0 / float(np.sqrt(np.float64(D)))


def threads() -> int:
    """Number of host threads the oracle's row loops use."""
    return int(lib().ora_threads())


def exp_det(t: float) -> float:
    return lib().ora_exp_det(float(t))


def log_det(x: float) -> float:
    return lib().ora_log_det(float(x))


def score(q: np.ndarray, k: np.ndarray, scale: float) -> float:
    q = np.ascontiguousarray(q, np.float32)
    k = np.ascontiguousarray(k, np.float32)
    return lib().ora_score(_ptr(q), _ptr(k), q.size, scale)


def attn_rowmax(Q, K, kv_lo=0, kv_hi=None, causal=False, scale=None, rows=None) -> np.ndarray:
    """Per-row f32 max score over keys [kv_lo, kv_hi). Shape [B,Hq,Sq] (or [n] with rows)."""
    kv_hi = K.shape[2] if kv_hi is None else kv_hi
    scale = default_scale(Q.shape[3]) if scale is None else scale
    keep = []
    r = all_rows(*Q.shape[:3]) if rows is None else np.ascontiguousarray(rows, np.int64)
    out = np.empty(len(r), np.float32)
    rc = lib().ora_attn_rowmax_rows(C.byref(_tensor(Q, keep)), C.byref(_tensor(K, keep)), len(r), _ptr(r),
                                    kv_lo, kv_hi, int(causal), scale, _ptr(out))
    if rc:
        raise ValueError("oracle: bad shapes or key range")
    return out.reshape(Q.shape[:3]) if rows is None else out


def attn_accumulate(Q, K, V, rowmax, kv_lo=0, kv_hi=None, causal=False, scale=None, rows=None):
    """Canonical (NUM [14,...,D], DEN [9,...]) digits of keys [kv_lo, kv_hi)."""
    kv_hi = K.shape[2] if kv_hi is None else kv_hi
    scale = default_scale(Q.shape[3]) if scale is None else scale
    keep = []
    r = all_rows(*Q.shape[:3]) if rows is None else np.ascontiguousarray(rows, np.int64)
    n, D = len(r), Q.shape[3]
    m = np.ascontiguousarray(np.asarray(rowmax, np.float32).reshape(-1))
    num = np.zeros((NUM_DIGITS, n, D), np.int64)
    den = np.zeros((DEN_DIGITS, n), np.int64)
    rc = lib().ora_attn_accumulate_rows(C.byref(_tensor(Q, keep)), C.byref(_tensor(K, keep)),
                                        C.byref(_tensor(V, keep)), n, _ptr(r), _ptr(m), kv_lo, kv_hi,
                                        int(causal), scale, _ptr(num), _ptr(den))
    if rc:
        raise ValueError("oracle: bad shapes, key range, or digit overflow")
    if rows is None:
        B, H, S = Q.shape[:3]
        return num.reshape(NUM_DIGITS, B, H, S, D), den.reshape(DEN_DIGITS, B, H, S)
    return num, den


def attn_finalize(num: np.ndarray, den: np.ndarray) -> np.ndarray:
    """f32 output with num's trailing shape ([..., D])."""
    D = num.shape[-1]
    n = den[0].size
    numc = np.ascontiguousarray(num, np.int64)
    denc = np.ascontiguousarray(den, np.int64)
    out = np.empty(n * D, np.float32)
    lib().ora_attn_finalize(_ptr(numc), _ptr(denc), n, D, _ptr(out))
    return out.reshape(num.shape[1:])


def det_attn(Q, K, V, causal=False, scale=None, rows=None, return_parts=False):
    """The whole path: global rowmax, exact digits over all keys, finalize."""
    m = attn_rowmax(Q, K, 0, K.shape[2], causal, scale, rows)
    num, den = attn_accumulate(Q, K, V, m, 0, K.shape[2], causal, scale, rows)
    out = attn_finalize(num, den)
    if return_parts:
        return out, m, num, den
    return out


def attn_backward(Q, K, V, dO, causal=False, scale=None):
    """(dQ, dK, dV) as f32 arrays shaped like Q, K, V: the backward reading
    stated in det_oracle.h (exact sums over the sequence axes)."""
    scale = default_scale(Q.shape[3]) if scale is None else scale
    if dO.dtype != torch.float32 or tuple(dO.shape) != tuple(Q.shape):
        raise ValueError("dO must be float32 shaped like Q")
    keep = []
    dq = np.zeros(tuple(Q.shape), np.float32)
    dk = np.zeros(tuple(K.shape), np.float32)
    dv = np.zeros(tuple(V.shape), np.float32)
    rc = lib().ora_attn_backward(C.byref(_tensor(Q, keep)), C.byref(_tensor(K, keep)), C.byref(_tensor(V, keep)),
                                 C.byref(_tensor(dO, keep)), int(causal), scale, _ptr(dq), _ptr(dk), _ptr(dv))
    if rc:
        raise ValueError("oracle: bad shapes")
    return dq, dk, dv


def digits_combine(acc: np.ndarray, part: np.ndarray, K: int, E_lo: int) -> np.ndarray:
    """canonical(acc + part); returns a new array."""
    a = np.ascontiguousarray(acc, np.int64).copy()
    p = np.ascontiguousarray(part, np.int64)
    n = a.size // K
    if lib().ora_digits_combine(_ptr(a), _ptr(p), n, K, E_lo):
        raise OverflowError("digit overflow")
    return a


def digits_to_double(digits: np.ndarray, K: int, E_lo: int) -> np.ndarray:
    d = np.ascontiguousarray(digits, np.int64)
    n = d.size // K
    out = np.empty(n, np.float64)
    lib().ora_digits_to_double(_ptr(d), n, K, E_lo, _ptr(out))
    return out.reshape(d.shape[1:])


def double_to_digits(x: np.ndarray, K: int, E_lo: int) -> np.ndarray:
    xs = np.ascontiguousarray(x, np.float64)
    out = np.zeros((K,) + xs.shape, np.int64)
    if lib().ora_double_to_digits(_ptr(xs), xs.size, K, E_lo, _ptr(out)):
        raise ValueError("value not representable in this digit format")
    return out


# ---------------------------------------------------------------- cross-entropy

def _logits(x: torch.Tensor):
    if x.dim() != 2 or (x.shape[1] > 1 and x.stride(1) != 1):
        raise ValueError("logits are [N, V] with unit column stride")
    ptr, code = _host_ptr(x)
    return x, ptr, code, x.stride(0)


def ce_rowmax(x: torch.Tensor, v_lo=0, v_hi=None) -> np.ndarray:
    arr, p, code, ld = _logits(x)
    N, V = x.shape
    v_hi = V if v_hi is None else v_hi
    out = np.empty(N, np.float32)
    lib().ora_ce_rowmax(p, code, N, ld, v_lo, v_hi, _ptr(out))
    return out


def ce_denom_digits(x: torch.Tensor, rowmax, v_lo=0, v_hi=None) -> np.ndarray:
    arr, p, code, ld = _logits(x)
    N, V = x.shape
    v_hi = V if v_hi is None else v_hi
    m = np.ascontiguousarray(rowmax, np.float32)
    den = np.zeros((DEN_DIGITS, N), np.int64)
    lib().ora_ce_denom_digits(p, code, N, ld, _ptr(m), v_lo, v_hi, _ptr(den))
    return den


def ce_finalize(den: np.ndarray, x: torch.Tensor, targets, rowmax):
    arr, p, code, ld = _logits(x)
    N = x.shape[0]
    t = np.ascontiguousarray(np.asarray(targets), np.int64)
    m = np.ascontiguousarray(rowmax, np.float32)
    d = np.ascontiguousarray(den, np.int64)
    loss = np.empty(N, np.float32)
    denom = np.empty(N, np.float64)
    lib().ora_ce_finalize(_ptr(d), p, code, N, ld, _ptr(t), _ptr(m), _ptr(loss), _ptr(denom))
    return loss, denom


def ce_forward(x: torch.Tensor, targets):
    """(loss [N] f32, rowmax [N] f32, denom [N] f64) over the whole vocabulary."""
    m = ce_rowmax(x)
    den = ce_denom_digits(x, m)
    loss, denom = ce_finalize(den, x, targets, m)
    return loss, m, denom


REDUCTIONS = {"none": 0, "mean": 1, "sum": 2}


def ce_reduce(loss: np.ndarray, reduction: str) -> np.ndarray:
    code = REDUCTIONS[reduction]
    l = np.ascontiguousarray(loss, np.float32)
    out = np.empty(len(l) if code == 0 else 1, np.float32)
    lib().ora_ce_reduce(_ptr(l), len(l), code, _ptr(out))
    return out if code == 0 else out[0]


def ce_backward(x: torch.Tensor, targets, rowmax, denom, grad_loss, reduction: str) -> np.ndarray:
    arr, p, code, ld = _logits(x)
    N, V = x.shape
    t = np.ascontiguousarray(np.asarray(targets), np.int64)
    m = np.ascontiguousarray(rowmax, np.float32)
    dn = np.ascontiguousarray(denom, np.float64)
    g = np.ascontiguousarray(np.asarray(grad_loss, np.float32).reshape(-1))
    grad = np.empty((N, V), np.float32)
    lib().ora_ce_backward(p, code, N, V, ld, _ptr(t), _ptr(m), _ptr(dn), _ptr(g), REDUCTIONS[reduction],
                          _ptr(grad), V)
    return grad
