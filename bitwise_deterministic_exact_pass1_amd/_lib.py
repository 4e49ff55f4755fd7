"""ctypes binding of libdet_attn.so (argument marshalling only).

Every computation happens in the HIP kernels behind the C ABI declared in
include/det_attn.h; this module converts torch tensors to descriptors, takes
the current HIP stream, allocates the workspace the library asks for, and
raises on a nonzero return code.  If the shared library is missing the import
fails loudly: there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdet_attn.so")

DET_F32, DET_BF16 = 0, 1
NUM_DIGITS, NUM_ELO, DEN_DIGITS, DEN_ELO = 14, -298, 9, -149

ERRORS = {-1: "DET_E_NULL", -2: "DET_E_SHAPE", -3: "DET_E_DTYPE", -4: "DET_E_STRIDE", -5: "DET_E_WORKSPACE",
          -6: "DET_E_HIP", -7: "DET_E_VALUE"}


class DetError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{ERRORS.get(code, code)}: {msg}")
        self.code = code


class Tensor(C.Structure):
    _fields_ = [("data", C.c_void_p), ("dtype", C.c_int32), ("B", C.c_int64), ("H", C.c_int64),
                ("S", C.c_int64), ("D", C.c_int64), ("sB", C.c_int64), ("sH", C.c_int64), ("sS", C.c_int64)]


class Out(C.Structure):
    _fields_ = [("data", C.c_void_p), ("sB", C.c_int64), ("sH", C.c_int64), ("sS", C.c_int64)]


# name -> (restype, argtypes); mirrors include/det_attn.h
_P, _I32, _I64, _D, _SZ = C.c_void_p, C.c_int32, C.c_int64, C.c_double, C.c_size_t
_T, _O = C.POINTER(Tensor), C.POINTER(Out)
SIGNATURES = {
    "det_digit_format": (C.c_int, [_I32, C.POINTER(_I32), C.POINTER(_I32)]),
    "det_last_error": (C.c_char_p, []),
    "det_profile_begin": (C.c_int, []),
    "det_profile_end": (_SZ, [C.c_char_p, _SZ]),
    "det_debug_force_generic": (C.c_int, [_I32]),
    "det_debug_checks": (C.c_int, [_I32]),
    "det_debug_pass2_layout": (C.c_int, [_I32]),
    "det_debug_score_source": (C.c_int, [_I32]),
    "det_attn_workspace_size": (_SZ, [_T, _T, _T, _I32]),
    "det_attn": (C.c_int, [_T, _T, _T, _I32, _D, _O, _P, _SZ, _P]),
    "det_attn_noalloc": (C.c_int, [_T, _T, _T, _I32, _D, _O, _P]),
    "det_attn_stats": (C.c_int, [_T, _T, _T, _I32, _D, _O, _P, _P, _P, _SZ, _P]),
    "det_attn_backward_workspace_size": (_SZ, [_T, _T, _T, _I32]),
    "det_attn_backward": (C.c_int, [_T, _T, _T, _T, _T, _P, _P, _I32, _D, _O, _O, _O, _P, _SZ, _P]),
    "det_attn_rowmax_workspace_size": (_SZ, [_T, _T, _I64, _I64, _I64, _I64]),
    "det_attn_rowmax": (C.c_int, [_T, _T, _I64, _I64, _I64, _I64, _I32, _D, _P, _P, _SZ, _P]),
    "det_attn_accumulate_workspace_size": (_SZ, [_T, _T, _T, _I64, _I64, _I64, _I64]),
    "det_attn_accumulate": (C.c_int, [_T, _T, _T, _P, _I64, _I64, _I64, _I64, _I32, _D, _P, _P, _I32, _P, _SZ,
                                      _P]),
    "det_rowmax_combine": (C.c_int, [_P, _P, _I64, _P]),
    "det_digits_combine": (C.c_int, [_P, _P, _I64, _I32, _P]),
    "det_digits_normalize": (C.c_int, [_P, _I64, _I32, _P]),
    "det_attn_finalize": (C.c_int, [_P, _P, _I64, _I64, _I64, _I64, _O, _P]),
    "det_attn_sharded_workspace_size": (_SZ, [_T, _T, _T, _P, _I32, _I32]),
    "det_attn_sharded": (C.c_int, [_T, _T, _T, _P, _I32, _P, _I32, _D, _O, _P, _SZ, _P]),
    "det_ce_rowmax": (C.c_int, [_P, _I32, _I64, _I64, _I64, _I64, _P, _P]),
    "det_ce_denom_digits": (C.c_int, [_P, _I32, _I64, _I64, _P, _I64, _I64, _P, _I32, _P]),
    "det_ce_finalize": (C.c_int, [_P, _P, _I32, _I64, _I64, _I64, _P, _P, _P, _P, _P]),
    "det_ce_forward_workspace_size": (_SZ, [_I64]),
    "det_ce_forward": (C.c_int, [_P, _I32, _I64, _I64, _I64, _P, _P, _P, _P, _P, _SZ, _P]),
    "det_ce_reduce_workspace_size": (_SZ, [_I64]),
    "det_ce_reduce": (C.c_int, [_P, _I64, _I32, _P, _P, _SZ, _P]),
    "det_ce_backward": (C.c_int, [_P, _I32, _I64, _I64, _I64, _I64, _P, _P, _P, _P, _I32, _P, _I64, _P]),
}

_lib = None


def lib() -> C.CDLL:
    """Load libdet_attn.so (raises ImportError when it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m bitwise_deterministic_exact_pass1_amd.build`")
        h = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


def force_generic(on: bool) -> None:
    """Testing aid: send every tile through the library's generic exact path
    (bit-identical results) until switched off again."""
    check(lib().det_debug_force_generic(int(bool(on))))


def input_checks(on: bool) -> None:
    """Verify caller-supplied row maxima (accumulate) and targets (cross-
    entropy) on the device; calls then wait for their stream and raise on a
    violation.  Off by default."""
    check(lib().det_debug_checks(int(bool(on))))


def pass2_layout(mode: int) -> None:
    """Testing aid: pick pass 2's kernel layout for bf16 head dims <= 128
    (0: by key-range length, 1: eight waves each making weights and
    multiplying, 2: split weight-making and multiplying waves); the outputs
    are the same bits either way."""
    check(lib().det_debug_pass2_layout(int(mode)))


def score_source(mode: int) -> None:
    """Testing aid: how pass 2 gets bf16 scores (0: kept when the workspace
    allows, 1: kept, 2: recomputed from the digit rows); the outputs are the
    same bits either way."""
    check(lib().det_debug_score_source(int(mode)))


def profile_begin() -> None:
    check(lib().det_profile_begin())


def profile_end() -> dict:
    """{kernel: (launches, total_ms)} for the launches since profile_begin()."""
    buf = C.create_string_buffer(1 << 16)
    lib().det_profile_end(buf, len(buf))
    return _parse(buf.value.decode())


def _parse(text: str) -> dict:
    out = {}
    for line in text.splitlines():
        name, cnt, ms = line.split()
        out[name] = (int(cnt), float(ms))
    return out


def check(rc: int) -> None:
    if rc != 0:
        raise DetError(rc, lib().det_last_error().decode())
