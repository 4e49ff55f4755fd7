"""The C ABI without a GPU: the library loads, exports every function that
include/det_attn.h declares, and rejects bad arguments on the host before any
HIP call (the checks are synchronous and need no device)."""
import ctypes as C
import os
import re

import pytest

from bitwise_deterministic_exact_pass1_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "det_attn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(det_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        from bitwise_deterministic_exact_pass1_amd import build
        build.build()
    return L.lib()


def test_every_declared_symbol_is_exported_and_bound(lib):
    names = _declared()
    assert len(names) >= 20
    for n in names:
        assert hasattr(lib, n), n
        assert n in L.SIGNATURES, n  # the binding declares every entry point


def test_digit_format(lib):
    n, e = C.c_int32(), C.c_int32()
    assert lib.det_digit_format(0, C.byref(n), C.byref(e)) == 0 and (n.value, e.value) == (14, -298)
    assert lib.det_digit_format(1, C.byref(n), C.byref(e)) == 0 and (n.value, e.value) == (9, -149)
    assert lib.det_digit_format(2, C.byref(n), C.byref(e)) == -7


def _t(B=1, H=2, S=8, D=16, dtype=L.DET_BF16, data=0x1000, strides=None):
    sB, sH, sS = strides or (H * S * D, S * D, D)
    return L.Tensor(data, dtype, B, H, S, D, sB, sH, sS)


def _call_attn(lib, q, k, v, causal=0, ws=0x10000, nbytes=1 << 30, out=True):
    o = L.Out(0x2000, 2 * 8 * 16, 8 * 16, 16) if out else None
    return lib.det_attn(C.byref(q) if q else None, C.byref(k), C.byref(v), causal, 0.25,
                        C.byref(o) if o else None, ws, nbytes, None)


def test_attention_argument_errors(lib):
    q, k, v = _t(), _t(H=1), _t(H=1)
    assert _call_attn(lib, None, k, v) == -1
    assert b"q" in lib.det_last_error()
    assert _call_attn(lib, q, k, v, out=False) == -1
    assert _call_attn(lib, _t(D=257), _t(H=1, D=257), _t(H=1, D=257)) == -2
    assert _call_attn(lib, _t(D=0), _t(H=1, D=0), _t(H=1, D=0)) == -2
    assert _call_attn(lib, _t(H=3), k, v) == -2 or _call_attn(lib, _t(H=3), _t(H=2), _t(H=2)) == -2
    assert _call_attn(lib, _t(S=8), _t(H=1, S=9), _t(H=1, S=9), causal=1) == -2
    assert _call_attn(lib, q, _t(H=1, dtype=L.DET_F32), _t(H=1, dtype=L.DET_F32)) == -3
    assert _call_attn(lib, _t(dtype=5), _t(H=1, dtype=5), _t(H=1, dtype=5)) == -3
    assert _call_attn(lib, q, k, _t(H=1, S=7)) == -2
    assert _call_attn(lib, _t(strides=(-1, 16, 16)), k, v) == -4
    assert _call_attn(lib, q, k, v, ws=0) == -5
    assert _call_attn(lib, q, k, v, ws=0x10001) == -5
    assert _call_attn(lib, q, k, v, nbytes=16) == -5


def test_range_and_split_errors(lib):
    q, k, v = _t(), _t(H=1), _t(H=1)
    rm = lib.det_attn_rowmax(C.byref(q), C.byref(k), 0, 8, 3, 2, 0, 1.0, 0x3000, 0x10000, 1 << 30, None)
    assert rm == -2
    assert lib.det_attn_rowmax(C.byref(q), C.byref(k), 0, 8, 0, 9, 0, 1.0, 0x3000, 0x10000, 1 << 30, None) == -2
    # query ranges: lo > hi, below 0, past Sq
    for qlo, qhi in [(5, 4), (-1, 4), (0, 9)]:
        assert lib.det_attn_rowmax(C.byref(q), C.byref(k), qlo, qhi, 0, 8, 0, 1.0, 0x3000, 0x10000, 1 << 30,
                                   None) == -2
        assert lib.det_attn_accumulate(C.byref(q), C.byref(k), C.byref(v), 0x4000, qlo, qhi, 0, 8, 0, 1.0, 0x5000,
                                       0x6000, 0, 0x10000, 1 << 30, None) == -2
        assert lib.det_attn_rowmax_workspace_size(C.byref(q), C.byref(k), qlo, qhi, 0, 8) == 0
        assert lib.det_attn_accumulate_workspace_size(C.byref(q), C.byref(k), C.byref(v), qlo, qhi, 0, 8) == 0
    assert lib.det_attn_accumulate(C.byref(q), C.byref(k), C.byref(v), 0x4000, 0, 8, 0, 8, 0, 1.0, None, 0x5000, 0,
                                   0x10000, 1 << 30, None) == -1
    # an empty query range needs no pointer, no workspace and launches nothing
    assert lib.det_attn_rowmax(C.byref(q), C.byref(k), 4, 4, 0, 8, 0, 1.0, None, None, 0, None) == 0
    assert lib.det_attn_accumulate(C.byref(q), C.byref(k), C.byref(v), None, 4, 4, 0, 8, 0, 1.0, None, None, 0,
                                   None, 0, None) == 0
    # a null rowmax with rows to compute
    assert lib.det_attn_rowmax(C.byref(q), C.byref(k), 2, 4, 0, 8, 0, 1.0, None, 0x10000, 1 << 30, None) == -1
    o = L.Out(0x2000, 256, 128, 16)
    bad = (C.c_int64 * 2)(4, 3)
    assert lib.det_attn_sharded(C.byref(q), C.byref(k), C.byref(v), bad, 2, None, 0, 1.0, C.byref(o), 0x10000,
                                1 << 30, None) == -7
    good = (C.c_int64 * 2)(4, 4)
    perm = (C.c_int32 * 2)(1, 1)
    assert lib.det_attn_sharded(C.byref(q), C.byref(k), C.byref(v), good, 2, perm, 0, 1.0, C.byref(o), 0x10000,
                                1 << 30, None) == -7
    assert lib.det_digits_combine(0x1000, 0x2000, 10, 7, None) == -7
    assert lib.det_digits_normalize(0x1000, 10, 7, None) == -7
    assert lib.det_digits_normalize(0x1000, -1, 9, None) == -2
    assert lib.det_digits_normalize(None, 10, 14, None) == -1
    assert lib.det_digits_normalize(None, 0, 9, None) == 0
    assert lib.det_attn_finalize(0x1000, 0x2000, 1, 1, 4, 300, C.byref(o), None) == -2


def test_workspace_sizes_are_host_only(lib):
    q, k, v = _t(B=2, H=8, S=1024, D=128), _t(B=2, H=2, S=1024, D=128), _t(B=2, H=2, S=1024, D=128)
    n = lib.det_attn_workspace_size(C.byref(q), C.byref(k), C.byref(v), 1)
    assert n > 0 and n % 256 == 0
    splits = (C.c_int64 * 4)(256, 256, 256, 256)
    ns = lib.det_attn_sharded_workspace_size(C.byref(q), C.byref(k), C.byref(v), splits, 4, 1)
    assert ns > 0
    assert lib.det_attn_rowmax_workspace_size(C.byref(q), C.byref(k), 0, 1024, 0, 1024) > 0
    assert lib.det_attn_accumulate_workspace_size(C.byref(q), C.byref(k), C.byref(v), 0, 1024, 0, 512) > 0
    # fewer query rows never need more workspace
    assert (lib.det_attn_accumulate_workspace_size(C.byref(q), C.byref(k), C.byref(v), 100, 200, 0, 512)
            <= lib.det_attn_accumulate_workspace_size(C.byref(q), C.byref(k), C.byref(v), 0, 1024, 0, 512))
    # an invalid descriptor yields 0 rather than a crash
    assert lib.det_attn_workspace_size(None, C.byref(k), C.byref(v), 0) == 0


def _call_bwd(lib, q, k, v, o, g, rowmax=0x6000, den=0x7000, out=True, ws=0x10000, nbytes=1 << 30):
    d = L.Out(0x2000, 2 * 8 * 16, 8 * 16, 16) if out else None
    return lib.det_attn_backward(C.byref(q), C.byref(k), C.byref(v), C.byref(o), C.byref(g), rowmax, den, 0, 0.25,
                                 C.byref(d) if d else None, C.byref(d) if d else None, C.byref(d) if d else None,
                                 ws, nbytes, None)


def test_backward_argument_errors(lib):
    q, k, v = _t(), _t(H=1), _t(H=1)
    o, g = _t(dtype=L.DET_F32), _t(dtype=L.DET_F32)
    assert _call_bwd(lib, q, k, v, _t(dtype=L.DET_BF16), g) == -3  # o must be f32
    assert _call_bwd(lib, q, k, v, o, _t(S=7, dtype=L.DET_F32)) == -2  # dout shaped like q
    assert _call_bwd(lib, q, k, v, o, g, rowmax=0) == -1
    assert _call_bwd(lib, q, k, v, o, g, out=False) == -1
    assert _call_bwd(lib, q, k, v, o, g, ws=0) == -5
    assert _call_bwd(lib, q, k, _t(H=1, S=9), o, g) == -2
    assert lib.det_attn_backward_workspace_size(C.byref(q), C.byref(k), C.byref(v), 0) > 0
    so = L.Out(0x2000, 256, 128, 16)
    assert lib.det_attn_stats(C.byref(q), C.byref(k), C.byref(v), 0, 0.25, C.byref(so), None, 0x7000, 0x10000,
                              1 << 30, None) == -1


def test_cross_entropy_argument_errors(lib):
    assert lib.det_ce_rowmax(0x1000, 3, 4, 10, 0, 10, 0x2000, None) == -3
    assert lib.det_ce_rowmax(0x1000, 1, 4, 10, 0, 11, 0x2000, None) == -2
    assert lib.det_ce_rowmax(None, 1, 4, 10, 0, 10, 0x2000, None) == -1
    assert lib.det_ce_denom_digits(0x1000, 1, 4, 10, None, 0, 10, 0x3000, 0, None) == -1
    assert lib.det_ce_finalize(0x1, 0x1000, 1, 4, 10, 8, 0x2, 0x3, 0x4, 0x5, None) == -4
    assert lib.det_ce_forward(0x1000, 1, 4, 10, 10, None, 0x1, 0x2, 0x3, None, 0, None) == -1
    assert lib.det_ce_reduce(0x1000, 4, 3, 0x2000, None, 0, None) == -7
    assert lib.det_ce_backward(0x1000, 1, 4, 10, 10, 0, 0x1, 0x2, 0x3, 0x4, 1, 0x5, 9, None) == -4
    assert lib.det_ce_backward(0x1000, 1, 4, 10, 10, 0, 0x1, 0x2, 0x3, 0x4, 5, 0x5, 10, None) == -7
    assert lib.det_ce_backward(0x1000, 1, 4, 10, 10, -3, 0x1, 0x2, 0x3, 0x4, 1, 0x5, 10, None) == -7
    assert lib.det_ce_backward(0x1000, 1, 4, 10, 10, 0, None, 0x2, 0x3, 0x4, 1, 0x5, 10, None) == -1


def _no_device():
    import torch
    return torch.cuda.device_count() == 0  # counts devices without initialising one


# (B, Hq, Hkv, S, D, causal) of the workloads; the key splits used with them
_LAYOUT_CASES = [
    (1, 2, 2, 128, 64, 0, [32] * 4),
    (2, 8, 2, 1024, 128, 1, [64] * 16),
    (1, 32, 8, 8192, 128, 1, [1024] * 8),
    (1, 32, 8, 2048, 256, 1, [256] * 8),
    (1, 56, 56, 37810, 128, 0, [64] * 590 + [50]),
]


@pytest.fixture
def score_source(lib, request):
    """The score-source testing switch, reset to its default afterwards."""
    assert lib.det_debug_score_source(request.param) == 0
    yield request.param
    assert lib.det_debug_score_source(0) == 0


@pytest.mark.skipif(not _no_device(), reason="passes dummy device pointers: only where no device exists")
@pytest.mark.parametrize("score_source", [0, 1, 2], indirect=True)
@pytest.mark.parametrize("dtype", [L.DET_F32, L.DET_BF16])
@pytest.mark.parametrize("case", _LAYOUT_CASES, ids=lambda c: "x".join(map(str, c[:5])))
def test_workspace_layout_fits_the_reported_size(lib, case, dtype, score_source):
    """Each entry point carves its workspace on the host before it launches
    anything; given exactly the size its *_workspace_size reports, it must get
    past that (and then fail at its first HIP call, there being no device)
    rather than report that its layout outgrew the workspace.  For each way
    pass 2 may get bf16 scores (kept, recomputed, or chosen by size)."""
    B, Hq, Hkv, S, D, causal, splits = case
    q = _t(B=B, H=Hq, S=S, D=D, dtype=dtype, data=0x100000)
    k = _t(B=B, H=Hkv, S=S, D=D, dtype=dtype, data=0x200000)
    v = _t(B=B, H=Hkv, S=S, D=D, dtype=dtype, data=0x300000)
    o = L.Out(0x400000, Hq * S * D, S * D, D)
    ws = 0x10000000
    n = lib.det_attn_workspace_size(C.byref(q), C.byref(k), C.byref(v), causal)
    rc = lib.det_attn(C.byref(q), C.byref(k), C.byref(v), causal, 0.125, C.byref(o), ws, n, None)
    assert rc == -6, (rc, lib.det_last_error())
    sp = (C.c_int64 * len(splits))(*splits)
    n = lib.det_attn_sharded_workspace_size(C.byref(q), C.byref(k), C.byref(v), sp, len(splits), causal)
    rc = lib.det_attn_sharded(C.byref(q), C.byref(k), C.byref(v), sp, len(splits), None, causal, 0.125,
                              C.byref(o), ws, n, None)
    assert rc == -6, (rc, lib.det_last_error())
    lo, hi = S // 4, S // 4 + splits[0]
    for qlo, qhi in [(0, S), (S // 3, S // 3 + 40)]:
        n = lib.det_attn_rowmax_workspace_size(C.byref(q), C.byref(k), qlo, qhi, lo, hi)
        rc = lib.det_attn_rowmax(C.byref(q), C.byref(k), qlo, qhi, lo, hi, causal, 0.125, 0x500000, ws, n, None)
        assert rc == -6, (rc, lib.det_last_error())
        n = lib.det_attn_accumulate_workspace_size(C.byref(q), C.byref(k), C.byref(v), qlo, qhi, lo, hi)
        rc = lib.det_attn_accumulate(C.byref(q), C.byref(k), C.byref(v), 0x500000, qlo, qhi, lo, hi, causal, 0.125,
                                     0x600000, 0x700000, 0, ws, n, None)
        assert rc == -6, (rc, lib.det_last_error())
    n = lib.det_attn_workspace_size(C.byref(q), C.byref(k), C.byref(v), causal)
    rc = lib.det_attn_stats(C.byref(q), C.byref(k), C.byref(v), causal, 0.125, C.byref(o), 0x500000, 0x600000, ws,
                            n, None)
    assert rc == -6, (rc, lib.det_last_error())
    of = _t(B=B, H=Hq, S=S, D=D, dtype=L.DET_F32, data=0x400000)
    n = lib.det_attn_backward_workspace_size(C.byref(q), C.byref(k), C.byref(v), causal)
    rc = lib.det_attn_backward(C.byref(q), C.byref(k), C.byref(v), C.byref(of), C.byref(of), 0x500000, 0x600000,
                               causal, 0.125, C.byref(o), C.byref(o), C.byref(o), ws, n, None)
    assert rc == -6, (rc, lib.det_last_error())


def test_testing_switches_reject_unknown_modes(lib):
    """The pass-2 testing switches take modes 0-2 and refuse others with
    DET_E_VALUE, leaving the current mode as it was."""
    for fn in (lib.det_debug_score_source, lib.det_debug_pass2_layout):
        assert fn(3) == -7 and fn(-1) == -7  # DET_E_VALUE
        for m in (2, 1, 0):
            assert fn(m) == 0
