"""det_attn_noalloc (the entry point that allocates nothing: its scratch is
the library's fixed device array) against det_attn with a caller workspace,
bit for bit, through the C ABI: two calls in a row, the second smaller, then
a problem whose smallest chunk does not fit the fixed scratch."""
import ctypes as C
import sys

import numpy as np
import pytest
import torch

from bitwise_deterministic_exact_pass1_amd import _lib as L
from bitwise_deterministic_exact_pass1_amd import workloads as W

pytestmark = pytest.mark.gpu


def _desc(t):
    B, H, S, D = t.shape
    return L.Tensor(t.data_ptr(), L.DET_BF16 if t.dtype == torch.bfloat16 else L.DET_F32, B, H, S, D,
                    t.stride(0), t.stride(1), t.stride(2))


def _noalloc(q, k, v, causal, scale):
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device=q.device)
    o = L.Out(out.data_ptr(), out.stride(0), out.stride(1), out.stride(2))
    lib = L.lib()
    rc = lib.det_attn_noalloc(C.byref(_desc(q)), C.byref(_desc(k)), C.byref(_desc(v)), int(causal), scale,
                              C.byref(o), torch.cuda.current_stream().cuda_stream)
    return rc, out


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_noalloc_matches_det_attn_two_calls(dtype):
    assert torch.cuda.is_available()
    from bitwise_deterministic_exact_pass1_amd import attention as A
    cases = [(61, 2, 8, 2, 700, 128, True), (62, 1, 4, 2, 90, 40, False)]  # the second call is smaller
    for seed, B, Hq, Hkv, S, D, causal in cases:
        print(f"noalloc: seed {seed} B={B} Hq={Hq} Hkv={Hkv} S={S} D={D} causal={causal} {dtype}", file=sys.stderr,
              flush=True)
        q, k, v = [t.cuda() for t in W.attn_inputs(seed, B, Hq, Hkv, S, S, D, dtype)]
        scale = W.default_scale(D)
        rc, got = _noalloc(q, k, v, causal, scale)
        torch.cuda.synchronize()
        assert rc == 0, L.lib().det_last_error().decode()
        ref = A.det_attn(q, k, v, causal, scale)
        assert torch.equal(got.view(torch.int32), ref.view(torch.int32))


def test_noalloc_rejects_a_problem_larger_than_its_scratch():
    # 32 query rows against 2^20 keys of 512 heads need far more than the fixed scratch;
    # the call fails before launching anything (the tensors are never read)
    q = torch.empty(1, 512, 32, 128, dtype=torch.bfloat16, device="cuda")
    kv = torch.empty(1, 512, 1 << 20, 128, dtype=torch.bfloat16, device="meta")
    k = L.Tensor(0x1000, L.DET_BF16, 1, 512, 1 << 20, 128, *kv.stride()[:3])
    o = L.Out(q.data_ptr(), 32 * 128 * 512, 32 * 128, 128)
    rc = L.lib().det_attn_noalloc(C.byref(_desc(q)), C.byref(k), C.byref(k), 0, 0.1, C.byref(o), None)
    assert rc == -5
    assert b"fixed scratch" in L.lib().det_last_error()
