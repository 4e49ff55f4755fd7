"""GPU parity of the attention backward (exact sums over the sequence axes)
against the CPU oracle, bit for bit, plus the forward's per-row statistics it
consumes, key-order invariance and the autograd wrapper.  Inputs come from the
seeded generators in workloads.py; the upstream gradient is N(0,1) f32."""
import sys

import numpy as np
import pytest
import torch

from bitwise_deterministic_exact_pass1_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def A():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    from bitwise_deterministic_exact_pass1_amd import attention
    return attention


def say(msg):
    print(msg, file=sys.stderr, flush=True)


def bits(x):
    if isinstance(x, torch.Tensor):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(x, np.float32).view(np.uint32)


def assert_bits_equal(a, b, what):
    ua, ub = bits(a), bits(b)
    if not np.array_equal(ua, ub):
        bad = np.argwhere(ua != ub)
        raise AssertionError(f"{what}: {len(bad)} of {ua.size} differ; first at {bad[0].tolist()}")


def upstream(seed, shape):
    return torch.randn(*shape, generator=torch.Generator().manual_seed(seed))


def gpu_backward(A, q, k, v, dO, causal, scale):
    Q, K, V = q.cuda(), k.cuda(), v.cuda()
    out, m, den = A.det_attn_with_stats(Q, K, V, causal, scale)
    return A.det_attn_backward(Q, K, V, out, dO.cuda(), m, den, causal, scale)


CASES = [
    # (seed, B, Hq, Hkv, S_q, S_kv, D, dtype, causal)
    (901, 1, 4, 2, 40, 40, 16, torch.float32, True),
    (902, 1, 4, 2, 40, 40, 16, torch.float32, False),
    (903, 1, 4, 2, 72, 72, 64, torch.bfloat16, True),
    (904, 2, 2, 1, 33, 50, 64, torch.bfloat16, False),
    (905, 1, 2, 2, 45, 45, 3, torch.bfloat16, True),
    (906, 1, 2, 1, 37, 37, 100, torch.float32, True),
    (907, 1, 2, 2, 24, 24, 256, torch.bfloat16, False),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"s{c[0]}-D{c[6]}-{str(c[7])[6:]}-{'c' if c[8] else 'n'}")
def test_backward_bit_exact(A, oracle, case):
    seed, B, Hq, Hkv, Sq, Skv, D, dtype, causal = case
    q, k, v = W.attn_inputs(seed, B, Hq, Hkv, Sq, Skv, D, dtype)
    dO = upstream(seed + 1, (B, Hq, Sq, D))
    scale = W.default_scale(D)
    say(f"backward {case}: oracle")
    ref = oracle.attn_backward(q, k, v, dO, causal, scale)
    say("backward: gpu")
    got = gpu_backward(A, q, k, v, dO, causal, scale)
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        assert_bits_equal(a, b, name)


def test_backward_gqa_causal_several_tiles(A, oracle):
    """B=2 Hq=8 Hkv=2 S=200 D=128 bf16 causal: many 16-row and 16-key tiles,
    ragged at both ends, four query heads per key head."""
    q, k, v = W.attn_inputs(910, 2, 8, 2, 200, 200, 128, torch.bfloat16)
    dO = upstream(911, (2, 8, 200, 128))
    scale = W.default_scale(128)
    say("backward gqa S=200: oracle")
    ref = oracle.attn_backward(q, k, v, dO, True, scale)
    got = gpu_backward(A, q, k, v, dO, True, scale)
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        assert_bits_equal(a, b, name)


def test_forward_stats(A, oracle):
    """det_attn_with_stats: the same output as det_attn, the oracle's row
    maxima, and RN64 of the oracle's exact denominators."""
    q, k, v = W.attn_inputs(912, 1, 4, 2, 130, 130, 64, torch.bfloat16)
    scale = W.default_scale(64)
    Q, K, V = q.cuda(), k.cuda(), v.cuda()
    out, m, den = A.det_attn_with_stats(Q, K, V, True, scale)
    assert torch.equal(out, A.det_attn(Q, K, V, True, scale))
    ref, rm, num, dd = oracle.det_attn(q, k, v, True, scale, return_parts=True)
    assert_bits_equal(m, rm, "rowmax")
    den_ref = oracle.digits_to_double(dd.reshape(dd.shape[0], -1), oracle.DEN_DIGITS, oracle.DEN_ELO)
    assert np.array_equal(den.cpu().numpy().reshape(-1), den_ref)


def test_backward_key_permutation_invariance(A):
    """Non-causal: permuting K/V rows permutes dK/dV and leaves dQ's bits."""
    q, k, v = W.attn_inputs(913, 1, 4, 2, 64, 96, 32, torch.bfloat16)
    dO = upstream(914, (1, 4, 64, 32))
    scale = W.default_scale(32)
    base = gpu_backward(A, q, k, v, dO, False, scale)
    p = torch.randperm(96, generator=torch.Generator().manual_seed(915))
    dq, dk, dv = gpu_backward(A, q, k[:, :, p].contiguous(), v[:, :, p].contiguous(), dO, False, scale)
    assert torch.equal(dq, base[0])
    assert torch.equal(dk, base[1][:, :, p.cuda()])
    assert torch.equal(dv, base[2][:, :, p.cuda()])


def test_autograd_wrapper(A):
    q, k, v = W.attn_inputs(916, 1, 4, 2, 48, 48, 32, torch.bfloat16)
    G = upstream(917, (1, 4, 48, 32)).cuda()
    scale = W.default_scale(32)
    Q, K, V = [t.cuda().requires_grad_() for t in (q, k, v)]
    out = A.det_attn_autograd(Q, K, V, True, scale)
    (out * G).sum().backward()
    dq, dk, dv = gpu_backward(A, q, k, v, G.cpu(), True, scale)
    assert torch.equal(Q.grad, dq.to(torch.bfloat16))
    assert torch.equal(K.grad, dk.to(torch.bfloat16))
    assert torch.equal(V.grad, dv.to(torch.bfloat16))


def test_backward_small_workspace_row_chunks(A):
    """The smallest workspace the library accepts (the size of one 32-row
    chunk, read from its DET_E_WORKSPACE message) makes it take the query rows
    in chunks of 32 (dK and dV keep adding into the same digits, dQ is
    finished chunk by chunk); the gradients must be the same bits."""
    import re
    import ctypes as C
    from bitwise_deterministic_exact_pass1_amd import _lib
    q, k, v = W.attn_inputs(918, 2, 8, 2, 200, 200, 128, torch.bfloat16)
    dO = upstream(919, (2, 8, 200, 128)).cuda()
    scale = W.default_scale(128)
    Q, K, V = q.cuda(), k.cuda(), v.cuda()
    out, m, den = A.det_attn_with_stats(Q, K, V, True, scale)
    ref = A.det_attn_backward(Q, K, V, out, dO, m, den, True, scale)
    L = _lib.lib()
    dq_, dk_, dv_ = A._desc(Q), A._desc(K), A._desc(V)
    full = L.det_attn_backward_workspace_size(C.byref(dq_), C.byref(dk_), C.byref(dv_), 1)
    g = [torch.empty_like(t, dtype=torch.float32) for t in (Q, K, V)]
    rc = L.det_attn_backward(C.byref(dq_), C.byref(dk_), C.byref(dv_), C.byref(A._desc(out)), C.byref(A._desc(dO)),
                             m.data_ptr(), den.data_ptr(), 1, scale, C.byref(A._out(g[0])), C.byref(A._out(g[1])),
                             C.byref(A._out(g[2])), 256, 256, A._stream(Q))
    assert _lib.ERRORS[rc] == "DET_E_WORKSPACE"  # a host-side check: nothing was launched
    small = int(re.search(r"need at least (\d+)", L.det_last_error().decode()).group(1))
    assert small < full
    ws = torch.empty(small + 256, dtype=torch.uint8, device=Q.device)
    addr = (ws.data_ptr() + 255) & ~255
    say(f"backward with {small} of {full} workspace bytes")
    _lib.check(L.det_attn_backward(C.byref(dq_), C.byref(dk_), C.byref(dv_), C.byref(A._desc(out)),
                                   C.byref(A._desc(dO)), m.data_ptr(), den.data_ptr(), 1, scale,
                                   C.byref(A._out(g[0])), C.byref(A._out(g[1])), C.byref(A._out(g[2])), addr, small,
                                   A._stream(Q)))
    for a, b in zip(g, ref):
        assert torch.equal(a, b)


def _backward_both_paths(A, q, k, v, dO, causal, scale):
    """The gradients with the matrix-core sums, then with every tile forced
    onto the per-term digit sums (the library's testing switch)."""
    from bitwise_deterministic_exact_pass1_amd import _lib
    fast = gpu_backward(A, q, k, v, dO, causal, scale)
    _lib.force_generic(True)
    try:
        slow = gpu_backward(A, q, k, v, dO, causal, scale)
    finally:
        _lib.force_generic(False)
    return fast, slow


@pytest.mark.parametrize("shape", [
    (920, 2, 8, 2, 200, 200, 128, torch.bfloat16, True),
    (921, 1, 4, 1, 70, 130, 48, torch.bfloat16, False),
    (922, 1, 2, 2, 65, 65, 256, torch.bfloat16, True),
    (923, 1, 4, 2, 96, 96, 40, torch.float32, True),
], ids=["gqa-c-d128", "rect-n-d48", "d256-c", "f32-c-d40"])
def test_backward_matrix_core_and_per_term_sums_bit_identical(A, shape):
    seed, B, Hq, Hkv, Sq, Skv, D, dtype, causal = shape
    q, k, v = W.attn_inputs(seed, B, Hq, Hkv, Sq, Skv, D, dtype)
    dO = upstream(seed + 50, (B, Hq, Sq, D))
    say(f"backward both paths {shape}")
    fast, slow = _backward_both_paths(A, q, k, v, dO, causal, W.default_scale(D))
    for name, a, b in zip(("dq", "dk", "dv"), fast, slow):
        assert_bits_equal(a, b, name)


def test_backward_wide_ranges_mix_the_paths(A, oracle):
    """Single entries far below their column's range (a Q entry scaled by
    2^-60, a K entry by 2^-30, an upstream entry by 2^-40) make one column
    group of dK, dQ and dV need more digits than the matrix-core sums hold, so
    those tiles take the per-term sums while the other column groups stay on
    the matrix cores; all must match the oracle."""
    q, k, v = W.attn_inputs(930, 1, 4, 2, 100, 100, 64, torch.bfloat16)
    q[0, 1, 7, 5] = q[0, 1, 7, 5] * 2.0 ** -60
    k[0, 0, 40, 9] = k[0, 0, 40, 9] * 2.0 ** -30
    dO = upstream(931, (1, 4, 100, 64))
    dO[0, 0, 90, 3] *= 2.0 ** -40
    dO[0, 2, 11, :] *= 8.0
    scale = W.default_scale(64)
    say("backward wide ranges: oracle")
    ref = oracle.attn_backward(q, k, v, dO, True, scale)
    got = gpu_backward(A, q, k, v, dO, True, scale)
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        assert_bits_equal(a, b, name)


def test_backward_full_bench_size_both_paths_and_fp64(A):
    """The bench workload (B=2 Hq=8 Hkv=2 S=1024 D=128 bf16 causal, N(0,1) f32
    upstream gradient), too large for the oracle: the matrix-core sums and the
    per-term digit sums (two independent exact arithmetics) must give the same
    bits, and every gradient must lie within f32 rounding of fp64 autograd
    (2^-20 of the gradient scale, as the oracle's own pin)."""
    q, k, v = W.attn_inputs(2, 2, 8, 2, 1024, 1024, 128, torch.bfloat16)
    dO = upstream(4242, (2, 8, 1024, 128))
    scale = W.default_scale(128)
    say("backward at the bench size: both paths")
    fast, slow = _backward_both_paths(A, q, k, v, dO, True, scale)
    for name, a, b in zip(("dq", "dk", "dv"), fast, slow):
        assert_bits_equal(a, b, name)
    say("backward at the bench size: fp64 autograd on the GPU")
    Q, K, V = [t.cuda().double().requires_grad_() for t in (q, k, v)]
    Kr, Vr = K.repeat_interleave(4, 1), V.repeat_interleave(4, 1)
    s = torch.matmul(Q, Kr.transpose(-1, -2).contiguous()) * scale
    s = s.masked_fill(~torch.ones(1024, 1024, dtype=torch.bool, device=s.device).tril(), float("-inf"))
    torch.matmul(torch.softmax(s, -1), Vr).backward(dO.cuda().double())
    for name, a, b in zip(("dq", "dk", "dv"), fast, (Q.grad, K.grad, V.grad)):
        err = (a.double() - b).abs().max().item()
        tol = 2.0 ** -20 * (b.abs().max().item() + 1)
        assert err <= tol, (name, err, tol)


def test_backward_strided_nhd_views_and_strided_upstream(A, oracle):
    """Q, K, V as [B, H, S, D] views of one interleaved QKV buffer (row stride
    3 H D, head stride D, as the long workload's layout; GQA with the same
    head count for K and V here), a causal case, and an upstream gradient that
    is itself a strided view: the gradients must equal the oracle's on the
    same views, bit for bit."""
    S, H, D = 77, 4, 32
    buf = torch.randn(S, 3 * H * D, generator=torch.Generator().manual_seed(940)).to(torch.bfloat16)
    views = [torch.as_strided(buf, (1, H, S, D), (S * 3 * H * D, D, 3 * H * D, 1), off * H * D) for off in range(3)]
    q, k, v = views
    gbuf = torch.randn(S, 2 * H * D, generator=torch.Generator().manual_seed(941))
    dO = torch.as_strided(gbuf, (1, H, S, D), (S * 2 * H * D, D, 2 * H * D, 1), H * D)
    scale = W.default_scale(D)
    say("backward strided views: oracle")
    ref = oracle.attn_backward(q, k, v, dO, True, scale)
    bd, gd = buf.cuda(), gbuf.cuda()
    Qd, Kd, Vd = [torch.as_strided(bd, (1, H, S, D), (S * 3 * H * D, D, 3 * H * D, 1), off * H * D) for off in range(3)]
    dOd = torch.as_strided(gd, (1, H, S, D), (S * 2 * H * D, D, 2 * H * D, 1), H * D)
    out, m, den = A.det_attn_with_stats(Qd, Kd, Vd, True, scale)
    got = A.det_attn_backward(Qd, Kd, Vd, out, dOd, m, den, True, scale)
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        assert_bits_equal(a, b, name)


def test_backward_empty_ranges(A):
    """No keys: every dQ is +0 (no term); no queries: dK and dV are +0 and the
    call launches nothing else.  Non-causal, so the shapes may differ."""
    import ctypes as C
    from bitwise_deterministic_exact_pass1_amd import _lib
    L = _lib.lib()
    for Sq, Skv in ((5, 0), (0, 7)):
        q = torch.randn(1, 2, Sq, 8).to(torch.bfloat16).cuda()
        k = torch.randn(1, 1, Skv, 8).to(torch.bfloat16).cuda()
        v = torch.randn(1, 1, Skv, 8).to(torch.bfloat16).cuda()
        o = torch.zeros(1, 2, Sq, 8, device="cuda")
        dO = torch.randn(1, 2, Sq, 8).cuda()
        m = torch.full((1, 2, Sq), float("-inf"), device="cuda")
        den = torch.zeros(1, 2, Sq, dtype=torch.float64, device="cuda")
        g = [torch.full(t.shape, 7.0, device="cuda") for t in (q, k, v)]  # sentinels
        dq_, dk_, dv_ = A._desc(q), A._desc(k), A._desc(v)
        n = L.det_attn_backward_workspace_size(C.byref(dq_), C.byref(dk_), C.byref(dv_), 0)
        ws = torch.empty(max(n, 256) + 256, dtype=torch.uint8, device="cuda")
        addr = (ws.data_ptr() + 255) & ~255
        _lib.check(L.det_attn_backward(C.byref(dq_), C.byref(dk_), C.byref(dv_), C.byref(A._desc(o)),
                                       C.byref(A._desc(dO)), m.data_ptr(), den.data_ptr(), 0, 0.25,
                                       C.byref(A._out(g[0])), C.byref(A._out(g[1])), C.byref(A._out(g[2])),
                                       addr, max(n, 256), A._stream(q)))
        torch.cuda.synchronize()
        for t in g:
            assert not t.any() and not torch.signbit(t).any()


def test_backward_large_causal_share_chunks_both_paths_and_fp64(A):
    """The causal share B=1 Hq=32 Hkv=8 S=8192 D=128 bf16: the default
    workspace takes the query rows in several chunks; the matrix-core and
    per-term sums must give the same bits, and the gradients must lie within
    f32 rounding of fp64 autograd (computed on the GPU head by head)."""
    wl = W.attn_workload("cp_share_bf16")
    q, k, v, scale = wl["q"], wl["k"], wl["v"], wl["scale"]
    dO = upstream(4343, tuple(q.shape))
    say("backward S=8192 Hq=32: both paths")
    fast, slow = _backward_both_paths(A, q, k, v, dO, True, scale)
    for name, a, b in zip(("dq", "dk", "dv"), fast, slow):
        assert_bits_equal(a, b, name)
    say("backward S=8192 Hq=32: fp64 autograd per head group")
    S, grp = q.shape[2], q.shape[1] // k.shape[1]
    mask = ~torch.ones(S, S, dtype=torch.bool, device="cuda").tril()
    ref = [torch.zeros(t.shape, dtype=torch.float64) for t in (q, k, v)]
    for hk in range(k.shape[1]):
        hs = slice(hk * grp, (hk + 1) * grp)
        Q = q[:, hs].cuda().double().requires_grad_()
        K = k[:, hk:hk + 1].cuda().double().requires_grad_()
        V = v[:, hk:hk + 1].cuda().double().requires_grad_()
        s = torch.matmul(Q, K.expand(-1, grp, -1, -1).transpose(-1, -2).contiguous()) * scale
        torch.matmul(torch.softmax(s.masked_fill(mask, float("-inf")), -1), V.expand(-1, grp, -1, -1)).backward(
            dO[:, hs].cuda().double())
        ref[0][:, hs] = Q.grad.cpu()
        ref[1][:, hk:hk + 1] = K.grad.cpu()
        ref[2][:, hk:hk + 1] = V.grad.cpu()
        del Q, K, V, s
    for name, a, b in zip(("dq", "dk", "dv"), fast, ref):
        err = (a.cpu().double() - b).abs().max().item()
        tol = 2.0 ** -20 * (b.abs().max().item() + 1)
        assert err <= tol, (name, err, tol)


def _dyadic(seed, shape, lo, hi):
    """Integers in [-64, 64) times 2^e, e uniform in [lo, hi]: few significant
    bits at many binades, so most entries end in long runs of zero bits."""
    g = torch.Generator().manual_seed(seed)
    m = torch.randint(-64, 64, shape, generator=g).double()
    e = torch.randint(lo, hi + 1, shape, generator=g).double()
    return (m * torch.pow(2.0, e)).float()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_backward_right_operands_on_coarse_grids(A, oracle, dtype):
    """The right operands' grids (K, Q, dO columns) sit at each column's lowest
    set bit, so an entry can lie above its own f32 lsb grid and its digits are
    made by a right shift.  Dyadic Q, K, V, dO with a few full-precision
    entries mixed in exercise both shift directions; the matrix-core sums must
    match the per-term sums and the oracle bit for bit."""
    B, Hq, Hkv, S, D = 1, 4, 2, 80, 64
    q = _dyadic(940, (B, Hq, S, D), -12, 0).to(dtype)
    k = _dyadic(941, (B, Hkv, S, D), -12, 0).to(dtype)
    v = _dyadic(942, (B, Hkv, S, D), -20, 0).to(dtype)
    dO = _dyadic(943, (B, Hq, S, D), -24, 2)
    dO[0, 1, 5, :8] = torch.randn(8, generator=torch.Generator().manual_seed(944))
    q[0, 0, 3, 10] = 1.0 + 2.0 ** -7
    k[0, 1, 60, 20] = 2.0 ** -14
    scale = W.default_scale(D)
    say(f"backward coarse grids {dtype}")
    ref = oracle.attn_backward(q, k, v, dO, True, scale)
    fast, slow = _backward_both_paths(A, q, k, v, dO, True, scale)
    for name, a, b, c in zip(("dq", "dk", "dv"), fast, slow, ref):
        assert_bits_equal(a, c, name)
        assert_bits_equal(b, c, name + " (per-term)")
