"""GPU parity of the attention path against the CPU oracle (bit-exact), plus
the shard-invariance properties of the det-attn page ("Correctness": every KV
split and block permutation, and repeated runs, are torch.equal to the fused
result).  Inputs come from the seeded generators in workloads.py."""
import contextlib
import itertools
import os
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


def u32(x):
    """Bit pattern of an f32 array/tensor (NaN-safe equality)."""
    if isinstance(x, torch.Tensor):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(x, np.float32).view(np.uint32)


def assert_bits_equal(a, b, what=""):
    ua, ub = u32(a), u32(b)
    if not np.array_equal(ua, ub):
        bad = np.argwhere(ua != ub)
        raise AssertionError(f"{what}: {len(bad)} of {ua.size} differ; first at {bad[0].tolist()}")


def gpu(*ts):
    return [t.cuda() for t in ts]


# ---------------------------------------------------------------- tiny MHA f32 (S=128, D=64)

def test_tiny_fused_and_primitives_bit_exact(A, oracle):
    wl = W.attn_workload("tiny_mha_f32")
    q, k, v, scale = wl["q"], wl["k"], wl["v"], wl["scale"]
    say("tiny: oracle")
    ref, m, num, den = oracle.det_attn(q, k, v, False, scale, return_parts=True)
    Q, K, V = gpu(q, k, v)
    say("tiny: det_attn")
    out = A.det_attn(Q, K, V, False, scale)
    assert_bits_equal(out, ref, "det_attn")
    say("tiny: rowmax")
    gm = A.rowmax(Q, K, 0, 128, False, scale)
    assert_bits_equal(gm, m, "rowmax")
    say("tiny: accumulate")
    gn, gd = A.accumulate(Q, K, V, gm, 0, 128, False, scale)
    assert np.array_equal(gn.cpu().numpy(), num) and np.array_equal(gd.cpu().numpy(), den)
    assert_bits_equal(A.finalize(gn, gd), ref, "finalize")


def test_tiny_all_24_shard_orders(A):
    wl = W.attn_workload("tiny_mha_f32")
    Q, K, V = gpu(wl["q"], wl["k"], wl["v"])
    ref = A.det_attn(Q, K, V, False, wl["scale"])
    for order in itertools.permutations(range(4)):
        out = A.det_attn_sharded(Q, K, V, [32] * 4, False, wl["scale"], order=order)
        assert torch.equal(out, ref), order
    for order in list(itertools.permutations(range(4)))[::6]:
        out = A.det_attn_composed(Q, K, V, [32] * 4, False, wl["scale"], order=order)
        assert torch.equal(out, ref), order


def test_tiny_physical_block_permutations(A):
    """Non-causal: permuting whole 32-key blocks of K and V together."""
    wl = W.attn_workload("tiny_mha_f32")
    Q, K, V = gpu(wl["q"], wl["k"], wl["v"])
    ref = A.det_attn(Q, K, V, False, wl["scale"])
    for perm in itertools.permutations(range(4)):
        idx = torch.cat([torch.arange(32 * p, 32 * p + 32) for p in perm]).cuda()
        out = A.det_attn(Q, K[:, :, idx], V[:, :, idx], False, wl["scale"])
        assert torch.equal(out, ref), perm


# ---------------------------------------------------------------- causal GQA bf16 (B=2, Hq=8, Hkv=2, S=1024, D=128)

@pytest.fixture(scope="module")
def gqa(A):
    wl = W.attn_workload("gqa_causal_bf16")
    Q, K, V = gpu(wl["q"], wl["k"], wl["v"])
    say("gqa: det_attn")
    out = A.det_attn(Q, K, V, True, wl["scale"])
    torch.cuda.synchronize()
    return wl, Q, K, V, out


def test_gqa_causal_fused_bit_exact(gqa, oracle):
    wl, Q, K, V, out = gqa
    say("gqa: oracle (full)")
    ref = oracle.det_attn(wl["q"], wl["k"], wl["v"], True, wl["scale"])
    assert_bits_equal(out, ref, "det_attn gqa")


def test_gqa_causal_rowmax_and_digits_bit_exact(A, gqa, oracle):
    wl, Q, K, V, out = gqa
    gm = A.rowmax(Q, K, 0, 1024, True, wl["scale"])
    gn, gd = A.accumulate(Q, K, V, gm, 0, 1024, True, wl["scale"])
    rng = np.random.default_rng(20)
    rows = np.stack([rng.integers(0, 2, 48), rng.integers(0, 8, 48), rng.integers(0, 1024, 48)], 1)
    rows = np.concatenate([rows, [[0, 0, 0], [1, 7, 1023], [0, 3, 1], [1, 4, 511]]]).astype(np.int64)
    say("gqa: oracle rows")
    m = oracle.attn_rowmax(wl["q"], wl["k"], 0, 1024, True, wl["scale"], rows=rows)
    num, den = oracle.attn_accumulate(wl["q"], wl["k"], wl["v"], m, 0, 1024, True, wl["scale"], rows=rows)
    b, h, i = rows.T
    assert_bits_equal(gm.cpu().numpy()[b, h, i], m, "rowmax")
    gnc, gdc = gn.cpu().numpy(), gd.cpu().numpy()
    assert np.array_equal(gnc[:, b, h, i, :], num)
    assert np.array_equal(gdc[:, b, h, i], den)
    assert gnc[:13].min() >= 0 and gnc[:13].max() < 2 ** 32  # canonical


@pytest.mark.parametrize("splits", [[256] * 4, [64] * 16])
def test_gqa_causal_shard_invariance(A, gqa, splits):
    wl, Q, K, V, ref = gqa
    n = len(splits)
    for s in range(8):
        order = W.shard_order(1000 + 2 + 100 * n + s, n)
        out = A.det_attn_sharded(Q, K, V, splits, True, wl["scale"], order=order)
        assert torch.equal(out, ref), (splits[0], order)
    out = A.det_attn_composed(Q, K, V, splits, True, wl["scale"], order=W.shard_order(77 + n, n))
    assert torch.equal(out, ref)


def test_gqa_repeat_runs_identical(A, gqa):
    wl, Q, K, V, ref = gqa
    for _ in range(3):
        assert torch.equal(A.det_attn(Q, K, V, True, wl["scale"]), ref)


# ---------------------------------------------------------------- context-parallel share (sampled rows)

def _sample_rows(B, H, S, n, seed):
    rng = np.random.default_rng(seed)
    rows = np.stack([rng.integers(0, B, n), rng.integers(0, H, n), rng.integers(0, S, n)], 1)
    edge = [[0, 0, 0], [B - 1, H - 1, S - 1], [0, H - 1, 1], [B - 1, 0, S // 2]]
    return np.concatenate([rows, edge]).astype(np.int64)


@pytest.mark.parametrize("name,nrows", [("cp_share_bf16", 20), ("cp_share_d256_bf16", 40)])
def test_cp_share_sampled_rows_bit_exact(A, oracle, name, nrows):
    wl = W.attn_workload(name)
    Q, K, V = gpu(wl["q"], wl["k"], wl["v"])
    say(f"{name}: det_attn")
    out = A.det_attn(Q, K, V, True, wl["scale"])
    B, Hq, S, D = wl["q"].shape
    rows = _sample_rows(B, Hq, S, nrows, 31)
    say(f"{name}: oracle rows")
    ref = oracle.det_attn(wl["q"], wl["k"], wl["v"], True, wl["scale"], rows=rows)
    b, h, i = rows.T
    assert_bits_equal(out.cpu().numpy()[b, h, i], ref, name)
    for mode in (1, 2):
        say(f"{name}: det_attn, score source {mode}")
        with score_source(mode):
            o2 = A.det_attn(Q, K, V, True, wl["scale"])
        assert torch.equal(o2, out), f"score source {mode}"
    blk = 1024 if name == "cp_share_bf16" else 256
    say(f"{name}: 8 x {blk} shards")
    sh = A.det_attn_sharded(Q, K, V, [blk] * 8, True, wl["scale"], order=W.shard_order(1003, 8))
    assert torch.equal(sh, out)


# ---------------------------------------------------------------- long non-causal strided NHD

@pytest.fixture(scope="module")
def long_nhd(A):
    say("long: building the interleaved QKV buffer")
    buf = W.long_nhd_buffer()
    return buf, buf.cuda()


def test_long_nhd_sampled_rows_bit_exact(A, oracle, long_nhd):
    buf, dbuf = long_nhd
    q, k, v = W.long_nhd_views(buf)
    Q, K, V = W.long_nhd_views(dbuf)
    scale = W.default_scale(128)
    say("long: det_attn (full)")
    out = A.det_attn(Q, K, V, False, scale)
    torch.cuda.synchronize()
    rows = _sample_rows(1, 56, W.LONG_S, 12, 55)
    say("long: oracle rows")
    ref = oracle.det_attn(q, k, v, False, scale, rows=rows)
    b, h, i = rows.T
    assert_bits_equal(out.cpu().numpy()[b, h, i], ref, "long nhd")
    for mode in (1, 2):  # kept and recomputed scores, whichever the default chose
        say(f"long: det_attn, score source {mode}")
        with score_source(mode):
            o2 = A.det_attn(Q, K, V, False, scale)
        torch.cuda.synchronize()
        assert torch.equal(o2, out), f"score source {mode}"
        del o2


def test_long_nhd_591_blocks_all_rows(A, long_nhd):
    """KV split into 590 blocks of 64 plus 50, composed in two seeded orders,
    over every query row of all 56 heads: torch.equal to the fused result."""
    buf, dbuf = long_nhd
    Q, K, V = W.long_nhd_views(dbuf)
    scale = W.default_scale(128)
    say("long: fused reference")
    ref = A.det_attn(Q, K, V, False, scale)
    splits = [64] * 590 + [50]
    for seed in (1005, 2005):
        say(f"long: 591 shards order seed {seed}, all rows")
        out = A.det_attn_sharded(Q, K, V, splits, False, scale, order=W.shard_order(seed, 591))
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        del out


# ---------------------------------------------------------------- edge cases

@pytest.mark.parametrize("D", [1, 3, 17, 100, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_head_dims_and_ragged_tails(A, oracle, D, causal):
    q, k, v = W.attn_inputs(300 + D, 1, 4, 2, 45, 45, D, torch.bfloat16)
    scale = W.default_scale(D)
    ref = oracle.det_attn(q, k, v, causal, scale)
    out = A.det_attn(*gpu(q, k, v), causal, scale)
    assert_bits_equal(out, ref, f"D={D}")


def test_noncausal_rectangular_and_one_key(A, oracle):
    q, k, v = W.attn_inputs(401, 2, 3, 1, 70, 300, 32, torch.float32)
    ref = oracle.det_attn(q, k, v, False, 0.2)
    assert_bits_equal(A.det_attn(*gpu(q, k, v), False, 0.2), ref, "rect")
    q, k, v = W.attn_inputs(402, 1, 2, 2, 5, 1, 16, torch.float32)
    out = A.det_attn(*gpu(q, k, v), False, 0.25)
    assert torch.equal(out.cpu(), v.expand(1, 2, 5, 16))


def test_wide_score_spread_tiny_and_subnormal_weights(A, oracle):
    """Large scores make most weights tiny or subnormal in f32, exercising every
    window flush; tiny V entries put products far below the others."""
    q, k, v = W.attn_inputs(403, 1, 2, 1, 64, 64, 16, torch.float32, std=6.0)
    v[0, 0, ::7, ::3] *= 1e-30
    v[0, 0, 5, :] = 0.0
    for scale in (1.0, 3.0):
        ref = oracle.det_attn(q, k, v, False, scale)
        out = A.det_attn(*gpu(q, k, v), False, scale)
        assert_bits_equal(out, ref, f"spread scale={scale}")
        assert np.isfinite(ref).all()


def test_special_values(A, oracle):
    q, k, v = W.attn_inputs(404, 1, 1, 1, 9, 9, 8, torch.float32)
    kz = torch.zeros_like(k)
    assert_bits_equal(A.det_attn(*gpu(q, kz, v), False, 0.5), oracle.det_attn(q, kz, v, False, 0.5), "K=0")
    vz = torch.zeros_like(v)
    out = A.det_attn(*gpu(q, k, vz), False, 0.5)
    assert torch.equal(out.cpu(), torch.zeros_like(out.cpu())) and not torch.signbit(out).any()


def test_empty_key_range_gives_neg_inf_and_nan(A):
    q, k, v = gpu(*W.attn_inputs(405, 1, 2, 2, 8, 8, 16, torch.float32))
    m = A.rowmax(q, k, 4, 4)
    assert torch.isneginf(m).all()
    num, den = A.accumulate(q, k, v, m, 4, 4)
    assert not num.any() and not den.any()
    assert torch.isnan(A.finalize(num, den)).all()


def test_accumulate_add_into_equals_combine(A):
    q, k, v = gpu(*W.attn_inputs(406, 1, 2, 1, 50, 50, 24, torch.bfloat16))
    m = A.rowmax(q, k, 0, 50, True)
    n1, d1 = A.accumulate(q, k, v, m, 0, 20, True)
    n2, d2 = A.accumulate(q, k, v, m, 20, 50, True)
    nall, dall = A.accumulate(q, k, v, m, 0, 50, True)
    na, da = n1.clone(), d1.clone()
    A.accumulate(q, k, v, m, 20, 50, True, num=na, den=da)
    assert torch.equal(na, nall) and torch.equal(da, dall)
    A.combine_digits(n1, n2)
    A.combine_digits(d1, d2)
    assert torch.equal(n1, nall) and torch.equal(d1, dall)
    # a caller-side int64 add (non-canonical) finalizes to the same output
    n3, d3 = A.accumulate(q, k, v, m, 0, 20, True)
    assert torch.equal(A.finalize(n3 + n2, d3 + d2), A.finalize(nall, dall))


def test_empty_query_rows(A):
    q, k, v = gpu(*W.attn_inputs(407, 1, 2, 2, 0, 16, 16, torch.float32))
    out = A.det_attn(q, k, v, False)
    assert out.shape == (1, 2, 0, 16)


# ---------------------------------------------------------------- both deposit paths

@contextlib.contextmanager
def generic_path():
    """Send every tile through the generic exact deposit instead of the
    matrix-core one (the library's testing switch)."""
    from bitwise_deterministic_exact_pass1_amd import _lib
    _lib.force_generic(True)
    try:
        yield
    finally:
        _lib.force_generic(False)


@pytest.mark.parametrize("case", ["tiny", "gqa_small", "d3", "d256", "rect"])
def test_matrix_core_and_generic_paths_bit_identical(A, oracle, case):
    if case == "tiny":
        wl = W.attn_workload("tiny_mha_f32")
        q, k, v, causal, scale = wl["q"], wl["k"], wl["v"], False, wl["scale"]
    elif case == "gqa_small":
        q, k, v = W.attn_inputs(501, 2, 4, 2, 200, 200, 128, torch.bfloat16)
        causal, scale = True, W.default_scale(128)
    elif case == "d3":
        q, k, v = W.attn_inputs(502, 1, 2, 1, 70, 70, 3, torch.bfloat16)
        causal, scale = True, W.default_scale(3)
    elif case == "d256":
        q, k, v = W.attn_inputs(503, 1, 2, 2, 96, 96, 256, torch.bfloat16)
        causal, scale = False, W.default_scale(256)
    else:
        q, k, v = W.attn_inputs(504, 1, 3, 3, 33, 131, 64, torch.float32)
        causal, scale = False, 0.15
    Q, K, V = gpu(q, k, v)
    fast = A.det_attn(Q, K, V, causal, scale)
    m = A.rowmax(Q, K, 0, K.shape[2], causal, scale)
    nf, df = A.accumulate(Q, K, V, m, 0, K.shape[2], causal, scale)
    with generic_path():
        gen = A.det_attn(Q, K, V, causal, scale)
        ng, dg = A.accumulate(Q, K, V, m, 0, K.shape[2], causal, scale)
    assert torch.equal(fast, gen)
    assert torch.equal(nf, ng) and torch.equal(df, dg)
    assert_bits_equal(fast, oracle.det_attn(q, k, v, causal, scale), case)


@pytest.mark.parametrize("causal", [False, True])
def test_bf16_scores_outlier_rows_take_the_fp64_chain(A, oracle, causal):
    """Rows whose entries span many binades break the matrix-core exactness
    bound (or need more than four int8 digits); those items are recomputed by
    the fp64 chain and must still match the oracle bit for bit."""
    q, k, v = W.attn_inputs(601, 1, 4, 2, 96, 96, 128, torch.float32)
    q[0, 1, 3, 5] = 1e-9
    q[0, 2, 40, :7] = 3e-12
    k[0, 0, 7, 9] = 2e-10
    k[0, 1, 50, 100] = 5e-13
    k[0, 1, 51, :] *= 1e6
    q, k, v = q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)
    ref = oracle.det_attn(q, k, v, causal, 0.02)
    out = A.det_attn(*gpu(q, k, v), causal, 0.02)
    assert_bits_equal(out, ref, "outliers")
    m = A.rowmax(*gpu(q, k), 0, 96, causal, 0.02)
    assert_bits_equal(m, oracle.attn_rowmax(q, k, 0, 96, causal, 0.02), "rowmax")


@pytest.mark.parametrize("nkeys", [40, 300])
def test_pairs_outside_the_refined_bound_deferred_and_overflowing(A, oracle, nkeys):
    """Query rows and keys each holding one small entry at the same position:
    every such pair fails both the item bound and the refined per-pair bound
    (equal positions), so its score must come from the fp64 chain.  Two rows
    against 40 keys (80 pairs: several extra blocks of deferred pairs) and
    against 300 keys (600 pairs: more than a tile can defer, the tile takes
    the generic path) must both match the oracle bit for bit."""
    q, k, v = W.attn_inputs(611, 1, 2, 1, 64, 320, 128, torch.float32)
    for r in (5, 21):
        q[0, 1, r, 77] = 2.0 ** -15 * 1.5
    k[0, 0, :nkeys, 77] = 2.0 ** -18 * 1.25
    q, k, v = q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)
    ref = oracle.det_attn(q, k, v, False, 0.05)
    out = A.det_attn(*gpu(q, k, v), False, 0.05)
    assert_bits_equal(out, ref, f"{nkeys} keys")


def test_small_workspace_many_row_chunks_bit_identical(A, gqa):
    """A workspace a sixth of the default size makes the library run the query
    rows in several chunks (K and V are prepared by the first chunk's launches
    only); the output must be the same bits."""
    import ctypes as C
    from bitwise_deterministic_exact_pass1_amd import _lib
    wl, Q, K, V, out = gqa
    say("gqa: det_attn with a small workspace")
    q, k, v = A._desc(Q), A._desc(K), A._desc(V)
    L = _lib.lib()
    full = L.det_attn_workspace_size(C.byref(q), C.byref(k), C.byref(v), 1)
    small = (full // 6) // 256 * 256
    ws = torch.empty(small + 256, dtype=torch.uint8, device=Q.device)
    addr = (ws.data_ptr() + 255) & ~255
    o2 = torch.empty_like(out)
    _lib.check(L.det_attn(C.byref(q), C.byref(k), C.byref(v), 1, wl["scale"], C.byref(A._out(o2)), addr, small,
                          A._stream(Q)))
    assert torch.equal(o2, out)


# ---------------------------------------------------------------- V columns wider than the digit grid

def v_with_low_bits(v, D):
    """bf16 V with a few entries whose bits reach far below the rest of their
    column: wholly (2^-40, -2^-60, 3 2^-45) or partly (1.0078125 2^-30,
    1.5 2^-33) under a five-digit column grid."""
    v = v.clone()
    for b, h, j, d, x in [(0, 0, 17, 5, 2.0 ** -40), (0, 0, 250, 5, -1.0078125 * 2.0 ** -30),
                          (0, 1, 3, D - 1, 3 * 2.0 ** -45), (0, 1, 299, 40, -2.0 ** -60),
                          (0, 0, 0, 0, 1.5 * 2.0 ** -33)]:
        v[b, h, j, d] = x
    return v


@pytest.mark.parametrize("causal,D", [(False, 128), (True, 128), (True, 256)])
def test_v_columns_wider_than_the_digit_grid(A, oracle, causal, D):
    """The matrix-core part on the coarser column grid plus the exact remainder
    products: the fused, sharded and digit paths equal the oracle and the
    generic path bit for bit."""
    q, k, v = W.attn_inputs(610 + D + int(causal), 1, 4, 2, 300, 300, D, torch.bfloat16)
    v = v_with_low_bits(v, D)
    scale = W.default_scale(D)
    say(f"wide V columns: oracle causal={causal} D={D}")
    ref = oracle.det_attn(q, k, v, causal, scale)
    Q, K, V = gpu(q, k, v)
    out = A.det_attn(Q, K, V, causal, scale)
    assert_bits_equal(out, ref, "fused")
    sh = A.det_attn_sharded(Q, K, V, [100, 64, 136], causal, scale, order=[2, 0, 1])
    assert torch.equal(sh, out)
    m = A.rowmax(Q, K, 0, 300, causal, scale)
    n1, d1 = A.accumulate(Q, K, V, m, 0, 300, causal, scale)
    assert torch.equal(A.finalize(n1, d1), out)
    with generic_path():
        n2, d2 = A.accumulate(Q, K, V, m, 0, 300, causal, scale)
    assert torch.equal(n1, n2) and torch.equal(d1, d2)


def test_v_remainder_list_overflow_takes_the_generic_path(A, oracle):
    """More remainders than the list holds: their heads take the generic exact
    path, with the same bits."""
    q, k, v = W.attn_inputs(620, 1, 2, 2, 640, 640, 32, torch.bfloat16)
    g = torch.Generator().manual_seed(621)
    idx = torch.randperm(640 * 32, generator=g)[:5000]
    flat = v[0, 1].reshape(-1)
    flat[idx] = (flat[idx] * 2.0 ** -45).to(torch.bfloat16)
    v[0, 1] = flat.reshape(640, 32)
    scale = W.default_scale(32)
    say("remainder overflow: oracle")
    ref = oracle.det_attn(q, k, v, True, scale)
    out = A.det_attn(*gpu(q, k, v), True, scale)
    assert_bits_equal(out, ref, "overflow")


# ---------------------------------------------------------------- both pass-2 layouts

@contextlib.contextmanager
def pass2_layout(mode):
    """Force one of pass 2's two kernel layouts for bf16 head dims <= 128 (the
    library's testing switch; 0 restores the choice by key-range length)."""
    from bitwise_deterministic_exact_pass1_amd import _lib
    _lib.pass2_layout(mode)
    try:
        yield
    finally:
        _lib.pass2_layout(0)


def _layout_case(case):
    if case == "gqa_causal":
        q, k, v = W.attn_inputs(701, 2, 4, 2, 333, 333, 128, torch.bfloat16)
        return q, k, v, True, W.default_scale(128)
    if case == "d64_rect":
        q, k, v = W.attn_inputs(702, 1, 3, 1, 77, 450, 64, torch.bfloat16)
        return q, k, v, False, W.default_scale(64)
    if case == "d17_causal":
        q, k, v = W.attn_inputs(703, 1, 2, 2, 130, 130, 17, torch.bfloat16)
        return q, k, v, True, W.default_scale(17)
    if case == "wide_v":
        q, k, v = W.attn_inputs(704, 1, 4, 2, 300, 300, 128, torch.bfloat16)
        return q, k, v_with_low_bits(v, 128), True, W.default_scale(128)
    q, k, v = W.attn_inputs(705, 1, 2, 1, 64, 320, 128, torch.float32)
    if case.startswith("deferred"):
        nkeys = int(case.split("_")[1])
        for r in (5, 21):
            q[0, 1, r, 77] = 2.0 ** -15 * 1.5
        k[0, 0, :nkeys, 77] = 2.0 ** -18 * 1.25
    else:  # outlier rows: many binades, more than four digits
        q[0, 1, 3, 5] = 1e-9
        q[0, 0, 40, :7] = 3e-12
        k[0, 0, 7, 9] = 2e-10
        k[0, 0, 51, :] *= 1e6
    return q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16), False, 0.05


@contextlib.contextmanager
def score_source(mode):
    """Force how pass 2 gets bf16 scores: 1 kept from pass 1, 2 recomputed
    from the digit rows (the library's testing switch; 0 restores the choice
    by workspace size)."""
    from bitwise_deterministic_exact_pass1_amd import _lib
    _lib.score_source(mode)
    try:
        yield
    finally:
        _lib.score_source(0)


LAYOUT_CASES = ["gqa_causal", "d64_rect", "d17_causal", "wide_v", "deferred_40", "deferred_300", "outliers"]


@pytest.mark.parametrize("case", LAYOUT_CASES)
def test_kept_and_recomputed_scores_bit_identical(A, oracle, case):
    """Pass 2 reading the scores pass 1 kept, or recomputing them from the
    digit rows, in either kernel layout, gives the oracle's bits: fused,
    sharded with ragged splits, and as digits."""
    q, k, v, causal, scale = _layout_case(case)
    say(f"score sources: {case}")
    Q, K, V = gpu(q, k, v)
    S = K.shape[2]
    splits = [S // 3, 5, S - S // 3 - 5]
    res = {}
    for mode in (1, 2):
        for layout in (1, 2):
            with score_source(mode), pass2_layout(layout):
                out = A.det_attn(Q, K, V, causal, scale)
                sh = A.det_attn_sharded(Q, K, V, splits, causal, scale, order=[2, 0, 1])
                m = A.rowmax(Q, K, 0, S, causal, scale)
                n, d = A.accumulate(Q, K, V, m, 0, S, causal, scale)
            torch.cuda.synchronize()
            assert torch.equal(sh, out), f"source {mode} layout {layout}: sharded != fused"
            res[mode, layout] = (out, n, d)
    ref = res[1, 2]
    for key, (out, n, d) in res.items():
        assert torch.equal(out, ref[0]) and torch.equal(n, ref[1]) and torch.equal(d, ref[2]), key
    assert_bits_equal(ref[0], oracle.det_attn(q, k, v, causal, scale), case)


@pytest.mark.parametrize("case", LAYOUT_CASES)
def test_pass2_layouts_bit_identical(A, oracle, case):
    """With recomputed scores, pass 2's two kernel layouts (split
    weight-making and multiplying waves, or eight waves doing both) give the
    same bits as each other and as the oracle: fused, sharded with ragged
    splits, and as digits."""
    q, k, v, causal, scale = _layout_case(case)
    say(f"pass-2 layouts: {case}")
    Q, K, V = gpu(q, k, v)
    S = K.shape[2]
    splits = [S // 3, 5, S - S // 3 - 5]  # ragged, one shard shorter than a key block
    res = {}
    for mode in (1, 2):
        with pass2_layout(mode), score_source(2):
            out = A.det_attn(Q, K, V, causal, scale)
            sh = A.det_attn_sharded(Q, K, V, splits, causal, scale, order=list(range(len(splits)))[::-1])
            m = A.rowmax(Q, K, 0, S, causal, scale)
            n, d = A.accumulate(Q, K, V, m, 0, S, causal, scale)
        torch.cuda.synchronize()
        assert torch.equal(sh, out), f"layout {mode}: sharded != fused"
        res[mode] = (out, n, d)
    assert torch.equal(res[1][0], res[2][0])
    assert torch.equal(res[1][1], res[2][1]) and torch.equal(res[1][2], res[2][2])
    assert_bits_equal(res[1][0], oracle.det_attn(q, k, v, causal, scale), case)
