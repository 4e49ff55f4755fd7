"""GPU parity of the entry points' range arguments and of long key ranges
(det-attn page, "API": rowmax and accumulate over [kv_lo, kv_hi) for a block
of query rows; "Method": the sums are exact whatever the number of keys, so
one launch over 2^17 or 2^19 keys must still equal the oracle bit for bit)."""
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
    if isinstance(x, torch.Tensor):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(x, np.float32).view(np.uint32)


def _long_inputs(seed, Hq, Sq, Skv, D, top_col=True):
    """Zero queries (every score 0, every weight 1: DEN is the key count) and
    N(0,1) bf16 values, with column 0 at 3.984375 on every key but one, which
    holds 2^-29: that column spans 38 bits, so it takes five digits with the
    largest top digit the grid allows."""
    q = torch.zeros(1, Hq, Sq, D, dtype=torch.bfloat16)
    k = torch.randn(1, 1, Skv, D, generator=torch.Generator().manual_seed(seed)).to(torch.bfloat16)
    v = torch.randn(1, 1, Skv, D, generator=torch.Generator().manual_seed(seed + 1)).to(torch.bfloat16)
    if top_col:
        v[0, 0, :, 0] = 3.984375
        v[0, 0, 17, 0] = 2.0 ** -29
    return q, k, v


@pytest.mark.parametrize("Skv,Hq,Sq,D", [(2 ** 17 + 64, 2, 33, 40), (2 ** 19 + 4096, 1, 2, 8)],
                         ids=["den-2^17", "top-class-2^19"])
def test_long_key_range_one_launch_bit_exact(A, oracle, Skv, Hq, Sq, D):
    """2^17 + 64 keys of weight 1 put DEN * 2^46 past 2^63; 2^19 + 4096 keys
    put the top shift class of the five-digit column past 2^31.  Fused output,
    the primitives' digits and a two-shard composition (both orders) all equal
    the oracle bit for bit."""
    q, k, v = _long_inputs(900 + Sq, Hq, Sq, Skv, D)
    say(f"long range: Skv={Skv} Hq={Hq} Sq={Sq} D={D}: oracle")
    ref, m, num, den = oracle.det_attn(q, k, v, False, 0.125, return_parts=True)
    Q, K, V = q.cuda(), k.cuda(), v.cuda()
    say("long range: det_attn")
    out = A.det_attn(Q, K, V, False, 0.125)
    assert np.array_equal(u32(out), u32(ref))
    say("long range: accumulate")
    gm = A.rowmax(Q, K, 0, Skv, False, 0.125)
    assert np.array_equal(u32(gm), u32(m))
    gn, gd = A.accumulate(Q, K, V, gm, 0, Skv, False, 0.125)
    assert np.array_equal(gn.cpu().numpy(), num) and np.array_equal(gd.cpu().numpy(), den)
    half = Skv // 2
    for order in ([0, 1], [1, 0]):
        say(f"long range: sharded {order}")
        sh = A.det_attn_sharded(Q, K, V, [half, Skv - half], False, 0.125, order=order)
        assert torch.equal(sh, out)


def test_query_subranges_bit_exact_and_rows_outside_untouched(A, oracle):
    """rowmax and accumulate over query rows [q_lo, q_hi): the rows inside
    equal the oracle's, the rows outside keep what the caller's arrays held,
    and composing query blocks and key shards gives the fused output."""
    B, Hq, Hkv, S, D = 1, 4, 2, 150, 72
    q, k, v = W.attn_inputs(950, B, Hq, Hkv, S, S, D, torch.bfloat16)
    Q, K, V = q.cuda(), k.cuda(), v.cuda()
    scale = W.default_scale(D)
    ref, m, num, den = oracle.det_attn(q, k, v, True, scale, return_parts=True)
    for qlo, qhi in [(0, 150), (37, 101), (149, 150), (64, 64)]:
        say(f"subrange [{qlo},{qhi})")
        sentinel = torch.full((B, Hq, S), 7.0, device="cuda")
        gm = A.rowmax(Q, K, 0, S, True, scale, q_lo=qlo, q_hi=qhi, out=sentinel)
        got = gm.cpu().numpy()
        assert np.array_equal(u32(got[:, :, qlo:qhi]), u32(m[:, :, qlo:qhi]))
        assert (got[:, :, :qlo] == 7.0).all() and (got[:, :, qhi:] == 7.0).all()
        fill_n = torch.full((14, B, Hq, S, D), 5, dtype=torch.int64, device="cuda")
        fill_d = torch.full((9, B, Hq, S), 5, dtype=torch.int64, device="cuda")
        # new arrays: the range holds the digits, the rest stays zero
        gn, gd = A.accumulate(Q, K, V, torch.from_numpy(m).cuda(), 0, S, True, scale, q_lo=qlo, q_hi=qhi)
        assert np.array_equal(gn.cpu().numpy()[:, :, :, qlo:qhi], num[:, :, :, qlo:qhi])
        assert np.array_equal(gd.cpu().numpy()[:, :, :, qlo:qhi], den[:, :, :, qlo:qhi])
        assert not gn[:, :, :, :qlo].any() and not gn[:, :, :, qhi:].any()
        # add_into = 1 adds keys [0, 90) into rows that hold 5 in every digit,
        # and keys [90, S) into zeros
        zn = torch.zeros_like(fill_n)
        zd = torch.zeros_like(fill_d)
        A.accumulate(Q, K, V, torch.from_numpy(m).cuda(), 0, 90, True, scale, num=fill_n, den=fill_d, q_lo=qlo,
                     q_hi=qhi)
        A.accumulate(Q, K, V, torch.from_numpy(m).cuda(), 90, S, True, scale, num=zn, den=zd, q_lo=qlo, q_hi=qhi)
        # rows outside the range still hold 5 in every digit (never normalized)
        assert (fill_n[:, :, :, :qlo] == 5).all() and (fill_n[:, :, :, qhi:] == 5).all()
        assert (fill_d[:, :, :, :qlo] == 5).all() and (fill_d[:, :, :, qhi:] == 5).all()
        if qhi > qlo:
            # inside: (the 5s + keys [0, 90)) - the 5s + keys [90, S) is the whole sum by value
            # (finalize takes any non-overflowing digit sum)
            fives = torch.full_like(fill_n[:, :, :, qlo:qhi], 5)
            fn = fill_n[:, :, :, qlo:qhi] - fives + zn[:, :, :, qlo:qhi]
            fd = fill_d[:, :, :, qlo:qhi] - torch.full_like(fill_d[:, :, :, qlo:qhi], 5) + zd[:, :, :, qlo:qhi]
            out = A.finalize(fn.contiguous(), fd.contiguous(), (B, Hq, qhi - qlo, D))
            assert np.array_equal(u32(out), u32(ref[:, :, qlo:qhi]))


def test_digits_normalize_of_a_caller_side_sum(A):
    """A caller-side int64 sum of canonical digit arrays (the cross-entropy
    page's sum(...)) normalizes to exactly what the library's combine makes."""
    q, k, v = [t.cuda() for t in W.attn_inputs(951, 1, 2, 1, 70, 70, 24, torch.bfloat16)]
    m = A.rowmax(q, k, 0, 70, True)
    parts = [A.accumulate(q, k, v, m, lo, hi, True) for lo, hi in [(0, 20), (20, 45), (45, 70)]]
    nsum = parts[0][0] + parts[1][0] + parts[2][0]
    dsum = parts[0][1] + parts[1][1] + parts[2][1]
    ncomb, dcomb = parts[0][0].clone(), parts[0][1].clone()
    for n_, d_ in parts[1:]:
        A.combine_digits(ncomb, n_)
        A.combine_digits(dcomb, d_)
    A.normalize_digits(nsum)
    A.normalize_digits(dsum)
    assert torch.equal(nsum, ncomb) and torch.equal(dsum, dcomb)
    assert (nsum[:13] >= 0).all() and (nsum[:13] < 2 ** 32).all()
