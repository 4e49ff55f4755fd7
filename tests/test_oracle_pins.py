"""Pins of the CPU oracle to mathematics (no GPU).

Each test ties one part of the oracle to something other than itself: a
correctly rounded reference (mpmath at 200+ bits), Python's exact integers and
correctly rounded int->float conversion, a closed form, or brute-force fp64
softmax attention.  The method is the det-attn page ("Method") and the
det-cross-entropy page ("Method").
"""
import math
import random
from fractions import Fraction

import mpmath
import numpy as np
import pytest
import torch

from bitwise_deterministic_exact_pass1_amd import workloads as W

mpmath.mp.prec = 256
F32_MIN_SUB = Fraction(1, 2 ** 149)


def rn32_exact(x) -> float:
    """Correctly rounded binary32 (ties to even, gradual underflow) of a real
    given as mpmath mpf or Fraction; returned as a Python float."""
    x = Fraction(x) if not isinstance(x, Fraction) else x
    if x == 0:
        return 0.0
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = math.floor(math.log2(a)) if a.numerator and a.denominator else 0
    # fix e so that 2^e <= a < 2^(e+1)
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp_exp = max(e, -126) - 23
    q = a / Fraction(2) ** ulp_exp
    n = q.numerator // q.denominator
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * float(Fraction(n) * Fraction(2) ** ulp_exp)


def mp_frac(x: mpmath.mpf) -> Fraction:
    m, e = mpmath.mpf(x).man_exp
    return Fraction(int(m)) * (Fraction(2) ** int(e))


def ulp64(x: float) -> float:
    return math.ulp(x)


# ---------------------------------------------------------------- elementary routines

def test_exp_det_accuracy_and_rn32(oracle):
    """exp_det is within 2 fp64 ulps of e^t on [-104, 0], and its RN32 equals the
    correctly rounded binary32 e^t except within 2^-50 relative of a midpoint."""
    rng = random.Random(7)
    pts = [0.0, -0.0, -1e-300, -1e-17, -0.5, -0.34657359027997264, -0.3465735902799727, -1.0,
           -87.33654475055310898657, -87.3365, -103.972, -103.0, -104.0]
    pts += [-rng.uniform(0, 104) for _ in range(3000)] + [-rng.uniform(0, 10) for _ in range(3000)]
    mismatches = 0
    for t in pts:
        got = oracle.exp_det(t)
        ref = mpmath.exp(mpmath.mpf(t))
        assert abs(mpmath.mpf(got) - ref) <= 2 * ulp64(float(ref)), t
        w = float(np.float32(got))
        want = rn32_exact(mp_frac(ref))
        if w != want:
            # only allowed when e^t sits within 2^-50 (relative) of an f32 rounding midpoint
            mid = (Fraction(w) + Fraction(want)) / 2
            assert abs(mp_frac(ref) - mid) <= abs(mid) * Fraction(1, 2 ** 50), t
            mismatches += 1
    assert mismatches <= 2
    assert oracle.exp_det(0.0) == 1.0 and oracle.exp_det(-0.0) == 1.0
    assert oracle.exp_det(-104.5) == 0.0 and oracle.exp_det(-1e6) == 0.0


def test_exp_det_never_exceeds_one_and_is_monotone_in_f32(oracle):
    ts = sorted(-x for x in np.linspace(0, 30, 20001))  # ascending t in [-30, 0]
    ws = [float(np.float32(oracle.exp_det(t))) for t in ts]
    assert max(ws) == 1.0
    assert all(a <= b for a, b in zip(ws, ws[1:]))


def test_log_det_accuracy(oracle):
    rng = random.Random(3)
    xs = [1.0, 1.0 + 2 ** -52, 1.4142135623730951, 1.4142135623730954, 2.0, 3.0, 128256.0, 2.0 ** 40]
    xs += [1.0 + rng.random() * 10 ** rng.uniform(0, 6) for _ in range(4000)]
    for x in xs:
        got = oracle.log_det(x)
        ref = mpmath.log(mpmath.mpf(x))
        tol = 2 * ulp64(float(ref)) if ref != 0 else 0.0
        assert abs(mpmath.mpf(got) - ref) <= max(tol, 2 ** -1074), x
    assert oracle.log_det(1.0) == 0.0


# ---------------------------------------------------------------- score rule

def test_score_uses_ascending_sequential_fp64_chain(oracle):
    """Terms 2^60, 1, -2^60 in that order: the fp64 chain loses the 1, so s = 0;
    exact or reordered summation would give 1."""
    q = np.array([2.0 ** 30, 1.0, 2.0 ** 30], np.float32)
    k = np.array([2.0 ** 30, 1.0, -2.0 ** 30], np.float32)
    assert oracle.score(q, k, 1.0) == 0.0
    q2 = np.array([2.0 ** 30, 2.0 ** 30, 1.0], np.float32)
    k2 = np.array([2.0 ** 30, -2.0 ** 30, 1.0], np.float32)
    assert oracle.score(q2, k2, 1.0) == 1.0


def test_score_scale_applied_after_dot_then_rn32(oracle):
    """s = RN32(RN64(scale * dot)): with scale = 1/sqrt(128) and a dot of 3,
    scaling each element first would round differently."""
    scale = W.default_scale(128)
    assert scale.hex() == "0x1.6a09e667f3bccp-4"
    q = np.ones(3, np.float32)
    assert oracle.score(q, q, scale) == float(np.float32(3.0 * scale))
    # power-of-two inputs: the chain is exact, s is a closed form
    q = np.array([0.5, 0.25, 2.0, -4.0], np.float32)
    k = np.array([2.0, 8.0, 0.125, 0.5], np.float32)
    assert oracle.score(q, k, 0.125) == (1 + 2 + 0.25 - 2) * 0.125


def test_score_matches_python_float_chain(oracle):
    """Random f32 rows: products of f32 values are exact in binary64, so the
    Python loop acc = acc + q*k is the same fma chain."""
    rng = np.random.default_rng(11)
    for D in (1, 3, 64, 128, 256):
        for _ in range(30):
            q = rng.standard_normal(D).astype(np.float32) * np.float32(rng.uniform(0.1, 10))
            k = rng.standard_normal(D).astype(np.float32)
            acc = 0.0
            for a, b in zip(q.tolist(), k.tolist()):
                acc = acc + a * b
            assert oracle.score(q, k, 0.0625) == float(np.float32(0.0625 * acc))


# ---------------------------------------------------------------- digits / exact sums

def _digits_of_int(n: int, K: int):
    """Canonical radix-2^32 digits of a Python int (top digit signed)."""
    out = []
    for _ in range(K - 1):
        out.append(n & 0xFFFFFFFF)
        n >>= 32
    out.append(n)
    return out


def _int_of_digits(ds) -> int:
    return sum(int(d) << (32 * k) for k, d in enumerate(ds))


def test_digits_roundtrip_and_rounding(oracle):
    rng = random.Random(5)
    vals = []
    for _ in range(2000):
        e = rng.randint(-298 + 60, 100)
        mant = rng.getrandbits(120) - (1 << 119)
        vals.append(mant << (e + 298 - 60) if e + 298 - 60 >= 0 else mant)
    vals += [0, 1, -1, (1 << 53) + 1, ((1 << 53) + 1) << 10, -((1 << 54) + 3), (1 << 400) - 1]
    digits = np.array([_digits_of_int(v, 14) for v in vals], dtype=object)
    arr = np.array([[int(x) for x in row] for row in digits], dtype=np.int64).T.copy()
    got = oracle.digits_to_double(arr, 14, -298)
    for v, g in zip(vals, got.tolist()):
        assert g == float(Fraction(v, 2 ** 298)), v  # int/int true division is correctly rounded
    # doubles -> digits -> exact integer
    xs = np.array([1.0, -1.0, 2.0 ** -298, 3.5, -(2.0 ** 120) * 1.25, 1e-50, 0.0])
    d = oracle.double_to_digits(xs, 14, -298)
    for j, x in enumerate(xs.tolist()):
        assert _int_of_digits(d[:, j]) == int(Fraction(x) * 2 ** 298)
        assert d[:13, j].min() >= 0 and d[:13, j].max() < 2 ** 32


def test_digits_combine_is_exact_canonical_sum(oracle):
    rng = random.Random(9)
    K = 9
    a_vals = [rng.getrandbits(200) - (1 << 199) for _ in range(500)]
    b_vals = [rng.getrandbits(150) - (1 << 149) for _ in range(500)]
    A = np.array([_digits_of_int(v, K) for v in a_vals], np.int64).T.copy()
    B = np.array([_digits_of_int(v, K) for v in b_vals], np.int64).T.copy()
    # non-canonical input: move 5 units from digit 1 into digit 0 of B
    B[0] += 5 << 32
    B[1] -= 5
    C = oracle.digits_combine(A, B, K, -149)
    for j in range(500):
        assert list(C[:, j]) == _digits_of_int(a_vals[j] + b_vals[j], K)


# ---------------------------------------------------------------- accumulate / finalize

def _python_chain(qrow, krow):
    acc = 0.0
    for a, b in zip(qrow, krow):
        acc = acc + a * b
    return acc


def test_accumulate_equals_exact_python_sums(oracle):
    """NUM/DEN digits equal Python-int exact sums of w*V, with w from exp_det
    (pinned above) of scores from an independent Python chain."""
    torch.manual_seed(0)
    for causal, dtype, (Hq, Hkv) in [(False, torch.float32, (2, 2)), (True, torch.bfloat16, (4, 2))]:
        S, D, scale = 9, 5, 0.3
        q, k, v = W.attn_inputs(21, 1, Hq, Hkv, S, S, D, dtype, std=2.0)
        m = oracle.attn_rowmax(q, k, 2, 8, causal, scale)
        num, den = oracle.attn_accumulate(q, k, v, m, 2, 8, causal, scale)
        qf, kf, vf = q.float().numpy(), k.float().numpy(), v.float().numpy()
        g = Hq // Hkv
        for h in range(Hq):
            for i in range(S):
                vis = [j for j in range(2, 8) if not causal or j <= i]
                ss = [float(np.float32(scale * _python_chain(qf[0, h, i].tolist(), kf[0, h // g, j].tolist())))
                      for j in vis]
                mm = max(ss) if ss else -math.inf
                assert m[0, h, i] == np.float32(mm)
                ws = [Fraction(float(np.float32(oracle.exp_det(s - mm)))) for s in ss]
                dexact = sum(ws, Fraction(0))
                assert _int_of_digits(den[:, 0, h, i]) == int(dexact * 2 ** 149)
                for d in range(D):
                    nexact = sum((w * Fraction(float(vf[0, h // g, j, d])) for w, j in zip(ws, vis)), Fraction(0))
                    assert _int_of_digits(num[:, 0, h, i, d]) == int(nexact * 2 ** 298)
                    assert num[:13, 0, h, i, d].min() >= 0


def test_finalize_rule(oracle):
    """out = RN32(RN64(NUM)/RN64(DEN)), checked with Python's correctly rounded
    int->float and IEEE division."""
    rng = random.Random(4)
    nums, dens = [], []
    for _ in range(300):
        nums.append(rng.getrandbits(300) - (1 << 299))
        dens.append(rng.getrandbits(170) + (1 << 149))
    N = np.array([_digits_of_int(v, 14) for v in nums], np.int64).T.reshape(14, 300, 1).copy()
    Dn = np.array([_digits_of_int(v, 9) for v in dens], np.int64).T.copy()
    out = oracle.attn_finalize(N, Dn)
    for j in range(300):
        n64 = float(Fraction(nums[j], 2 ** 298))
        d64 = float(Fraction(dens[j], 2 ** 149))
        assert out[j, 0] == np.float32(n64 / d64)


# ---------------------------------------------------------------- whole attention

def _fp64_attention(q, k, v, causal, scale):
    q, k, v = q.double(), k.double(), v.double()
    g = q.shape[1] // k.shape[1]
    k = k.repeat_interleave(g, 1)
    v = v.repeat_interleave(g, 1)
    s = (q @ k.transpose(-1, -2)) * scale
    if causal:
        S = q.shape[2]
        s = s.masked_fill(torch.ones(S, S, dtype=torch.bool).triu(1), -math.inf)
    return torch.softmax(s, -1) @ v


@pytest.mark.parametrize("D", [1, 3, 64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_oracle_matches_fp64_softmax_attention(oracle, D, causal, dtype):
    """Within 1e-6 absolute of fp64 softmax attention (the only rounding is the
    f32 score and the final f32 store)."""
    q, k, v = W.attn_inputs(100 + D, 2, 4, 2, 33, 33, D, dtype)
    scale = W.default_scale(D)
    out = oracle.det_attn(q, k, v, causal, scale)
    ref = _fp64_attention(q, k, v, causal, scale).numpy()
    assert np.abs(out - ref).max() <= 1e-6


def test_gqa_head_mapping_is_repeat_interleave(oracle):
    """Query head h reads KV head h // (Hq/Hkv): equal to MHA with K,V repeated."""
    q, k, v = W.attn_inputs(5, 1, 6, 2, 17, 17, 8, torch.float32)
    a = oracle.det_attn(q, k, v, True, 0.35)
    b = oracle.det_attn(q, k.repeat_interleave(3, 1), v.repeat_interleave(3, 1), True, 0.35)
    assert np.array_equal(a, b)


# ---------------------------------------------------------------- shard invariance

def _sharded(oracle, q, k, v, causal, scale, ranges, order):
    m = None
    for idx in order:
        lo, hi = ranges[idx]
        part = oracle.attn_rowmax(q, k, lo, hi, causal, scale)
        m = part if m is None else np.maximum(m, part)
    num = den = None
    for idx in order:
        lo, hi = ranges[idx]
        n_, d_ = oracle.attn_accumulate(q, k, v, m, lo, hi, causal, scale)
        if num is None:
            num, den = n_, d_
        else:
            num = oracle.digits_combine(num, n_, 14, -298).reshape(n_.shape)
            den = oracle.digits_combine(den, d_, 9, -149).reshape(d_.shape)
    return oracle.attn_finalize(num, den), m, num, den


def test_oracle_shard_invariance_all_orders(oracle):
    """kv_splits [32]*4 in all 24 composition orders == the unsplit result (config 1 shape)."""
    import itertools
    wl = W.attn_workload("tiny_mha_f32")
    q, k, v, scale = wl["q"], wl["k"], wl["v"], wl["scale"]
    ref, m0, n0, d0 = oracle.det_attn(q, k, v, False, scale, return_parts=True)
    ranges = W.kv_split_ranges([32] * 4)
    for order in itertools.permutations(range(4)):
        out, m, num, den = _sharded(oracle, q, k, v, False, scale, ranges, order)
        assert np.array_equal(num, n0) and np.array_equal(den, d0)
        assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))


def test_oracle_physical_block_permutation_noncausal(oracle):
    """Reordering K/V rows by whole blocks (non-causal) leaves the bits unchanged."""
    import itertools
    wl = W.attn_workload("tiny_mha_f32")
    q, k, v, scale = wl["q"], wl["k"], wl["v"], wl["scale"]
    ref = oracle.det_attn(q, k, v, False, scale)
    for perm in list(itertools.permutations(range(4)))[::5]:
        idx = torch.cat([torch.arange(32 * p, 32 * p + 32) for p in perm])
        out = oracle.det_attn(q, k[:, :, idx], v[:, :, idx], False, scale)
        assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))


def test_oracle_random_splits_causal_gqa(oracle):
    rng = random.Random(13)
    q, k, v = W.attn_inputs(77, 1, 4, 2, 40, 40, 16, torch.bfloat16)
    ref = oracle.det_attn(q, k, v, True, 0.25)
    for _ in range(6):
        cuts = sorted(rng.sample(range(1, 40), rng.randint(1, 6)))
        splits = [b - a for a, b in zip([0] + cuts, cuts + [40])]
        order = list(range(len(splits)))
        rng.shuffle(order)
        out, *_ = _sharded(oracle, q, k, v, True, 0.25, W.kv_split_ranges(splits), order)
        assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))


# ---------------------------------------------------------------- special cases

def test_special_cases(oracle):
    # one key: out = V exactly
    q, k, v = W.attn_inputs(8, 1, 2, 2, 5, 1, 16, torch.float32)
    out = oracle.det_attn(q, k, v, False, 0.25)
    assert np.array_equal(out, v.expand(1, 2, 5, 16).numpy())
    # causal row 0 sees only key 0
    q, k, v = W.attn_inputs(9, 1, 2, 1, 6, 6, 8, torch.bfloat16)
    out = oracle.det_attn(q, k, v, True, 0.3)
    assert np.array_equal(out[:, :, 0], v.float().numpy()[:, [0, 0], 0])
    # K = 0: every weight is 1, out = RN32(RN64(sum V)/n)
    q, k, v = W.attn_inputs(10, 1, 1, 1, 3, 7, 4, torch.float32)
    k = torch.zeros_like(k)
    out = oracle.det_attn(q, k, v, False, 0.5)
    vs = v.double().numpy()[0, 0]
    for d in range(4):
        exact = sum(Fraction(float(x)) for x in vs[:, d])
        assert out[0, 0, 0, d] == np.float32(float(exact) / 7.0)
    # V = 0: +0.0
    v0 = torch.zeros_like(v)
    out = oracle.det_attn(q, k, v0, False, 0.5)
    assert np.all(out == 0) and not np.any(np.signbit(out))
    # empty key range: rowmax -inf, zero digits; finalize of zero DEN gives NaN
    m = oracle.attn_rowmax(q, k, 3, 3, False, 0.5)
    assert np.all(np.isneginf(m))
    num, den = oracle.attn_accumulate(q, k, v, m, 3, 3, False, 0.5)
    assert not num.any() and not den.any()
    assert np.all(np.isnan(oracle.attn_finalize(num, den)))


# ---------------------------------------------------------------- cross-entropy

def _fp64_ce(x, t):
    xd = x.double().numpy()
    out = []
    for i in range(xd.shape[0]):
        m = xd[i].max()
        lse = m + math.log(math.fsum(np.exp(xd[i] - m).tolist()))
        out.append(lse - xd[i, t[i]])
    return np.array(out)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_ce_loss_and_grad_vs_fp64(oracle, dtype):
    x, t = W.ce_inputs(seed=31, N=64, V=3001, dtype=dtype)
    loss, m, denom = oracle.ce_forward(x, t)
    ref = _fp64_ce(x, t.numpy())
    assert np.abs(loss - ref).max() <= 2e-6
    xd = x.double()
    p = torch.softmax(xd, -1)
    onehot = torch.nn.functional.one_hot(t, x.shape[1]).double()
    g_none = oracle.ce_backward(x, t, m, denom, np.ones(64, np.float32), "none")
    gref = (p - onehot).numpy()
    assert np.abs(g_none - gref).max() <= 2e-7
    g_mean = oracle.ce_backward(x, t, m, denom, np.ones(1, np.float32), "mean")
    assert np.abs(g_mean - gref / 64).max() <= 5e-9
    g_sum = oracle.ce_backward(x, t, m, denom, np.full(1, 0.5, np.float32), "sum")
    assert np.abs(g_sum - gref * 0.5).max() <= 2e-7


def test_ce_reductions_are_exact_sums(oracle):
    rng = np.random.default_rng(2)
    loss = (rng.random(1000) * 10).astype(np.float32)
    exact = sum(Fraction(float(v)) for v in loss)
    assert oracle.ce_reduce(loss, "sum") == np.float32(float(exact))
    assert oracle.ce_reduce(loss, "mean") == np.float32(float(exact) / 1000.0)
    assert np.array_equal(oracle.ce_reduce(loss, "none"), loss)


def test_ce_closed_forms(oracle):
    # all logits equal: den = V, loss = log_det(V), within 1 ulp of ln V
    V = 1000
    x = torch.zeros(2, V)
    t = torch.tensor([0, 999])
    loss, m, denom = oracle.ce_forward(x, t)
    assert np.all(denom == V)
    assert np.all(loss == np.float32(oracle.log_det(float(V))))
    assert abs(oracle.log_det(float(V)) - math.log(V)) <= math.ulp(math.log(V))
    # a single vocabulary entry: loss 0, grad 0
    x1 = torch.randn(3, 1)
    l1, m1, d1 = oracle.ce_forward(x1, torch.zeros(3, dtype=torch.int64))
    assert np.all(l1 == 0)


def test_ce_vocab_split_invariance(oracle):
    x, t = W.ce_inputs(seed=33, N=32, V=4000, dtype=torch.bfloat16)
    ref_loss, ref_m, ref_den = oracle.ce_forward(x, t)
    for nsplit in (2, 4, 8):
        bounds = np.linspace(0, 4000, nsplit + 1).astype(int)
        shards = list(zip(bounds[:-1], bounds[1:]))
        order = W.shard_order(40 + nsplit, nsplit)
        m = np.max([oracle.ce_rowmax(x, lo, hi) for lo, hi in shards], axis=0)
        den = None
        for s in order:
            lo, hi = shards[s]
            part = oracle.ce_denom_digits(x, m, lo, hi)
            den = part if den is None else oracle.digits_combine(den, part, 9, -149).reshape(part.shape)
        loss, denom = oracle.ce_finalize(den, x, t, m)
        assert np.array_equal(loss.view(np.uint32), ref_loss.view(np.uint32))
        assert np.array_equal(denom, ref_den)


# ---------------------------------------------------------------- attention backward

def _fp64_backward(q, k, v, dO, causal, scale):
    """Gradients of plain fp64 softmax attention (torch autograd, CPU)."""
    Q, K, V = [t.double().requires_grad_() for t in (q, k, v)]
    g = q.shape[1] // k.shape[1]
    Kr, Vr = K.repeat_interleave(g, 1), V.repeat_interleave(g, 1)
    s = (Q @ Kr.transpose(-1, -2).contiguous()) * scale
    if causal:
        Sq = q.shape[2]
        s = s.masked_fill(~torch.ones(Sq, Sq, dtype=torch.bool).tril(), float("-inf"))
    (torch.softmax(s, -1) @ Vr).backward(dO.double())
    return Q.grad.numpy(), K.grad.numpy(), V.grad.numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_backward_matches_fp64_autograd(oracle, causal, dtype):
    """Within f32 rounding of the fp64 gradients: the scores, weights, p and ds
    are each rounded to f32 once (relative 2^-24) and the exact sums once more,
    so every gradient lies within 2^-20 (max|grad| + 1) of the fp64 value.  A
    dropped scale, a sign, or a transposed operand is off by O(1)."""
    q, k, v = W.attn_inputs(71, 1, 4, 2, 24, 24, 16, dtype)
    dO = torch.randn(1, 4, 24, 16, generator=torch.Generator().manual_seed(72))
    got = oracle.attn_backward(q, k, v, dO, causal, 0.25)
    ref = _fp64_backward(q, k, v, dO, causal, 0.25)
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        tol = 2.0 ** -20 * (np.abs(b).max() + 1)
        assert np.abs(a - b).max() <= tol, (name, np.abs(a - b).max(), tol)


def test_backward_single_key_closed_form(oracle):
    """One key: O = V_0 exactly, so delta_i equals dp_i0 bit for bit and every
    ds is 0 (dQ = dK = +0); p = 1, so dV_0 = RN32(RN64(exact sum of dO)) over
    all query heads and rows, which math.fsum rounds correctly."""
    q, k, v = W.attn_inputs(73, 1, 4, 2, 9, 1, 8, torch.float32)
    dO = torch.randn(1, 4, 9, 8, generator=torch.Generator().manual_seed(74))
    dq, dk, dv = oracle.attn_backward(q, k, v, dO, False, 0.3)
    assert not dq.any() and not np.signbit(dq).any()
    assert not dk.any() and not np.signbit(dk).any()
    for hk in range(2):
        for d in range(8):
            terms = [float(x) for x in dO[0, 2 * hk:2 * hk + 2, :, d].reshape(-1)]
            assert dv[0, hk, 0, d] == np.float32(math.fsum(terms))


def test_backward_zero_upstream(oracle):
    q, k, v = W.attn_inputs(75, 1, 2, 1, 12, 12, 8, torch.bfloat16)
    dq, dk, dv = oracle.attn_backward(q, k, v, torch.zeros(1, 2, 12, 8), True, 0.35)
    for g in (dq, dk, dv):
        assert not g.any() and not np.signbit(g).any()


def test_backward_uniform_scores_closed_form(oracle):
    """K = 0: every score is 0, every weight 1, and p_ij = RN32(1/n_i) with n_i
    the keys row i sees; dV_jd = RN32(exact sum of p_ij dO_id) (Fractions) and
    dQ = 0 (every term has a zero factor)."""
    q, k, v = W.attn_inputs(76, 1, 2, 1, 10, 10, 4, torch.float32)
    k = torch.zeros_like(k)
    dO = torch.randn(1, 2, 10, 4, generator=torch.Generator().manual_seed(77))
    for causal in (False, True):
        dq, dk, dv = oracle.attn_backward(q, k, v, dO, causal, 0.5)
        assert not dq.any()
        for j in range(10):
            for d in range(4):
                tot = Fraction(0)
                for h in range(2):
                    for i in range(10):
                        if causal and j > i:
                            continue
                        n = i + 1 if causal else 10
                        p = float(np.float32(1.0 / n))
                        tot += Fraction(p) * Fraction(float(dO[0, h, i, d]))
                assert dv[0, 0, j, d] == rn32_exact(tot), (causal, j, d)


def test_backward_sequence_permutations(oracle):
    """The sums over keys and over queries are exact: permuting K/V rows
    permutes dK/dV and leaves dQ's bits; permuting Q/dO rows permutes dQ and
    leaves dK/dV's bits (non-causal, where the order of rows carries no mask)."""
    q, k, v = W.attn_inputs(78, 1, 4, 2, 20, 28, 16, torch.bfloat16)
    dO = torch.randn(1, 4, 20, 16, generator=torch.Generator().manual_seed(79))
    base = oracle.attn_backward(q, k, v, dO, False, 0.25)
    pk = torch.randperm(28, generator=torch.Generator().manual_seed(80))
    dq, dk, dv = oracle.attn_backward(q, k[:, :, pk], v[:, :, pk], dO, False, 0.25)
    assert np.array_equal(dq.view(np.uint32), base[0].view(np.uint32))
    assert np.array_equal(dk.view(np.uint32), base[1][:, :, pk.numpy()].view(np.uint32))
    assert np.array_equal(dv.view(np.uint32), base[2][:, :, pk.numpy()].view(np.uint32))
    pq = torch.randperm(20, generator=torch.Generator().manual_seed(81))
    dq, dk, dv = oracle.attn_backward(q[:, :, pq], k, v, dO[:, :, pq].contiguous(), False, 0.25)
    assert np.array_equal(dq.view(np.uint32), base[0][:, :, pq.numpy()].view(np.uint32))
    assert np.array_equal(dk.view(np.uint32), base[1].view(np.uint32))
    assert np.array_equal(dv.view(np.uint32), base[2].view(np.uint32))


def test_backward_rounding_points_exact(oracle):
    """Every rounding point of the backward reading, recomputed independently
    in Python on a tiny causal GQA case: the chains as sequential Python float
    sums (each f32 x f32 product is exact in binary64, so a product-then-add
    chain equals the fma chain), w from the pinned exp_det, den64 from a
    Fraction sum, p and ds rounded to f32, and the three gradient sums as exact
    Fractions rounded once (dK and dQ rounded, scaled, rounded again).  The
    oracle must agree bit for bit; scaling before rounding the sum, or a
    dropped RN64, changes some of these bits."""
    B, Hq, Hkv, S, D, sc = 1, 2, 1, 6, 4, 0.35
    q, k, v = W.attn_inputs(82, B, Hq, Hkv, S, S, D, torch.float32)
    dO = torch.randn(B, Hq, S, D, generator=torch.Generator().manual_seed(83))
    dq, dk, dv = oracle.attn_backward(q, k, v, dO, True, sc)
    O = oracle.det_attn(q, k, v, True, sc)
    f = lambda t: [[[float(x) for x in row] for row in h] for h in t[0]]
    Q, K, V, G = f(q), f(k), f(v), f(dO)

    def chain(a, b):
        acc = 0.0
        for x, y in zip(a, b):
            acc = acc + x * y
        return acc

    P = {}
    DS = {}
    for h in range(Hq):
        for i in range(S):
            s = [float(np.float32(sc * chain(Q[h][i], K[0][j]))) for j in range(i + 1)]
            m = max(s)
            w = [float(np.float32(oracle.exp_det(x - m))) for x in s]
            den = float(sum(Fraction(x) for x in w))
            delta = chain(G[h][i], [float(x) for x in O[0, h, i]])
            for j in range(i + 1):
                p = float(np.float32(w[j] / den))
                P[h, i, j] = p
                DS[h, i, j] = float(np.float32(p * (chain(G[h][i], V[0][j]) - delta)))
    for d in range(D):
        for j in range(S):
            tv = sum((Fraction(P[h, i, j]) * Fraction(G[h][i][d]) for h in range(Hq) for i in range(j, S)), Fraction(0))
            tk = sum((Fraction(DS[h, i, j]) * Fraction(Q[h][i][d]) for h in range(Hq) for i in range(j, S)), Fraction(0))
            assert dv[0, 0, j, d] == np.float32(float(tv))  # RN32(RN64(exact sum))
            assert dk[0, 0, j, d] == np.float32(sc * float(tk))
        for h in range(Hq):
            for i in range(S):
                tq = sum((Fraction(DS[h, i, j]) * Fraction(K[0][j][d]) for j in range(i + 1)), Fraction(0))
                assert dq[0, h, i, d] == np.float32(sc * float(tq))


# ---------------------------------------------------------------- cross-entropy rounding points, bit for bit

def _bits32(x) -> int:
    return int(np.float32(x).view(np.uint32))


def _ce_pin_rows(seed: int, N: int, V: int):
    """bf16 logit rows that reach the rounding points where a regrouped rule
    shows: half the rows are the cross-entropy workload's distribution (2 N(0,1)
    with the target raised by 4); in the other half the target is the row max
    at magnitude 4..48 and every other logit lies at least 17..40 (drawn per
    row) below it, so the loss is a logsumexp excess of 1e-6..1e-16 computed
    next to a large m, and the target's probability is that close to 1."""
    x, t = W.ce_inputs(seed=seed, N=N, V=V, dtype=torch.float32)
    g = torch.Generator().manual_seed(seed + 1)
    for i in range(N // 2, N):
        big = float(torch.randint(8, 96, (1,), generator=g)) * 0.5 * (1 if i % 2 else -1)
        gmin = 17.0 + 23.0 * float(torch.rand(1, generator=g))
        gap = gmin + 13.0 * torch.rand(V, generator=g)
        row = big - gap
        row[t[i]] = big
        x[i] = row
    return x.to(torch.bfloat16), t


def test_ce_denom_digits_exact_on_random_rows(oracle):
    """den_i = the exact sum of RN32(exp_det(RN64(x - m))) over [v_lo, v_hi):
    recomputed term by term (Python float subtraction is RN64, exp_det is
    pinned above, numpy float32 is RN32) and summed as Fractions."""
    N, V = 12, 700
    x, t = _ce_pin_rows(71, N, V)
    xf = x.float().numpy().astype(np.float64)
    for lo, hi in [(0, V), (123, 517)]:
        m = oracle.ce_rowmax(x, lo, hi)
        den = oracle.ce_denom_digits(x, m, lo, hi)
        for i in range(N):
            assert _bits32(m[i]) == _bits32(max(xf[i, lo:hi].tolist()))
            ws = [Fraction(float(np.float32(oracle.exp_det(xv - float(m[i]))))) for xv in xf[i, lo:hi].tolist()]
            assert _int_of_digits(den[:, i]) == int(sum(ws, Fraction(0)) * 2 ** 149), (lo, hi, i)
            assert den[:8, i].min() >= 0 and den[:8, i].max() < 2 ** 32


def test_ce_finalize_rounding_points_bit_exact(oracle):
    """loss = RN32(RN64(RN64(m + log_det(den64)) - x_t)), den64 = RN64(den):
    den64 from Python's correctly rounded Fraction -> float, log_det pinned
    above, the two additions as Python float operations, RN32 by numpy.  The
    pin has power: on these rows the groupings m + (L - x_t), L + (m - x_t) and
    RN32(lse) - x_t each give other bits on some rows."""
    N, V = 40, 500
    x, t = _ce_pin_rows(72, N, V)
    xf = x.float().numpy().astype(np.float64)
    loss, m, denom = oracle.ce_forward(x, t)
    den = oracle.ce_denom_digits(x, m)
    alt = [0, 0, 0]
    for i in range(N):
        d64 = float(Fraction(_int_of_digits(den[:, i]), 2 ** 149))
        assert denom[i] == d64
        L = oracle.log_det(d64)
        mm, xt = float(m[i]), float(xf[i, int(t[i])])
        want = np.float32((mm + L) - xt)
        assert _bits32(loss[i]) == _bits32(want), i
        alt[0] += _bits32(np.float32(mm + (L - xt))) != _bits32(want)
        alt[1] += _bits32(np.float32(L + (mm - xt))) != _bits32(want)
        alt[2] += _bits32(np.float32(float(np.float32(mm + L)) - xt)) != _bits32(want)
    assert all(a > 0 for a in alt), alt


@pytest.mark.parametrize("reduction", ["none", "mean", "sum"])
def test_ce_backward_rounding_points_bit_exact(oracle, reduction):
    """grad = RN32(RN64(RN64(RN64(w / den64) - [v = t]) * c)) with c = g_i,
    RN64(g / N) or g: every operation recomputed in Python floats (each a
    binary64 IEEE operation) from the pinned exp_det and den64.  Power check:
    p*c - [v=t]*c (for the mean: c rounded to binary32), and p rounded to
    binary32 before the subtraction, give other bits on some entries."""
    N, V = 24, 300
    x, t = _ce_pin_rows(73, N, V)
    xf = x.float().numpy().astype(np.float64)
    loss, m, denom = oracle.ce_forward(x, t)
    rng = np.random.default_rng(74)
    gl = (rng.standard_normal(N if reduction == "none" else 1) * 3).astype(np.float32)
    if reduction == "mean":
        gl[0] = 1.0  # the usual upstream of a mean loss; 1/24 is not a binary32 value
    grad = oracle.ce_backward(x, t, m, denom, gl, reduction)
    alt = [0, 0]
    for i in range(N):
        g = float(gl[i if reduction == "none" else 0])
        c = g / N if reduction == "mean" else g
        for v in range(V):
            w = float(np.float32(oracle.exp_det(float(xf[i, v]) - float(m[i]))))
            p = w / float(denom[i])
            oh = 1.0 if v == int(t[i]) else 0.0
            want = np.float32((p - oh) * c)
            assert _bits32(grad[i, v]) == _bits32(want), (i, v)
            other = (p - oh) * float(np.float32(g / N)) if reduction == "mean" else p * c - oh * c
            alt[0] += _bits32(np.float32(other)) != _bits32(want)
            alt[1] += _bits32(np.float32((float(np.float32(p)) - oh) * c)) != _bits32(want)
    assert all(a > 0 for a in alt), alt


# ---------------------------------------------------------------- totalOrder max with signed zeros

def test_rowmax_total_order_signed_zero_bits(oracle):
    """The row max is IEEE totalOrder's (-0 < +0), compared as bit patterns.
    Attention: with f32 q = 2^-100 and k = -/+2^-100 the fp64 dot is -/+2^-200,
    whose RN32 score is -0 / +0; a key of -1 gives the normal score -2^-100.
    Cross-entropy: the same orders on bf16 logits."""
    f = np.float32
    q = torch.tensor([[[[2.0 ** -100]] * 4]], dtype=torch.float32)  # [1,1,4,1]
    cases = [  # keys of the row, expected rowmax bits
        ([-2.0 ** -100, 2.0 ** -100], 0x00000000),
        ([2.0 ** -100, -2.0 ** -100], 0x00000000),
        ([-2.0 ** -100, -1.0], 0x80000000),
        ([-1.0, -2.0 ** -100], 0x80000000),
    ]
    for keys, want in cases:
        k = torch.tensor(keys, dtype=torch.float32).reshape(1, 1, len(keys), 1)
        m = oracle.attn_rowmax(q, k, 0, len(keys), False, 1.0)
        assert all(_bits32(v) == want for v in m.reshape(-1)), (keys, [hex(_bits32(v)) for v in m.reshape(-1)])
    rows = [([-0.0, 0.0, -1.0], 0x00000000), ([0.0, -0.0], 0x00000000), ([-0.0, -1.0], 0x80000000),
            ([-1.0, -0.0, -3.0], 0x80000000), ([-0.0, -0.0], 0x80000000)]
    for vals, want in rows:
        x = torch.tensor([vals], dtype=torch.float32).to(torch.bfloat16)
        m = oracle.ce_rowmax(x)
        assert _bits32(m[0]) == want, (vals, hex(_bits32(m[0])))
        assert _bits32(f(max(vals, key=lambda z: (z, math.copysign(1, z))))) == want  # the pin's own reading
