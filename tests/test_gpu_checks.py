"""The library's input checks (det_debug_checks) and the out-of-range target
rule: a cross-entropy row whose target lies outside [0, V) reads no logit and
gets a NaN loss while every other output stays the same bits; with the checks
on, the call reports it.  det_attn_accumulate with the checks on refuses a
rowmax that lies below a visible score of its range and leaves num/den as they
were.  Targets outside the range sit on middle rows only, so that no read
could leave the logits' allocation."""
import sys

import numpy as np
import pytest
import torch

from bitwise_deterministic_exact_pass1_amd import _lib

pytestmark = pytest.mark.gpu

DET_E_VALUE = -7


def say(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def mods():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    from bitwise_deterministic_exact_pass1_amd import attention, cross_entropy
    return attention, cross_entropy


@pytest.fixture
def checks():
    _lib.input_checks(True)
    try:
        yield
    finally:
        _lib.input_checks(False)


def u32(x):
    return x.detach().cpu().contiguous().view(torch.int32).numpy()


def logits(N, V, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    x = (2.0 * torch.randn(N, V, generator=g)).to(dtype)
    t = torch.randint(0, V, (N,), generator=g, dtype=torch.int64)
    return x.cuda(), t.cuda()


# (dtype, V): the pattern-table kernel, the per-element bf16 kernel, f32
CE_CASES = [(torch.bfloat16, 16384), (torch.bfloat16, 1000), (torch.float32, 3000)]


@pytest.mark.parametrize("dtype,V", CE_CASES)
def test_forward_target_outside_the_vocabulary(mods, dtype, V):
    _, CE = mods
    N = 8
    say(f"checks: ce forward N={N} V={V} {dtype}")
    X, T = logits(N, V, dtype, 71 + V)
    loss0, m0, d0 = CE.forward(X, T)
    bad = T.clone()
    bad[2], bad[5] = -1, V
    loss, m, d = CE.forward(X, bad)
    torch.cuda.synchronize()
    assert torch.isnan(loss[2]) and torch.isnan(loss[5])
    keep = [i for i in range(N) if i not in (2, 5)]
    assert np.array_equal(u32(loss[keep]), u32(loss0[keep]))
    assert torch.equal(m, m0) and torch.equal(d, d0)


@pytest.mark.parametrize("dtype,V", CE_CASES)
def test_checks_report_targets_outside_the_vocabulary(mods, checks, dtype, V):
    _, CE = mods
    N = 8
    X, T = logits(N, V, dtype, 91 + V)
    ref = CE.forward(X, T)  # valid targets pass with the checks on
    bad = T.clone()
    bad[3] = V + 7
    with pytest.raises(_lib.DetError) as e:
        CE.forward(X, bad)
    assert e.value.code == DET_E_VALUE
    again = CE.forward(X, T)  # the count was cleared
    assert all(torch.equal(a, b) for a, b in zip(ref, again))


def test_finalize_target_outside_the_vocabulary(mods, checks):
    _, CE = mods
    N, V = 8, 16384
    X, T = logits(N, V, torch.bfloat16, 5)
    m = CE.rowmax(X)
    dg = CE.denom_digits(X, m)
    loss0, d0 = CE.finalize(dg, X, T, m)
    bad = T.clone()
    bad[4] = -3
    with pytest.raises(_lib.DetError) as e:
        CE.finalize(dg, X, bad, m)
    assert e.value.code == DET_E_VALUE
    _lib.input_checks(False)
    loss, d = CE.finalize(dg, X, bad, m)
    torch.cuda.synchronize()
    assert torch.isnan(loss[4])
    keep = [i for i in range(N) if i != 4]
    assert np.array_equal(u32(loss[keep]), u32(loss0[keep]))
    assert torch.equal(d, d0)


@pytest.mark.parametrize("causal", [False, True])
def test_accumulate_refuses_a_rowmax_below_a_score(mods, checks, causal):
    A, _ = mods
    say(f"checks: accumulate B=1 H=2 S=128 D=64 causal={causal}")
    g = torch.Generator().manual_seed(17)
    Q, K, V = (torch.randn(1, 2, 128, 64, generator=g).to(torch.bfloat16).cuda() for _ in range(3))
    kv_lo, kv_hi, q_lo, q_hi = 32, 96, 16, 112
    m = A.rowmax(Q, K, kv_lo, kv_hi, causal, q_lo=q_lo, q_hi=q_hi)
    m = torch.where(torch.isinf(m), torch.zeros_like(m), m)  # rows outside the range: any value
    num, den = A.accumulate(Q, K, V, m, kv_lo, kv_hi, causal, q_lo=q_lo, q_hi=q_hi)
    n0, d0 = num.clone(), den.clone()
    low = m.clone()
    row = 100  # sees keys 32..95 either way
    low[0, 1, row] = torch.nextafter(low[0, 1, row], torch.tensor(float("-inf"), device=low.device))
    with pytest.raises(_lib.DetError) as e:
        A.accumulate(Q, K, V, low, kv_lo, kv_hi, causal, num=num, den=den, q_lo=q_lo, q_hi=q_hi)
    assert e.value.code == DET_E_VALUE
    torch.cuda.synchronize()
    assert torch.equal(num, n0) and torch.equal(den, d0)
    # a rowmax above every score passes, and the switch off skips the check
    A.accumulate(Q, K, V, m + 1.0, kv_lo, kv_hi, causal, q_lo=q_lo, q_hi=q_hi)
    _lib.input_checks(False)
    A.accumulate(Q, K, V, low, kv_lo, kv_hi, causal, q_lo=q_lo, q_hi=q_hi)
    torch.cuda.synchronize()
