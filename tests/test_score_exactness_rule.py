"""The rule that decides when the integer dot product computed on the matrix
cores is the fp64 chain's score (the det-attn page's score is an fp64 sum;
the rule is restated here from its derivation, not imported): every product
q_d k_d of two bf16 values is exact in binary64; each is a multiple of
2^(lq_d + lk_d); so every partial sum is a multiple of 2^L, L = min_d
(lq_d + lk_d), and at most max|q| sum|k| in magnitude; when that bound is
below 2^(L+53) no partial sum rounds and the chain equals the exact dot
product.  L is bounded below by per-row statistics (smallest lsb exponent g,
its position p, the second smallest g2): L >= min(gq + gk2, gq2 + gk) when
the positions differ, else gq + gk.

The test checks the claim by brute force on bf16 rows built to sit on both
sides of the bound (single tiny entries, shared and distinct positions),
against a Python float chain and Fraction sums, and checks the split
composition of the dot product from its shift classes."""
import math
import random
from fractions import Fraction

import numpy as np
import torch


def _lsb(x):
    """lsb exponent of a bf16 value (8 significant bits), None for 0."""
    if x == 0:
        return None
    e = math.frexp(abs(x))[1] - 1
    return max(e, -126) - 7


def _row_stats(row):
    ls = [(_lsb(x), d) for d, x in enumerate(row) if x != 0]
    if not ls:
        return 0, 0, 32767, 0
    ls.sort()
    g, p = ls[0]
    g2 = ls[1][0] if len(ls) > 1 else 32767
    emax = max(math.frexp(abs(x))[1] - 1 for x in row if x != 0)
    return g, p, g2, emax


def _q_bound(row):
    g, p, g2, emax = _row_stats(row)
    return emax + 1 - g  # max|q| < 2^(bound + g)


def _k_bound(row):
    g, p, g2, emax = _row_stats(row)
    s = sum(abs(Fraction(x)) for x in row) / Fraction(2) ** g
    return max(int(s).bit_length(), 0) if s else 0  # sum|k| < 2^(bound + g)


def _pair_exact_by_rule(q, k):
    gq, pq, gq2, _ = _row_stats(q)
    gk, pk, gk2, _ = _row_stats(k)
    qb, kb = _q_bound(q), _k_bound(k)
    if qb + kb <= 53:
        return True
    L = min(gq + gk2, gq2 + gk) if pq != pk else gq + gk
    return qb + gq + kb + gk - L <= 53


def _chain(q, k):
    acc = 0.0
    for a, b in zip(q, k):
        acc = acc + a * b  # exact product, one rounding per step: the fma chain
    return acc


def _bf16_row(rng, D, tiny):
    x = torch.randn(D, generator=rng)
    for pos, e in tiny:
        x[pos] = float(torch.randn(1, generator=rng)) * 2.0 ** e
    return [float(v) for v in x.to(torch.bfloat16).float()]


def test_rule_implies_the_chain_is_exact():
    """Whenever the rule says exact, the chain equals the exact dot product;
    the rows are drawn so that both verdicts occur, and the refined bound
    (distinct tiny-entry positions) admits pairs the plain bound rejects."""
    rng = torch.Generator().manual_seed(5)
    prng = random.Random(6)
    counts = {"plain": 0, "refined": 0, "rejected": 0}
    for _ in range(3000):
        D = prng.choice([16, 64, 128])
        tq = [(prng.randrange(D), -prng.randint(8, 40))] if prng.random() < 0.7 else []
        tk = [(prng.randrange(D), -prng.randint(8, 40))] if prng.random() < 0.7 else []
        if tq and tk and prng.random() < 0.3:
            tk = [(tq[0][0], tk[0][1])]  # same position: the refined bound does not apply
        q, k = _bf16_row(rng, D, tq), _bf16_row(rng, D, tk)
        exact = sum((Fraction(a) * Fraction(b) for a, b in zip(q, k)), Fraction(0))
        plain = _q_bound(q) + _k_bound(k) <= 53
        if _pair_exact_by_rule(q, k):
            counts["plain" if plain else "refined"] += 1
            assert Fraction(_chain(q, k)) == exact
        else:
            counts["rejected"] += 1
    assert counts["refined"] > 100 and counts["rejected"] > 50, counts


def _fma(a, b, c):
    """binary64 fused multiply-add: the exact a*b + c, rounded once to nearest even."""
    return float(Fraction(a) * Fraction(b) + Fraction(c))


def _compose(C, e):
    """The kernels' composition of the shift classes C_0.. (3 or 4 digits per
    side: 5 or 7 classes): lo = classes 0..3 and hi = the rest, each by fma
    steps, then fma(hi, 2^32, lo) scaled by 2^e."""
    lo = _fma(float(C[3]), 2.0 ** 24, _fma(float(C[2]), 2.0 ** 16, _fma(float(C[1]), 2.0 ** 8, float(C[0]))))
    hi = float(C[4])
    if len(C) == 7:
        hi = _fma(float(C[6]), 2.0 ** 16, _fma(float(C[5]), 2.0 ** 8, hi))
    return math.ldexp(_fma(hi, 2.0 ** 32, lo), e)


def test_split_composition_of_the_shift_classes_is_exact():
    """dot = sum_c C_c 256^c over five or seven int32 classes (|C_c| <= 2^24)
    equals hi 2^32 + lo with lo from classes 0..3 and hi from the rest; every
    fma step forming lo and hi is exact (integers below 2^49 and 2^41), and
    the final fma is exact whenever the value itself is a binary64 number.
    A regrouping that rounds earlier (classes summed high to low, or hi and lo
    split elsewhere) fails on the draws with many significant bits."""
    rng = random.Random(7)
    checked = 0
    for _ in range(20000):
        nc = rng.choice([5, 7])
        # |C_c| <= 2^24: four digit pairs per class, 256 dimensions, |digit product| <= 2^14;
        # half the draws are multiples of 2^sh (few significant bits: often representable)
        sh = rng.randrange(0, 24) if rng.random() < 0.5 else 0
        C = [rng.randrange(-(1 << (24 - sh)), (1 << (24 - sh)) + 1) << sh for _ in range(nc)]
        dot = sum(c << (8 * i) for i, c in enumerate(C))
        lo = C[0] + (C[1] << 8) + (C[2] << 16) + (C[3] << 24)
        hi = sum(C[c] << (8 * (c - 4)) for c in range(4, nc))
        assert abs(lo) < 2 ** 49 and abs(hi) < 2 ** 41 and hi * 2 ** 32 + lo == dot
        e = rng.randrange(-200, 0)
        exact = Fraction(dot) * Fraction(2) ** e
        got = _compose(C, e)
        if Fraction(float(exact)) == exact:  # representable
            assert Fraction(got) == exact
            checked += 1
        else:  # one rounding of the exact value
            assert got == float(exact)
    assert checked > 2000, checked
