// qkrow.hpp -- statistics of a Q or K digit row and the test that decides,
// per (query row, key row) pair, whether the integer dot product computed on
// the matrix cores is the fp64 chain's result (the score rule: the fp64 fma
// chain over d ascending from +0, det-attn page, "Requirements and limits":
// fp64 scalar arithmetic).
//
// Every product q_d k_d of two bf16 values is exact in binary64, so the chain
// rounds only where a partial sum P_t = sum_{d<=t} q_d k_d is not a binary64
// number.  Each product is a multiple of 2^(lq_d + lk_d) (lq_d, lk_d: the lsb
// exponents of the entries), so every P_t is a multiple of 2^L with
// L = min_d (lq_d + lk_d), and |P_t| <= max|q| sum|k|.  If that bound is below
// 2^(L+53), every partial sum, and so the chain's result, is exact: it equals
// the exact dot product.  L is bounded below from per-row statistics: the
// smallest lsb exponent g of the row, the position p of an entry that has it,
// and the smallest lsb exponent g2 of the other entries; when the two rows'
// positions differ, L >= min(gq + gk2, gq2 + gk).
#pragma once

#include "dev_math.hpp"

namespace det {

// Row statistics as stored: int4 {g, digit count, log2 bound, p << 16 | (g2 & 0xffff)}.
// The bound is log2 of an upper bound of max|Xi| (Q rows) or of sum|Xi| (K
// rows), Xi = X 2^-g; g2 is +32767 for a row with at most one nonzero entry.
constexpr int kQKnoG2 = 32767;

__device__ __forceinline__ int qk_row_pack(int p, int g2) { return (p << 16) | (g2 & 0xffff); }
__device__ __forceinline__ int qk_row_g2(int w) { return (int)(int16_t)(w & 0xffff); }
__device__ __forceinline__ int qk_row_p(int w) { return (w >> 16) & 0xff; }

enum { kPairInt64 = 0, kPairInt128 = 1, kPairChain = 2 };

// How the score of the pair (Q row statistics qi, K row statistics ki, both
// with at most kmax digits or the pair goes to the chain) is obtained:
// kPairInt64: max|Qi| sum|Ki| < 2^53 on the grid 2^(gq+gk), so the integer
// dot product fits int64 and binary64 and is the chain's result;
// kPairInt128: the refined bound above holds, the dot product is the chain's
// result but may need more than 53 bits on that grid (composed in 128 bits);
// kPairChain: the chain itself.
// (branch-free: every operand is read and every test evaluated, then selected)
__device__ __forceinline__ int qk_pair_class(const int4 &qi, const int4 &ki, int kmax) {
    const bool digits = qi.y <= kmax && ki.y <= kmax;
    const bool crude = qi.z + ki.z <= 53;
    const int pq = qk_row_p(qi.w), pk = qk_row_p(ki.w);
    const int Lsame = qi.x + ki.x, Ldiff = min(qi.x + qk_row_g2(ki.w), qk_row_g2(qi.w) + ki.x);
    const int L = pq != pk ? Ldiff : Lsame;  // (both sides computed: a select, no branch)
    const int mag = qi.z + qi.x + ki.z + ki.x;  // log2 of a bound of max|q| sum|k|
    const bool fine = mag - L <= 53;
    return !digits ? kPairChain : crude ? kPairInt64 : fine ? kPairInt128 : kPairChain;
}

// The exact value dot 2^e of the integer dot product held in shift classes
// C[c][r] (dot = sum_c C_c 256^c over NC = 2 n - 1 int32 classes for n digits
// per row side, n = 3 or 4, each |C_c| < 2^24 for D <= 256), for a pair of
// class kPairInt64 or kPairInt128: dot = hi 2^32 + lo with lo = classes 0..3
// and hi = classes 4.., each formed by fma steps whose exact results are
// integers below 2^49 and 2^41 (so no step rounds); the value is a binary64
// number for either pair class, so the final fma hi 2^32 + lo, one rounding
// of that value, is exact, and so is the scaling by 2^e.
template <int NC>
__device__ __forceinline__ double qk_dot_value(const int __attribute__((ext_vector_type(4))) (&C)[NC], int r, int e) {
    static_assert(NC == 5 || NC == 7, "three or four digits per row side");
    const double lo =
        fma((double)C[3][r], 0x1p24, fma((double)C[2][r], 0x1p16, fma((double)C[1][r], 0x1p8, (double)C[0][r])));
    double hi = (double)C[4][r];
    if constexpr (NC == 7) hi = fma((double)C[6][r], 0x1p16, fma((double)C[5][r], 0x1p8, hi));
    return ldexp(fma(hi, 0x1p32, lo), e);
}

}  // namespace det
