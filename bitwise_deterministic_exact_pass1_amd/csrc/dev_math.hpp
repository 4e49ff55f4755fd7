// dev_math.hpp -- device-side numerics for gfx950: the fixed rounding rules of
// the exact two-pass softmax (det-attn page, "Method"; det-cross-entropy page,
// "Method"), total-order max keys, and exact conversions of radix-2^32 digit
// vectors.  All code is compiled with -ffp-contract=off: the only fused
// operations are the explicit fma() calls.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <climits>

namespace det {

// Digit formats: NUM 14 digits with lsb 2^-298, DEN (and CE den / loss sums)
// 9 digits with lsb 2^-149; radix 2^32, int64 digits, digit-major planes.
constexpr int kNumDigits = 14, kNumElo = -298;
constexpr int kDenDigits = 9, kDenElo = -149;

// RN64 of 1/ln2, ln2, ln2 - RN64(ln2), sqrt(2).
constexpr double kInvLn2 = 0x1.71547652b82fep+0;
constexpr double kLn2Hi = 0x1.62e42fefa39efp-1;
constexpr double kLn2Lo = 0x1.abc9e3b39803fp-56;
constexpr double kSqrt2 = 0x1.6a09e667f3bcdp+0;

// exp_det(t), t <= 0: t = n*ln2 + r with n = rint(t/ln2) (ties to even) and r
// from two fma steps against the split ln2; e^r by its Taylor series to r^13
// (coefficients RN64(1/k!)) in Horner form; times 2^n.  Zero below -104,
// where the f32 weight underflows to zero anyway.  FMA performs the Horner
// steps: any correctly rounded binary64 fused multiply-add.
constexpr double kExpC[14] = {
    1.0,                      // 1/0!
    1.0,                      // 1/1!
    0.5,                      // 1/2!
    0x1.5555555555555p-3,     // 1/3!
    0x1.5555555555555p-5,     // 1/4!
    0x1.1111111111111p-7,     // 1/5!
    0x1.6c16c16c16c17p-10,    // 1/6!
    0x1.a01a01a01a01ap-13,    // 1/7!
    0x1.a01a01a01a01ap-16,    // 1/8!
    0x1.71de3a556c734p-19,    // 1/9!
    0x1.27e4fb7789f5cp-22,    // 1/10!
    0x1.ae64567f544e4p-26,    // 1/11!
    0x1.1eed8eff8d898p-29,    // 1/12!
    0x1.6124613a86d09p-33,    // 1/13!
};

// Cody-Waite reduction of t: n and r with t = n ln2 + r.
__device__ __forceinline__ double exp_det_reduce(double t, double &n) {
    n = rint(t * kInvLn2);
    const double r = fma(-n, kLn2Hi, t);
    return fma(-n, kLn2Lo, r);
}

// The Horner steps of N independent arguments, step by step across them, so
// that their dependency chains interleave.
template <int N, class FMA>
__device__ __forceinline__ void exp_det_poly(const double (&r)[N], double (&p)[N], FMA fma_step) {
#pragma unroll
    for (int u = 0; u < N; ++u) p[u] = kExpC[13];
#pragma unroll
    for (int k = 12; k >= 0; --k) {
#pragma unroll
        for (int u = 0; u < N; ++u) p[u] = fma_step(p[u], r[u], kExpC[k]);
    }
}

template <class FMA>
__device__ __forceinline__ double exp_det_with(double t, FMA fma_step) {
    if (t < -104.0) return 0.0;
    double n;
    const double r[1] = {exp_det_reduce(t, n)};
    double p[1];
    exp_det_poly<1>(r, p, fma_step);
    return ldexp(p[0], (int)n);
}

struct FmaPlain {
    __device__ __forceinline__ double operator()(double a, double b, double c) const { return fma(a, b, c); }
};

// v_fma_f64 with three vector-register sources: the same IEEE operation as
// fma().  In a loop the constant addends then stay in registers hoisted out
// of it; plain fma() pairs each v_fmac_f64 with a copy of the constant.
struct FmaVreg {
    __device__ __forceinline__ double operator()(double a, double b, double c) const {
        double d;
        asm("v_fma_f64 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
        return d;
    }
};

__device__ __forceinline__ double exp_det(double t) { return exp_det_with(t, FmaPlain{}); }

// w = RN32(exp_det(RN64(s - m))).
template <class FMA = FmaPlain>
__device__ __forceinline__ float weight(float s, float m, FMA f = FMA{}) {
    return (float)exp_det_with((double)s - (double)m, f);
}

// log_det(x), x >= 1: x = f 2^e with f folded into (sqrt2/2, sqrt2];
// ln f = 2 atanh(u), u = (f-1)/(f+1), atanh(u)/u = sum_{k<=10} z^k/(2k+1), z = u^2;
// result e*ln2 + 2u*series, with ln2 split in two.
__device__ __forceinline__ double log_det(double x) {
    int e;
    double f = frexp(x, &e);  // x = f 2^e, f in [0.5, 1)
    f *= 2.0;
    e -= 1;
    if (f > kSqrt2) {
        f *= 0.5;
        e += 1;
    }
    const double u = (f - 1.0) / (f + 1.0);
    const double z = u * u;
    double q = 0x1.8618618618618p-5;       // 1/21
    q = fma(q, z, 0x1.af286bca1af28p-5);   // 1/19
    q = fma(q, z, 0x1.e1e1e1e1e1e1ep-5);   // 1/17
    q = fma(q, z, 0x1.1111111111111p-4);   // 1/15
    q = fma(q, z, 0x1.3b13b13b13b14p-4);   // 1/13
    q = fma(q, z, 0x1.745d1745d1746p-4);   // 1/11
    q = fma(q, z, 0x1.c71c71c71c71cp-4);   // 1/9
    q = fma(q, z, 0x1.2492492492492p-3);   // 1/7
    q = fma(q, z, 0x1.999999999999ap-3);   // 1/5
    q = fma(q, z, 0x1.5555555555555p-2);   // 1/3
    q = fma(q, z, 1.0);                    // 1/1
    const double ed = (double)e;
    return fma(ed, kLn2Hi, fma(ed, kLn2Lo, 2.0 * (u * q)));
}

// Value min/max of 64-bit integers (std::min returns a reference, which the
// compiler has been seen to keep in scratch memory when both operands are
// temporaries).
__device__ __forceinline__ int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }
__device__ __forceinline__ int64_t max64(int64_t a, int64_t b) { return a > b ? a : b; }

// A loaded value the compiler must materialise where this stands: a load in
// range for every lane, whose value a later select may drop, is otherwise
// moved into that select's branch with a wait of its own, so a batch of such
// loads would return one at a time.  Use after the whole batch is issued.
__device__ __forceinline__ float keep(float v) {
    asm volatile("" : "+v"(v));
    return v;
}

// ---------------------------------------------------------------- total order

// Monotone map of f32 onto uint32 under IEEE totalOrder (-0 < +0); NaNs are
// outside the contract.  max over keys == totalOrder max over floats.
__device__ __forceinline__ uint32_t order_key(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}
constexpr uint32_t kKeyNegInf = 0x007fffffu;  // order_key(-inf)

// ---------------------------------------------------------------- bf16 / f32

template <typename T> struct elem;
template <> struct elem<float> {
    __device__ static __forceinline__ float to_f32(float x) { return x; }
    static constexpr int mant_bits = 23;
};
struct bf16_t { uint16_t bits; };
template <> struct elem<bf16_t> {
    __device__ static __forceinline__ float to_f32(bf16_t x) { return __uint_as_float((uint32_t)x.bits << 16); }
    static constexpr int mant_bits = 7;
};

// floor(log2 |x|) for a nonzero finite f32 read from its bits; subnormals give
// -127, which is still a valid upper bound of the exponent for the grid logic
// below because their lsb is 2^-149 = 2^(-126-23).
__device__ __forceinline__ int f32_exp(float x) { return (int)((__float_as_uint(x) >> 23) & 0xff) - 127; }
__device__ __forceinline__ int f64_exp(double x) {
    return (int)((__double_as_longlong(x) >> 52) & 0x7ff) - 1023;
}

// ---------------------------------------------------------------- digit vectors

// Exact radix-2^32 contribution of the integer m * 2^sh (|m| < 2^53, 0 <= sh < 32)
// split into three limbs c0 + c1 2^32 + c2 2^64, each |c| < 2^32 and all with
// the sign of m.
struct limbs3 {
    int64_t c0, c1, c2;
};
__device__ __forceinline__ limbs3 split_limbs(int64_t m, int sh) {
    const bool neg = m < 0;
    const uint64_t a = neg ? (uint64_t)(-m) : (uint64_t)m;
    const uint64_t lo = a << sh;                            // low 64 bits of a*2^sh
    const uint64_t hi = sh ? (a >> (64 - sh)) : 0;          // bits 64.. (< 2^21)
    limbs3 r;
    r.c0 = (int64_t)(lo & 0xffffffffull);
    r.c1 = (int64_t)(lo >> 32);
    r.c2 = (int64_t)hi;
    if (neg) {
        r.c0 = -r.c0;
        r.c1 = -r.c1;
        r.c2 = -r.c2;
    }
    return r;
}

// Canonical form in place: d[0..K-2] in [0, 2^32), d[K-1] signed.  Exact while
// every |d[k]| < 2^62.
template <int K> __device__ __forceinline__ void canonicalize(int64_t (&d)[K]) {
#pragma unroll
    for (int k = 0; k < K - 1; ++k) {
        const int64_t c = d[k] >> 32;  // arithmetic shift: floor division
        d[k] -= c << 32;
        d[k + 1] += c;
    }
}

// Correctly rounded binary64 (ties to even) of X = sum_k d[k] 2^(32k + elo),
// with d canonical.  K <= 14.
template <int K> __device__ __forceinline__ double digits_to_f64(const int64_t (&dc)[K], int elo) {
    // magnitude limbs, all < 2^32, with two spare limbs for the signed top digit
    uint32_t L[K + 2];
    const bool neg = dc[K - 1] < 0;
    {
        // two's complement negation over (K-1) unsigned limbs + signed top
        uint64_t carry = neg ? 1 : 0;
#pragma unroll
        for (int k = 0; k < K - 1; ++k) {
            uint64_t v = (uint64_t)dc[k];
            if (neg) v = (~v) & 0xffffffffull;
            v += carry;
            L[k] = (uint32_t)v;
            carry = v >> 32;
        }
        int64_t top = dc[K - 1];
        uint64_t t = neg ? (uint64_t)(~top) + carry : (uint64_t)top;  // |top digit| after borrow
        L[K - 1] = (uint32_t)t;
        L[K] = (uint32_t)(t >> 32);
        L[K + 1] = 0;
    }
    int t = -1;
#pragma unroll
    for (int k = 0; k < K + 2; ++k)
        if (L[k]) t = k;
    if (t < 0) return 0.0;
    const int lz = __clz(L[t]);
    const int nb = 32 * t + (32 - lz);  // bit length
    double r;
    if (nb <= 64) {
        uint64_t m = 0;
#pragma unroll
        for (int k = 0; k < 2; ++k)
            if (k <= t) m |= (uint64_t)L[k] << (32 * k);
        if (nb <= 53) {
            r = ldexp((double)m, elo);
        } else {
            const int drop = nb - 53;
            const uint64_t keep = m >> drop;
            const uint64_t rem = m & ((1ull << drop) - 1);
            const uint64_t half = 1ull << (drop - 1);
            uint64_t mant = keep;
            if (rem > half || (rem == half && (keep & 1))) mant += 1;
            r = ldexp((double)mant, drop + elo);
        }
    } else {
        // top 96 bits from limbs t, t-1, t-2, shifted so the leading one is bit 95
        const uint32_t l2 = L[t], l1 = L[t - 1], l0 = (t >= 2) ? L[t - 2] : 0u;
        unsigned __int128 w = ((unsigned __int128)l2 << 64) | ((unsigned __int128)l1 << 32) | l0;
        w <<= lz;
        bool sticky = false;
        // bits of limb t-2 shifted out above are not lost (w has 128 bits); only
        // limbs below t-2 feed the sticky bit
#pragma unroll
        for (int k = 0; k < K + 2; ++k)
            if (k < t - 2 && L[k]) sticky = true;
        const uint64_t top64 = (uint64_t)(w >> 32);          // bits 95..32 of w
        const uint64_t below = (uint64_t)(w & 0xffffffffull);
        if (below) sticky = true;
        uint64_t mant = top64 >> 11;                         // 53 bits
        const uint64_t rbits = top64 & 0x7ffull;             // 11 dropped bits
        const bool round = (rbits >> 10) & 1;
        const bool rest = (rbits & 0x3ffull) || sticky;
        if (round && (rest || (mant & 1))) mant += 1;
        // value = mant * 2^(nb - 53) * 2^elo
        r = ldexp((double)mant, nb - 53 + elo);
    }
    return neg ? -r : r;
}

// ---------------------------------------------------------------- exact windows

// Add the exact window value acc (a multiple of 2^gexp, |acc| < 2^(gexp+53))
// into K radix-2^32 digits with lsb 2^elo at digits[k*plane].
template <int K>
__device__ __forceinline__ void flush_window(double acc, int gexp, int elo, int64_t *digits, int64_t plane) {
    if (acc == 0.0) return;
    const int64_t m = (int64_t)ldexp(acc, -gexp);  // exact integer, |m| < 2^53
    const int shift = gexp - elo;                  // >= 0 by construction
    const int k0 = shift >> 5;
    const limbs3 c = split_limbs(m, shift & 31);
    unsigned long long *dg = (unsigned long long *)digits;
    if (c.c0) atomicAdd(dg + (int64_t)k0 * plane, (unsigned long long)c.c0);
    if (c.c1) atomicAdd(dg + (int64_t)(k0 + 1) * plane, (unsigned long long)c.c1);
    if (c.c2) {
        if (k0 + 2 < K)
            atomicAdd(dg + (int64_t)(k0 + 2) * plane, (unsigned long long)c.c2);
        else  // only when k0 == K-2: fold the third limb into the (signed, wide) top digit
            atomicAdd(dg + (int64_t)(K - 1) * plane, (unsigned long long)(c.c2 << 32));
    }
}

// One exact window: terms t with |t| < 2^top and t a multiple of 2^lsb.
struct Window {
    double acc;
    int g;  // grid exponent; INT_MAX when empty
    __device__ __forceinline__ void init() {
        acc = 0.0;
        g = INT_MAX;
    }
    template <int K>
    __device__ __forceinline__ void add(double t, int lsb, int top, int gcap, int elo, int64_t *digits,
                                        int64_t plane) {
        lsb = min(lsb, gcap);
        const int ng = min(g, lsb);
        const int a = (acc != 0.0) ? f64_exp(acc) + 1 : INT_MIN;  // |acc| < 2^a
        if (max(a, top) <= ng + 52) {
            acc += t;  // exact: all terms on the 2^ng grid and |sum| < 2^(ng+53)
            g = ng;
        } else {
            flush_window<K>(acc, g, elo, digits, plane);
            acc = t;
            g = lsb;
        }
    }
    template <int K> __device__ __forceinline__ void flush(int elo, int64_t *digits, int64_t plane) {
        if (acc != 0.0) flush_window<K>(acc, g, elo, digits, plane);
        init();
    }
};

// Digit caps: the window grid never exceeds 2^gcap, so its lowest limb lands at
// digit <= K-2 and only the third limb can need folding into the top digit.
constexpr int kNumGcap = 32 * (kNumDigits - 2) + 31 + kNumElo;
constexpr int kDenGcap = 32 * (kDenDigits - 2) + 31 + kDenElo;

// ---------------------------------------------------------------- exact int128 helpers

__device__ __forceinline__ int clz128(unsigned __int128 u) {
    const uint64_t hi = (uint64_t)(u >> 64), lo = (uint64_t)u;
    return hi ? __clzll((long long)hi) : 64 + __clzll((long long)lo);
}

// Correctly rounded (ties to even) binary64 of N * 2^e for the 128-bit
// integer N = hi * 2^64 + lo (hi signed, lo unsigned); N * 2^e must lie in
// the normal range.  The top 64 bits of |N| are rounded by the (correctly
// rounded) uint64 conversion, with every lower bit folded into bit 0 as a
// sticky bit: bit 0 lies below the rounding position of a 64-bit value.
__device__ __forceinline__ double i128_to_f64(int64_t hi, uint64_t lo, int e) {
    // straight-line (selects only), so that a lane's conversions interleave
    const bool neg = hi < 0;
    const unsigned __int128 n = ((unsigned __int128)(uint64_t)hi << 64) | lo;
    const unsigned __int128 u = neg ? (unsigned __int128)0 - n : n;  // |N|
    const uint64_t uh = (uint64_t)(u >> 64), ul = (uint64_t)u;
    const int lz = uh ? __builtin_clzll(uh) : 64 + (ul ? __builtin_clzll(ul) : 64);
    const int s = max(64 - lz, 0);  // bits of |N| above the low 64: shift them out into the sticky bit
    const unsigned __int128 below = s ? (((unsigned __int128)1 << s) - 1) : 0;
    const uint64_t top = (uint64_t)(u >> s) | ((u & below) != 0 ? 1ull : 0ull);
    const double r = ldexp((double)top, e + s);
    return neg ? -r : r;
}

// Add x * 2^pos (pos >= 0, in units of the digit lsb) to K radix-2^32 digits.
template <int K>
__device__ __forceinline__ void add_i128_digits(__int128 x, int pos, int64_t *dg, int64_t plane) {
    if (x == 0) return;
    const bool neg = x < 0;
    unsigned __int128 u = neg ? (unsigned __int128)(-x) : (unsigned __int128)x;
    int k = pos >> 5;
    const int sh = pos & 31;
    // u * 2^sh < 2^(128+31): emit limbs of (u << sh) without losing the top bits
    const uint64_t top = sh ? (uint64_t)(u >> (128 - sh)) : 0;  // bits above 128 after the shift
    u <<= sh;
    unsigned long long *d = (unsigned long long *)dg;
    for (int t = 0; t < 5; ++t, ++k) {
        int64_t limb = t < 4 ? (int64_t)(uint32_t)(u >> (32 * t)) : (int64_t)top;
        if (!limb) continue;
        if (neg) limb = -limb;
        if (k < K) {
            atomicAdd(d + (int64_t)k * plane, (unsigned long long)limb);
        } else {  // fold into the signed top digit (only reached by values near the format's ceiling)
            atomicAdd(d + (int64_t)(K - 1) * plane, (unsigned long long)(limb << (32 * (k - (K - 1)))));
        }
    }
}

}  // namespace det
