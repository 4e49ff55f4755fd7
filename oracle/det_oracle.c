/*
 * det_oracle.c -- CPU oracle (TEST INFRASTRUCTURE ONLY; see det_oracle.h).
 *
 * Plain C, fp64, no blocking or fusion.  Exact sums use a 768-bit
 * two's-complement integer counted in units of 2^-298, which holds every
 * product of two f32 values exactly.  Parallelism is only over independent
 * output rows; no sum is split or reordered (and integer sums are exact, so
 * order could not matter anyway).
 *
 * Built with -ffp-contract=off so that every fma below is the only fused
 * operation: the score chain and the polynomials are written with explicit
 * fma() calls from libm (correctly rounded).
 */
#include "det_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

int32_t ora_version(void) { return 1; }

int32_t ora_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* Exact integer accumulator                                                 */
/* ------------------------------------------------------------------------ */

#define BIG_LIMBS 24      /* 24 x 32 = 768 bits */
#define BIG_UNIT (-298)   /* value = integer * 2^BIG_UNIT */

typedef struct { uint32_t w[BIG_LIMBS]; } big_t;

static void big_zero(big_t *a) { memset(a, 0, sizeof *a); }

static int big_is_negative(const big_t *a) { return (a->w[BIG_LIMBS - 1] >> 31) & 1; }

static int big_is_zero(const big_t *a) {
    for (int k = 0; k < BIG_LIMBS; k++)
        if (a->w[k]) return 0;
    return 1;
}

static void big_negate(big_t *a) {
    uint64_t carry = 1;
    for (int k = 0; k < BIG_LIMBS; k++) {
        uint64_t s = (uint64_t)(uint32_t)~a->w[k] + carry;
        a->w[k] = (uint32_t)s;
        carry = s >> 32;
    }
}

static void big_add(big_t *a, const big_t *b) {
    uint64_t carry = 0;
    for (int k = 0; k < BIG_LIMBS; k++) {
        uint64_t s = (uint64_t)a->w[k] + b->w[k] + carry;
        a->w[k] = (uint32_t)s;
        carry = s >> 32;
    }
}

/* a += (neg ? -1 : +1) * m * 2^sh, with sh >= 0 counted in units. */
static void big_add_mag(big_t *a, uint64_t m, int sh, int neg) {
    big_t t;
    big_zero(&t);
    int limb = sh / 32, bit = sh % 32;
    unsigned __int128 v = (unsigned __int128)m << bit; /* at most 96 bits */
    for (int k = 0; k < 3; k++) {
        uint32_t part = (uint32_t)(v >> (32 * k));
        if (!part) continue;
        if (limb + k >= BIG_LIMBS - 1) abort(); /* cannot happen for finite f32 inputs */
        t.w[limb + k] = part;
    }
    if (neg) big_negate(&t);
    big_add(a, &t);
}

/* a += x exactly.  x must be a finite double that is a multiple of 2^BIG_UNIT. */
static void big_add_double(big_t *a, double x) {
    if (x == 0.0) return;
    int e;
    double f = frexp(fabs(x), &e);          /* |x| = f * 2^e, f in [0.5, 1) */
    uint64_t m = (uint64_t)ldexp(f, 53);    /* exact 53-bit integer */
    int sh = e - 53 - BIG_UNIT;
    while (sh < 0) {                        /* drop trailing zero bits */
        if (m & 1) abort();                 /* x is below the accumulator's lsb */
        m >>= 1;
        sh++;
    }
    big_add_mag(a, m, sh, x < 0);
}

/* a += v * 2^(shift units), v a signed int64, shift >= 0. */
static void big_add_int64(big_t *a, int64_t v, int shift) {
    if (v == 0) return;
    uint64_t mag = v < 0 ? (uint64_t)0 - (uint64_t)v : (uint64_t)v;
    big_add_mag(a, mag, shift, v < 0);
}

static int big_bit(const big_t *a, int pos) { return (a->w[pos / 32] >> (pos % 32)) & 1; }

/* Correctly rounded (to nearest, ties to even) double of the exact value. */
static double big_to_double(const big_t *a0) {
    if (big_is_zero(a0)) return 0.0;
    big_t a = *a0;
    int neg = big_is_negative(&a);
    if (neg) big_negate(&a);
    int top = BIG_LIMBS * 32 - 1;
    while (!big_bit(&a, top)) top--;
    double r;
    if (top < 53) {
        uint64_t m = 0;
        for (int b = top; b >= 0; b--) m = (m << 1) | (uint64_t)big_bit(&a, b);
        r = ldexp((double)m, BIG_UNIT);
    } else {
        uint64_t m = 0;
        for (int b = top; b > top - 53; b--) m = (m << 1) | (uint64_t)big_bit(&a, b);
        int round = big_bit(&a, top - 53);
        int sticky = 0;
        for (int b = top - 54; b >= 0; b--) sticky |= big_bit(&a, b);
        if (round && (sticky || (m & 1))) m++;
        r = ldexp((double)m, top - 52 + BIG_UNIT); /* m == 2^53 is still exact */
    }
    return neg ? -r : r;
}

/* Canonical digits with lsb 2^E_lo: d_0..d_{K-2} in [0,2^32), d_{K-1} signed.
 * out[k * stride].  Returns -1 if the value is not a multiple of 2^E_lo or the
 * top digit does not fit an int64. */
static int big_to_digits(const big_t *a, int E_lo, int K, int64_t *out, int64_t stride) {
    int base = E_lo - BIG_UNIT;
    for (int b = 0; b < base; b++)
        if (big_bit(a, b)) return -1;
    for (int k = 0; k < K - 1; k++) {
        uint64_t d = 0;
        for (int b = 31; b >= 0; b--) d = (d << 1) | (uint64_t)big_bit(a, base + 32 * k + b);
        out[(int64_t)k * stride] = (int64_t)d;
    }
    /* top digit: bits from base + 32(K-1) upward, two's complement */
    int lo = base + 32 * (K - 1);
    int neg = big_is_negative(a);
    for (int b = lo + 63; b < BIG_LIMBS * 32; b++)
        if (big_bit(a, b) != neg) return -1; /* does not fit */
    uint64_t d = 0;
    for (int b = 63; b >= 0; b--) d = (d << 1) | (uint64_t)big_bit(a, lo + b);
    out[(int64_t)(K - 1) * stride] = (int64_t)d;
    return 0;
}

static void big_from_digits(big_t *a, const int64_t *digits, int64_t stride, int K, int E_lo) {
    big_zero(a);
    for (int k = 0; k < K; k++) big_add_int64(a, digits[(int64_t)k * stride], E_lo - BIG_UNIT + 32 * k);
}

/* ------------------------------------------------------------------------ */
/* Elementary routines                                                       */
/* ------------------------------------------------------------------------ */

/* Constants: RN64 of the named real numbers. */
static const double INV_LN2 = 0x1.71547652b82fep+0;  /* 1/ln 2 */
static const double LN2_HI = 0x1.62e42fefa39efp-1;   /* ln 2 */
static const double LN2_LO = 0x1.abc9e3b39803fp-56;  /* ln 2 - LN2_HI */
static const double SQRT2 = 0x1.6a09e667f3bcdp+0;    /* sqrt 2 */

/* 1/k!, k = 0..13 */
static const double INV_FACT[14] = {
    0x1p+0, 0x1p+0, 0x1p-1, 0x1.5555555555555p-3, 0x1.5555555555555p-5, 0x1.1111111111111p-7,
    0x1.6c16c16c16c17p-10, 0x1.a01a01a01a01ap-13, 0x1.a01a01a01a01ap-16, 0x1.71de3a556c734p-19,
    0x1.27e4fb7789f5cp-22, 0x1.ae64567f544e4p-26, 0x1.1eed8eff8d898p-29, 0x1.6124613a86d09p-33};

/* 1/(2k+1), k = 0..10 */
static const double INV_ODD[11] = {
    0x1p+0, 0x1.5555555555555p-2, 0x1.999999999999ap-3, 0x1.2492492492492p-3, 0x1.c71c71c71c71cp-4,
    0x1.745d1745d1746p-4, 0x1.3b13b13b13b14p-4, 0x1.1111111111111p-4, 0x1.e1e1e1e1e1e1ep-5,
    0x1.af286bca1af28p-5, 0x1.8618618618618p-5};

/* e^t for t <= 0: Cody-Waite reduction t = n ln2 + r (n nearest integer to
 * t/ln2, two-constant ln2), then the degree-13 Taylor polynomial of e^r in
 * Horner form, then scaling by 2^n.  Below -104 the f32 weight is 0. */
double ora_exp_det(double t) {
    if (t < -104.0) return 0.0;
    double n = rint(t * INV_LN2);
    double r = fma(-n, LN2_HI, t);
    r = fma(-n, LN2_LO, r);
    double p = INV_FACT[13];
    for (int k = 12; k >= 0; k--) p = fma(p, r, INV_FACT[k]);
    return ldexp(p, (int)n);
}

/* ln x for finite x >= 1 (the denominator is at least 1):
 * x = f 2^e with f in [1,2), folded to f in (sqrt2/2, sqrt2];
 * ln f = 2 atanh(u), u = (f-1)/(f+1), atanh(u) = u * sum_k u^(2k)/(2k+1). */
double ora_log_det(double x) {
    int e;
    double f = frexp(x, &e); /* x = f 2^e, f in [0.5, 1) */
    f = f * 2.0;
    e = e - 1; /* f in [1, 2) */
    if (f > SQRT2) {
        f = f / 2.0;
        e = e + 1;
    }
    double u = (f - 1.0) / (f + 1.0);
    double z = u * u;
    double q = INV_ODD[10];
    for (int k = 9; k >= 0; k--) q = fma(q, z, INV_ODD[k]);
    double ed = (double)e;
    return fma(ed, LN2_HI, fma(ed, LN2_LO, 2.0 * (u * q)));
}

/* ------------------------------------------------------------------------ */
/* Attention                                                                 */
/* ------------------------------------------------------------------------ */

/* bf16 is the top half of an f32; both widen exactly to double. */
static double ora_load(const ora_tensor *t, int64_t b, int64_t h, int64_t s, int64_t d) {
    int64_t off = b * t->sB + h * t->sH + s * t->sS + d;
    if (t->dtype == 0) return (double)((const float *)t->data)[off];
    uint32_t bits = (uint32_t)((const uint16_t *)t->data)[off] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static float max_total(float a, float b) {
    if (a > b) return a;
    if (b > a) return b;
    return signbit(a) ? b : a; /* equal values: +0 ranks above -0 */
}

float ora_score(const float *q, const float *k, int64_t D, double scale) {
    double acc = 0.0;
    for (int64_t d = 0; d < D; d++) acc = fma((double)q[d], (double)k[d], acc);
    return (float)(scale * acc);
}

static float score_at(const ora_tensor *q, const ora_tensor *k, int64_t b, int64_t hq, int64_t hk, int64_t i,
                      int64_t j, double scale) {
    double acc = 0.0;
    for (int64_t d = 0; d < q->D; d++) acc = fma(ora_load(q, b, hq, i, d), ora_load(k, b, hk, j, d), acc);
    return (float)(scale * acc);
}

static int shapes_ok(const ora_tensor *q, const ora_tensor *k, const ora_tensor *v, int64_t kv_lo, int64_t kv_hi,
                     int32_t causal) {
    if (q->B != k->B || q->D != k->D || k->H <= 0 || q->H % k->H != 0) return 0;
    if (v && (v->B != k->B || v->H != k->H || v->S != k->S || v->D != k->D)) return 0;
    if (kv_lo < 0 || kv_hi > k->S || kv_lo > kv_hi) return 0;
    if (causal && q->S != k->S) return 0;
    return 1;
}

/* key j visible to query i */
static int visible(int64_t i, int64_t j, int32_t causal) { return !causal || j <= i; }

int32_t ora_attn_rowmax_rows(const ora_tensor *q, const ora_tensor *k, int64_t n, const int64_t *rows,
                             int64_t kv_lo, int64_t kv_hi, int32_t causal, double scale, float *rowmax) {
    if (!shapes_ok(q, k, NULL, kv_lo, kv_hi, causal)) return -1;
    int64_t group = q->H / k->H;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t r = 0; r < n; r++) {
        int64_t b = rows[3 * r], hq = rows[3 * r + 1], i = rows[3 * r + 2];
        int64_t hk = hq / group;
        float m = -INFINITY;
        for (int64_t j = kv_lo; j < kv_hi; j++)
            if (visible(i, j, causal)) m = max_total(m, score_at(q, k, b, hq, hk, i, j, scale));
        rowmax[r] = m;
    }
    return 0;
}

int32_t ora_attn_accumulate_rows(const ora_tensor *q, const ora_tensor *k, const ora_tensor *v, int64_t n,
                                 const int64_t *rows, const float *rowmax, int64_t kv_lo, int64_t kv_hi,
                                 int32_t causal, double scale, int64_t *num, int64_t *den) {
    if (!shapes_ok(q, k, v, kv_lo, kv_hi, causal)) return -1;
    const int64_t D = q->D, group = q->H / k->H;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 4) reduction(| : failed)
    for (int64_t r = 0; r < n; r++) {
        int64_t b = rows[3 * r], hq = rows[3 * r + 1], i = rows[3 * r + 2];
        int64_t hk = hq / group;
        double m = (double)rowmax[r];
        big_t *acc = (big_t *)calloc((size_t)D, sizeof(big_t));
        big_t dsum;
        big_zero(&dsum);
        for (int64_t j = kv_lo; j < kv_hi; j++) {
            if (!visible(i, j, causal)) continue;
            float s = score_at(q, k, b, hq, hk, i, j, scale);
            float w = (float)ora_exp_det((double)s - m);
            big_add_double(&dsum, (double)w);
            for (int64_t d = 0; d < D; d++) big_add_double(&acc[d], (double)w * ora_load(v, b, hk, j, d));
        }
        for (int64_t d = 0; d < D; d++)
            failed |= big_to_digits(&acc[d], ORA_NUM_ELO, ORA_NUM_DIGITS, num + r * D + d, n * D) != 0;
        failed |= big_to_digits(&dsum, ORA_DEN_ELO, ORA_DEN_DIGITS, den + r, n) != 0;
        free(acc);
    }
    return failed ? -1 : 0;
}

/* ------------------------------------------------------------------------ */
/* Attention backward (the reading stated in det_oracle.h)                   */
/* ------------------------------------------------------------------------ */

/* Per query row of the forward over all keys: rowmax, RN64(DEN), and delta =
 * the fp64 fma chain of dO . O with O the f32 output. */
static void backward_row_stats(const ora_tensor *q, const ora_tensor *k, const ora_tensor *v,
                               const ora_tensor *dout, int64_t b, int64_t hq, int64_t hk, int64_t i, int32_t causal,
                               double scale, float *m_out, double *den_out, double *delta_out) {
    const int64_t D = q->D;
    float m = -INFINITY;
    for (int64_t j = 0; j < k->S; j++)
        if (visible(i, j, causal)) m = max_total(m, score_at(q, k, b, hq, hk, i, j, scale));
    big_t *num = (big_t *)calloc((size_t)D, sizeof(big_t));
    big_t den;
    big_zero(&den);
    for (int64_t j = 0; j < k->S; j++) {
        if (!visible(i, j, causal)) continue;
        float w = (float)ora_exp_det((double)score_at(q, k, b, hq, hk, i, j, scale) - (double)m);
        big_add_double(&den, (double)w);
        for (int64_t d = 0; d < D; d++) big_add_double(&num[d], (double)w * ora_load(v, b, hk, j, d));
    }
    double den64 = big_to_double(&den), delta = 0.0;
    for (int64_t d = 0; d < D; d++) {
        float o = (float)(big_to_double(&num[d]) / den64);
        delta = fma(ora_load(dout, b, hq, i, d), (double)o, delta);
    }
    free(num);
    *m_out = m;
    *den_out = den64;
    *delta_out = delta;
}

/* p_ij and ds_ij of one visible pair. */
static void backward_pair(const ora_tensor *q, const ora_tensor *k, const ora_tensor *v, const ora_tensor *dout,
                          int64_t b, int64_t hq, int64_t hk, int64_t i, int64_t j, double scale, float m,
                          double den64, double delta, float *p_out, float *ds_out) {
    float w = (float)ora_exp_det((double)score_at(q, k, b, hq, hk, i, j, scale) - (double)m);
    float p = (float)((double)w / den64);
    double dp = 0.0;
    for (int64_t d = 0; d < q->D; d++) dp = fma(ora_load(dout, b, hq, i, d), ora_load(v, b, hk, j, d), dp);
    *p_out = p;
    *ds_out = (float)((double)p * (dp - delta));
}

int32_t ora_attn_backward(const ora_tensor *q, const ora_tensor *k, const ora_tensor *v, const ora_tensor *dout,
                          int32_t causal, double scale, float *dq, float *dk, float *dv) {
    if (!shapes_ok(q, k, v, 0, k->S, causal)) return -1;
    if (dout->dtype != 0 || dout->B != q->B || dout->H != q->H || dout->S != q->S || dout->D != q->D) return -1;
    const int64_t B = q->B, Hq = q->H, Hkv = k->H, Sq = q->S, Skv = k->S, D = q->D, group = Hq / Hkv;
    const int64_t nq = B * Hq * Sq;
    float *m = (float *)malloc((size_t)(nq ? nq : 1) * sizeof(float));
    double *den = (double *)malloc((size_t)(nq ? nq : 1) * sizeof(double));
    double *delta = (double *)malloc((size_t)(nq ? nq : 1) * sizeof(double));
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t r = 0; r < nq; r++) {
        int64_t b = r / (Hq * Sq), hq = (r / Sq) % Hq, i = r % Sq;
        backward_row_stats(q, k, v, dout, b, hq, hq / group, i, causal, scale, &m[r], &den[r], &delta[r]);
    }
    /* dQ: exact sum over the keys of each query row */
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t r = 0; r < nq; r++) {
        int64_t b = r / (Hq * Sq), hq = (r / Sq) % Hq, i = r % Sq, hk = hq / group;
        big_t *acc = (big_t *)calloc((size_t)D, sizeof(big_t));
        for (int64_t j = 0; j < Skv; j++) {
            if (!visible(i, j, causal)) continue;
            float p, ds;
            backward_pair(q, k, v, dout, b, hq, hk, i, j, scale, m[r], den[r], delta[r], &p, &ds);
            for (int64_t d = 0; d < D; d++) big_add_double(&acc[d], (double)ds * ora_load(k, b, hk, j, d));
        }
        for (int64_t d = 0; d < D; d++) dq[r * D + d] = (float)(scale * big_to_double(&acc[d]));
        free(acc);
    }
    /* dK, dV: exact sums over the (query head, row) pairs that see each key */
    const int64_t nk = B * Hkv * Skv;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t c = 0; c < nk; c++) {
        int64_t b = c / (Hkv * Skv), hk = (c / Skv) % Hkv, j = c % Skv;
        big_t *ak = (big_t *)calloc((size_t)D, sizeof(big_t));
        big_t *av = (big_t *)calloc((size_t)D, sizeof(big_t));
        for (int64_t g = 0; g < group; g++) {
            int64_t hq = hk * group + g;
            for (int64_t i = 0; i < Sq; i++) {
                if (!visible(i, j, causal)) continue;
                int64_t r = (b * Hq + hq) * Sq + i;
                float p, ds;
                backward_pair(q, k, v, dout, b, hq, hk, i, j, scale, m[r], den[r], delta[r], &p, &ds);
                for (int64_t d = 0; d < D; d++) {
                    big_add_double(&ak[d], (double)ds * ora_load(q, b, hq, i, d));
                    big_add_double(&av[d], (double)p * ora_load(dout, b, hq, i, d));
                }
            }
        }
        for (int64_t d = 0; d < D; d++) {
            dk[c * D + d] = (float)(scale * big_to_double(&ak[d]));
            dv[c * D + d] = (float)big_to_double(&av[d]);
        }
        free(ak);
        free(av);
    }
    free(m);
    free(den);
    free(delta);
    return 0;
}

void ora_attn_finalize(const int64_t *num, const int64_t *den, int64_t n, int64_t D, float *out) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; r++) {
        big_t a;
        big_from_digits(&a, den + r, n, ORA_DEN_DIGITS, ORA_DEN_ELO);
        double dv = big_to_double(&a);
        for (int64_t d = 0; d < D; d++) {
            big_from_digits(&a, num + r * D + d, n * D, ORA_NUM_DIGITS, ORA_NUM_ELO);
            double nv = big_to_double(&a);
            out[r * D + d] = (float)(nv / dv);
        }
    }
}

int32_t ora_digits_combine(int64_t *acc, const int64_t *part, int64_t n, int32_t K, int32_t E_lo) {
    int failed = 0;
#pragma omp parallel for schedule(static) reduction(| : failed)
    for (int64_t r = 0; r < n; r++) {
        big_t a, b;
        big_from_digits(&a, acc + r, n, K, E_lo);
        big_from_digits(&b, part + r, n, K, E_lo);
        big_add(&a, &b);
        failed |= big_to_digits(&a, E_lo, K, acc + r, n) != 0;
    }
    return failed ? -1 : 0;
}

void ora_digits_to_double(const int64_t *digits, int64_t n, int32_t K, int32_t E_lo, double *out) {
    for (int64_t r = 0; r < n; r++) {
        big_t a;
        big_from_digits(&a, digits + r, n, K, E_lo);
        out[r] = big_to_double(&a);
    }
}

int32_t ora_double_to_digits(const double *x, int64_t n, int32_t K, int32_t E_lo, int64_t *digits) {
    for (int64_t r = 0; r < n; r++) {
        big_t a;
        big_zero(&a);
        big_add_double(&a, x[r]);
        if (big_to_digits(&a, E_lo, K, digits + r, n)) return -1;
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Cross-entropy                                                             */
/* ------------------------------------------------------------------------ */

static double ce_load(const void *logits, int32_t dtype, int64_t ld, int64_t i, int64_t v) {
    int64_t off = i * ld + v;
    if (dtype == 0) return (double)((const float *)logits)[off];
    uint32_t bits = (uint32_t)((const uint16_t *)logits)[off] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

void ora_ce_rowmax(const void *logits, int32_t dtype, int64_t N, int64_t ld, int64_t v_lo, int64_t v_hi,
                   float *rowmax) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < N; i++) {
        float m = -INFINITY;
        for (int64_t v = v_lo; v < v_hi; v++) m = max_total(m, (float)ce_load(logits, dtype, ld, i, v));
        rowmax[i] = m;
    }
}

void ora_ce_denom_digits(const void *logits, int32_t dtype, int64_t N, int64_t ld, const float *rowmax,
                         int64_t v_lo, int64_t v_hi, int64_t *den) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < N; i++) {
        big_t a;
        big_zero(&a);
        double m = (double)rowmax[i];
        for (int64_t v = v_lo; v < v_hi; v++) {
            float w = (float)ora_exp_det(ce_load(logits, dtype, ld, i, v) - m);
            big_add_double(&a, (double)w);
        }
        if (big_to_digits(&a, ORA_DEN_ELO, ORA_DEN_DIGITS, den + i, N)) abort();
    }
}

void ora_ce_finalize(const int64_t *den, const void *logits, int32_t dtype, int64_t N, int64_t ld,
                     const int64_t *targets, const float *rowmax, float *loss, double *denom) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < N; i++) {
        big_t a;
        big_from_digits(&a, den + i, N, ORA_DEN_DIGITS, ORA_DEN_ELO);
        double d64 = big_to_double(&a);
        double lse = (double)rowmax[i] + ora_log_det(d64);
        double xt = ce_load(logits, dtype, ld, i, targets[i]);
        loss[i] = (float)(lse - xt);
        denom[i] = d64;
    }
}

void ora_ce_reduce(const float *loss, int64_t N, int32_t reduction, float *out) {
    if (reduction == 0) {
        for (int64_t i = 0; i < N; i++) out[i] = loss[i];
        return;
    }
    big_t a;
    big_zero(&a);
    for (int64_t i = 0; i < N; i++) big_add_double(&a, (double)loss[i]);
    double s = big_to_double(&a);
    out[0] = reduction == 1 ? (float)(s / (double)N) : (float)s;
}

void ora_ce_backward(const void *logits, int32_t dtype, int64_t N, int64_t V, int64_t ld, const int64_t *targets,
                     const float *rowmax, const double *denom, const float *grad_loss, int32_t reduction,
                     float *grad, int64_t grad_ld) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < N; i++) {
        double c;
        if (reduction == 0) c = (double)grad_loss[i];
        else if (reduction == 1) c = (double)grad_loss[0] / (double)N;
        else c = (double)grad_loss[0];
        double m = (double)rowmax[i];
        for (int64_t v = 0; v < V; v++) {
            float w = (float)ora_exp_det(ce_load(logits, dtype, ld, i, v) - m);
            double p = (double)w / denom[i];
            double g = p - (v == targets[i] ? 1.0 : 0.0);
            grad[i * grad_ld + v] = (float)(g * c);
        }
    }
}
