/*
 * det_oracle.h -- CPU oracle for shard-invariant exact softmax attention and
 * deterministic cross-entropy.
 *
 * TEST INFRASTRUCTURE ONLY.  This library is the plain, slow, obviously
 * correct definition that the GPU library is checked against.  Only the test
 * suite, the smoke check and the benchmark's CPU-baseline leg may load it.
 * It shares no code, header, constant table or helper with the GPU library.
 *
 * What it computes follows the det-attn page ("Method": a global row max,
 * then exact long-accumulator sums of the exp-weighted values and of the
 * denominator) and the det-cross-entropy page ("Method": global row max, exact
 * denominator, loss = logsumexp - target logit, gradient softmax - onehot).
 * Every rounding point the pages leave open is fixed as follows:
 *
 *   score    s = RN32( RN64( scale * dot ) ),
 *            dot = fp64 fma chain over d = 0,1,..,D-1 starting at +0.0
 *   rowmax   IEEE totalOrder max (-0 < +0) of the visible s; empty -> -inf
 *   weight   w = RN32( exp_det( RN64(s - m) ) )        (exp_det below)
 *   sums     DEN = sum w, NUM_d = sum w * V_d, both exact (no rounding at all)
 *   digits   X = sum_k d_k 2^(32k + E_lo), radix 2^32 int64 digits,
 *            NUM: E_lo = -298, 14 digits;  DEN / CE den / CE loss sum:
 *            E_lo = -149, 9 digits.  Canonical: d_0..d_{K-2} in [0,2^32),
 *            d_{K-1} signed.  Planes are digit-major: [k][row][d].
 *   finalize out = RN32( RN64(NUM) / RN64(DEN) )   (0/0 -> NaN)
 *
 * Cross-entropy (per token row i, vocab range [v_lo, v_hi)):
 *   m = totalOrder max x;  w = RN32(exp_det(RN64(x - m)));  den = sum w exact
 *   den64 = RN64(den);  lse = RN64(m + log_det(den64));
 *   loss = RN32(RN64(lse - x[t]))
 *   reductions: none; sum = RN32(RN64(S)); mean = RN32(RN64(RN64(S) / N)),
 *   S = exact sum of the f32 losses.
 *   grad = RN32( RN64( RN64( RN64(w / den64) - [v == t] ) * c ) ),
 *   c = g_i (none), g (sum), RN64(g / N) (mean).
 */
#ifndef DET_ORACLE_H
#define DET_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* One attention operand.  data points at f32 (dtype 0) or bf16 (dtype 1)
 * elements; element (b,h,s,d) sits at b*sB + h*sH + s*sS + d. */
typedef struct {
    const void *data;
    int32_t dtype;
    int64_t B, H, S, D;
    int64_t sB, sH, sS;
} ora_tensor;

enum { ORA_NUM_DIGITS = 14, ORA_NUM_ELO = -298, ORA_DEN_DIGITS = 9, ORA_DEN_ELO = -149 };

int32_t ora_version(void);

/* Threads the row loops run on (OpenMP). */
int32_t ora_threads(void);

/* The two elementary routines, exported so tests can pin them. */
double ora_exp_det(double t);
double ora_log_det(double x);

/* Score of one query row against one key row (both f32 values, length D). */
float ora_score(const float *q, const float *k, int64_t D, double scale);

/* rows: n triplets (b, hq, i).  Returns 0, or -1 on a precondition failure. */
int32_t ora_attn_rowmax_rows(const ora_tensor *q, const ora_tensor *k, int64_t n, const int64_t *rows,
                             int64_t kv_lo, int64_t kv_hi, int32_t causal, double scale, float *rowmax);

/* Exact NUM/DEN digits of the keys in [kv_lo, kv_hi) for the given rows,
 * weighted against the caller's rowmax (one per row).
 * num: [14][n][D] canonical, den: [9][n] canonical. */
int32_t ora_attn_accumulate_rows(const ora_tensor *q, const ora_tensor *k, const ora_tensor *v, int64_t n,
                                 const int64_t *rows, const float *rowmax, int64_t kv_lo, int64_t kv_hi,
                                 int32_t causal, double scale, int64_t *num, int64_t *den);

/* out[n][D] = RN32(RN64(NUM)/RN64(DEN)); num [14][n][D], den [9][n];
 * any digit values whose exact sum fits are accepted (not only canonical). */
void ora_attn_finalize(const int64_t *num, const int64_t *den, int64_t n, int64_t D, float *out);

/* acc = canonical(acc + part) over n values of K digits with lsb 2^E_lo.
 * Returns 0, or -1 if the top digit would overflow int64. */
int32_t ora_digits_combine(int64_t *acc, const int64_t *part, int64_t n, int32_t K, int32_t E_lo);

/* RN64 of each digit-array value (planes [K][n]). */
void ora_digits_to_double(const int64_t *digits, int64_t n, int32_t K, int32_t E_lo, double *out);

/* Canonical digits of each double value (values must be multiples of
 * 2^E_lo); planes [K][n].  Returns 0 or -1. */
int32_t ora_double_to_digits(const double *x, int64_t n, int32_t K, int32_t E_lo, int64_t *digits);

/* Attention backward over the whole key range (no page gives a backward rule;
 * the reading fixed here keeps every sum over the sequence axes exact, so any
 * sharding of queries or keys gives the same bits):
 *   forward  m_i, den64_i = RN64(DEN_i), O_i as above (all keys)
 *   delta_i  = fp64 fma chain over d of dO_id * O_id, from +0.0
 *   dp_ij    = fp64 fma chain over d of dO_id * V_jd, from +0.0
 *   p_ij     = RN32( RN64( w_ij / den64_i ) )
 *   ds_ij    = RN32( RN64( p_ij * RN64( dp_ij - delta_i ) ) )
 *   dV_jd    = RN32( RN64( sum p_ij dO_id ) )            exact sum over the visible
 *   dK_jd    = RN32( RN64( scale * RN64( sum ds_ij Q_id ) ) )   (query head, row)
 *   dQ_id    = RN32( RN64( scale * RN64( sum ds_ij K_jd ) ) )   exact sum over keys
 * (dK, dV sum over the query heads that share key head hk).  dout: f32
 * [B,Hq,Sq,D].  Outputs are contiguous f32: dq [B,Hq,Sq,D], dk and dv
 * [B,Hkv,Skv,D].  Returns 0, or -1 on a precondition failure. */
int32_t ora_attn_backward(const ora_tensor *q, const ora_tensor *k, const ora_tensor *v, const ora_tensor *dout,
                          int32_t causal, double scale, float *dq, float *dk, float *dv);

/* Cross-entropy.  logits: dtype 0 f32 / 1 bf16, row i at logits + i*ld. */
void ora_ce_rowmax(const void *logits, int32_t dtype, int64_t N, int64_t ld, int64_t v_lo, int64_t v_hi,
                   float *rowmax);
void ora_ce_denom_digits(const void *logits, int32_t dtype, int64_t N, int64_t ld, const float *rowmax,
                         int64_t v_lo, int64_t v_hi, int64_t *den);
void ora_ce_finalize(const int64_t *den, const void *logits, int32_t dtype, int64_t N, int64_t ld,
                     const int64_t *targets, const float *rowmax, float *loss, double *denom);
/* reduction: 0 none (out[N] = loss), 1 mean, 2 sum (out[0]). */
void ora_ce_reduce(const float *loss, int64_t N, int32_t reduction, float *out);
/* grad_loss: [N] for reduction none, [1] otherwise. grad row i at grad + i*grad_ld. */
void ora_ce_backward(const void *logits, int32_t dtype, int64_t N, int64_t V, int64_t ld, const int64_t *targets,
                     const float *rowmax, const double *denom, const float *grad_loss, int32_t reduction,
                     float *grad, int64_t grad_ld);

#ifdef __cplusplus
}
#endif
#endif
