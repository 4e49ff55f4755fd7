/*
 * det_attn.h -- C ABI of the MI355X (gfx950) library for shard-invariant exact
 * softmax attention and deterministic cross-entropy.
 *
 * The operation follows the det-attn page, section "Method": a global row max
 *     rowmax_i = max_j s_ij,   s_ij = scale * Q_i . K_j,
 * then exact long-accumulator sums
 *     NUM_id = sum_j w_ij V_jd,   DEN_i = sum_j w_ij,   w_ij = exp(s_ij - rowmax_i),
 * where KV shards compose by an elementwise max (rowmax) and an int64 add of
 * digit arrays (NUM/DEN), and "finalize" turns digits into the f32 output
 * (same page, "API" table: det_attn, rowmax, accumulate, finalize,
 * det_attn_sharded).  The det-cross-entropy page, section "Method", applies
 * the same two reductions over a vocabulary axis (API table: forward, rowmax,
 * denom_digits, finalize).
 *
 * Rounding points (the pages leave them open; every result below is a fixed
 * function of the inputs, bit for bit):
 *   s    = RN32(RN64(scale * dot)), dot = fp64 fma chain over d = 0..D-1 from +0
 *   max  = IEEE totalOrder max (-0 < +0); a row with no visible key: -inf
 *   w    = RN32(exp_det(RN64(s - m))), exp_det = Cody-Waite reduction with
 *          n = rint(t/ln2), then the degree-13 Taylor polynomial in Horner
 *          form, times 2^n; exactly 0 for t < -104
 *   sums = exact (every w*V product is exact in binary64 and no sum rounds)
 *   out  = RN32(RN64(NUM) / RN64(DEN))    (a row with no visible key: NaN)
 *
 * Digit arrays ("Kulisch long accumulators"): X = sum_k d_k 2^(32k + E_lo),
 * int64 digits in radix 2^32, digit-major planes.
 *   NUM  : 14 digits, E_lo = -298, layout [14][B][Hq][Sq][D]
 *   DEN  :  9 digits, E_lo = -149, layout [9][B][Hq][Sq]
 *   CE den:  9 digits, E_lo = -149, layout [9][N]
 * Every array the library writes is canonical: digits 0..K-2 in [0, 2^32), the
 * top digit signed.  Inputs to combine/finalize may be any sum of up to 2^30
 * canonical arrays (for example an elementwise int64 add done by the caller).
 *
 * Conventions for every entry point:
 *   - Returns DET_OK (0) or a negative DET_E_* code; det_last_error() gives a
 *     thread-local message.  Argument checks run on the host before any HIP
 *     call, so they are testable without a GPU.
 *   - Pointers marked (device) are device memory; the caller owns every buffer.
 *     Nothing is allocated by the library except where a workspace size query
 *     says so; the caller passes that workspace (device, 256-byte aligned).
 *   - `stream` is a hipStream_t (NULL = default stream); all work is enqueued
 *     on it asynchronously, in a fixed launch configuration, so repeated calls
 *     give identical bits.
 *   - Q, K, V share one dtype (DET_F32 or DET_BF16); D <= 256; Hq % Hkv == 0;
 *     query head h reads KV head h / (Hq/Hkv).  Causal means key j is visible
 *     to query i iff j <= i (absolute indices) and requires Sq == Skv.
 *   - Inputs must be finite.  The preconditions on caller-supplied row maxima
 *     and targets are checked only under det_debug_checks(1).
 */
#ifndef DET_ATTN_H
#define DET_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { DET_F32 = 0, DET_BF16 = 1 };

enum {
    DET_OK = 0,
    DET_E_NULL = -1,      /* a required pointer is NULL */
    DET_E_SHAPE = -2,     /* sizes disagree, D outside [1,256], Hq % Hkv != 0, bad range, causal with Sq != Skv */
    DET_E_DTYPE = -3,     /* dtype not DET_F32/DET_BF16, or operands differ */
    DET_E_STRIDE = -4,    /* negative stride or an unsupported layout */
    DET_E_WORKSPACE = -5, /* workspace missing, too small, or misaligned */
    DET_E_HIP = -6,       /* a HIP runtime call or launch failed */
    DET_E_VALUE = -7      /* other invalid argument (reduction code, split list) */
};

enum { DET_NUM_DIGITS = 14, DET_NUM_ELO = -298, DET_DEN_DIGITS = 9, DET_DEN_ELO = -149 };

/* An attention operand [B, H, S, D]: element (b,h,s,d) at
 * data + (b*sB + h*sH + s*sS + d) elements (device memory, D stride 1).
 * The interleaved NHD layout of a fused QKV projection is expressed with
 * strides (sB, sH, sS) = (S*row, D, row). */
typedef struct {
    const void *data;
    int32_t dtype;
    int64_t B, H, S, D;
    int64_t sB, sH, sS;
} det_tensor;

/* f32 output [B, Hq, Sq, D] with D stride 1 (device memory). */
typedef struct {
    float *data;
    int64_t sB, sH, sS;
} det_out;

/* Digit format of NUM (which = 0) or DEN / CE den (which = 1). */
int det_digit_format(int32_t which, int32_t *n_digits, int32_t *lsb_exp2);

const char *det_last_error(void);

/* Per-kernel timing (a tracing aid; results never depend on it).
 * det_profile_begin(): from now on every kernel the library launches is
 * bracketed by two HIP events recorded on the stream it runs on.
 * det_profile_end(buf, len): waits for those events, writes one line
 * "kernel_name launches total_ms" per kernel into buf (NUL-terminated,
 * truncated to len), switches recording off and returns the full length
 * needed (including the NUL).  Not meant to be called while other threads
 * launch work through the library. */
int det_profile_begin(void);
size_t det_profile_end(char *buf, size_t len);

/* Testing aid (results never depend on it): with on != 0, every later call
 * sends every tile of the exact sums through the library's generic exact path
 * instead of the matrix-core path, until it is called again with 0.  Both
 * paths compute the same exact sums, so the outputs are bit-identical; the
 * switch lets tests check that.  Process-wide; returns DET_OK. */
int det_debug_force_generic(int32_t on);

/* Input checks (for debugging; results never depend on it): with on != 0,
 * every later call of det_attn_accumulate verifies on the device that no
 * visible score of its range lies above the supplied rowmax, and every later
 * det_ce_forward / det_ce_finalize that every target lies in [0, V).  These
 * calls then wait for their stream and return DET_E_VALUE on a violation:
 * det_attn_accumulate before touching num/den, the cross-entropy calls after
 * writing their outputs.  The accumulate check computes the range's row
 * maxima in memory it allocates (hipMalloc) for the check.  on = 0 (the
 * default) turns the checks off.  Process-wide; returns DET_OK. */
int det_debug_checks(int32_t on);

/* Testing aid (results never depend on it): pass 2 of bf16 attention with
 * head dims up to 128 has two kernel layouts with the same exact sums --
 * weight-making and multiplying waves on 32-key blocks, or every wave doing
 * both on 64-key blocks.  mode 0 (the default) picks by the key range's
 * length; 1 and 2 force the eight-wave and the split layout for every later
 * call.  Process-wide; DET_E_VALUE for another mode, else DET_OK. */
int det_debug_pass2_layout(int32_t mode);

/* Testing aid (results never depend on it): pass 2 of bf16 attention reads
 * the scores pass 1 kept in the workspace, or recomputes them from the digit
 * rows pass 1 prepared (no O(rows x keys) buffer).  mode 0 (the default)
 * keeps them whenever one 32-row tile's share fits the workspace; 1 keeps
 * and 2 recomputes for every later call.  Process-wide; DET_E_VALUE for
 * another mode, else DET_OK.  (Forcing 1 can make a small workspace fail the
 * size check with DET_E_WORKSPACE.) */
int det_debug_score_source(int32_t mode);

/* ---------------------------------------------------------------- attention */

/* det-attn page, "API": det_attn(Q, K, V, causal, scale) -- the whole path
 * (global rowmax, exact NUM/DEN over all keys, finalize) in one call.
 * Workspace: det_attn_workspace_size() bytes, or more; a larger workspace
 * lets the library process more query rows per launch (never changes bits). */
size_t det_attn_workspace_size(const det_tensor *q, const det_tensor *k, const det_tensor *v, int32_t causal);
int det_attn(const det_tensor *q, const det_tensor *k, const det_tensor *v, int32_t causal, double scale,
             const det_out *o, void *workspace, size_t ws_bytes, void *stream);

/* det_attn for callers that cannot allocate device memory (code under graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation and the same bits as det_attn, with no workspace argument.  Its
 * scratch is the library's own fixed device array of DET_NOALLOC_BYTES
 * (64 MiB), one per GPU the library runs on, held until the process ends; the
 * call allocates nothing.  Query rows are taken in chunks that fit it; a
 * problem whose smallest chunk (32 query rows) does not fit gets
 * DET_E_WORKSPACE before anything is launched.  Every call on one GPU uses
 * that GPU's one array, so calls that overlap on a GPU (other threads or
 * streams) race and must be serialized by the caller; nothing in the array
 * needs to start at zero.  Other errors as det_attn. */
enum { DET_NOALLOC_BYTES = 64 << 20 };
int det_attn_noalloc(const det_tensor *q, const det_tensor *k, const det_tensor *v, int32_t causal, double scale,
                     const det_out *o, void *stream);

/* det_attn plus the two per-row values its gradients need (det-attn page,
 * "Method": the global row max and the exact denominator): rowmax (device)
 * f32 [B][Hq][Sq] and den64 (device) f64 [B][Hq][Sq] = RN64(DEN).  Same
 * workspace as det_attn; o is bit-identical to det_attn's. */
int det_attn_stats(const det_tensor *q, const det_tensor *k, const det_tensor *v, int32_t causal, double scale,
                   const det_out *o, float *rowmax, double *den64, void *workspace, size_t ws_bytes, void *stream);

/* Gradients of det_attn over the whole key range.  The pages give no
 * backward rule; this one keeps every sum over the sequence axes exact (the
 * det-attn page's "Method" property), so any sharding of queries or keys
 * gives the same bits.  With w and den64 as in the forward:
 *   delta_i = fp64 fma chain over d of dO_id O_id;  dp_ij = the chain of dO_id V_jd
 *   p_ij = RN32(RN64(w_ij / den64_i));  ds_ij = RN32(RN64(p_ij RN64(dp_ij - delta_i)))
 *   dV_jd = RN32(RN64(sum p_ij dO_id)), dK_jd = RN32(RN64(scale RN64(sum ds_ij Q_id))),
 *   dQ_id = RN32(RN64(scale RN64(sum ds_ij K_jd))), every sum exact (dK and dV
 *   over all query heads that share the key head).
 * q, k, v: as det_attn.  o: the forward output and dout: its gradient, both
 * DET_F32 [B][Hq][Sq][D] (any strides, D stride 1).  rowmax, den64: (device)
 * from det_attn_stats.  dq: f32 [B][Hq][Sq][D]; dk, dv: f32 [B][Hkv][Skv][D]
 * (caller-owned device memory, D stride 1).  Rows without a visible key get
 * dq = 0.  Workspace: det_attn_backward_workspace_size() bytes or more (more
 * lets the library take more query rows per launch; bits never change). */
size_t det_attn_backward_workspace_size(const det_tensor *q, const det_tensor *k, const det_tensor *v,
                                        int32_t causal);
int det_attn_backward(const det_tensor *q, const det_tensor *k, const det_tensor *v, const det_tensor *o,
                      const det_tensor *dout, const float *rowmax, const double *den64, int32_t causal,
                      double scale, const det_out *dq, const det_out *dk, const det_out *dv, void *workspace,
                      size_t ws_bytes, void *stream);

/* det-attn page, "API": rowmax(Q, K, ..., kv_lo, kv_hi) -- per-query max
 * score over keys [kv_lo, kv_hi) (combine shards by max), for the query rows
 * [q_lo, q_hi) (absolute row indices; 0 <= q_lo <= q_hi <= Sq, else
 * DET_E_SHAPE).  rowmax: (device) f32 [B][Hq][Sq]; only rows in [q_lo, q_hi)
 * of each head are written, the others are left as they are.  Workspace:
 * det_attn_rowmax_workspace_size() with the same ranges. */
size_t det_attn_rowmax_workspace_size(const det_tensor *q, const det_tensor *k, int64_t q_lo, int64_t q_hi,
                                      int64_t kv_lo, int64_t kv_hi);
int det_attn_rowmax(const det_tensor *q, const det_tensor *k, int64_t q_lo, int64_t q_hi, int64_t kv_lo,
                    int64_t kv_hi, int32_t causal, double scale, float *rowmax, void *workspace, size_t ws_bytes,
                    void *stream);

/* det-attn page, "API": accumulate(Q, K, V, rowmax, ...) -- exact NUM/DEN
 * digits of keys [kv_lo, kv_hi) weighted against `rowmax` (which must be
 * >= every visible score, normally the composed global max), for the query
 * rows [q_lo, q_hi) (absolute; range rules as for det_attn_rowmax).
 * rowmax: (device) f32 [B][Hq][Sq] (rows in range are read);
 * num: (device) int64 [14][B][Hq][Sq][D]; den: (device) int64 [9][B][Hq][Sq].
 * Only rows in [q_lo, q_hi) of each head are touched: add_into = 0
 * overwrites them; 1 adds this shard to what they hold.  Those rows are
 * canonical afterwards either way. */
size_t det_attn_accumulate_workspace_size(const det_tensor *q, const det_tensor *k, const det_tensor *v,
                                          int64_t q_lo, int64_t q_hi, int64_t kv_lo, int64_t kv_hi);
int det_attn_accumulate(const det_tensor *q, const det_tensor *k, const det_tensor *v, const float *rowmax,
                        int64_t q_lo, int64_t q_hi, int64_t kv_lo, int64_t kv_hi, int32_t causal, double scale,
                        int64_t *num, int64_t *den, int32_t add_into, void *workspace, size_t ws_bytes,
                        void *stream);

/* Shard composition (det-attn page, "Method": max and int64 add).
 * det_rowmax_combine: acc[i] = totalOrder max(acc[i], part[i]), n values (device).
 * det_digits_combine: acc = canonical(acc + part) for n_values values of
 * n_digits digits each, planes [n_digits][n_values] (device). */
int det_rowmax_combine(float *acc, const float *part, int64_t n, void *stream);
int det_digits_combine(int64_t *acc, const int64_t *part, int64_t n_values, int32_t n_digits, void *stream);

/* Carry normalization of a digit array (det-attn page, "Method": shards
 * compose by int64 add; the page's caller-side sum of digit arrays is not
 * canonical): acc <- canonical(acc) in place, the same exact value, for
 * n_values values of n_digits (14 or 9, else DET_E_VALUE) digits, planes
 * [n_digits][n_values] (device).  Exact while every |digit| < 2^62 (any sum
 * of up to 2^30 canonical arrays). */
int det_digits_normalize(int64_t *acc, int64_t n_values, int32_t n_digits, void *stream);

/* det-attn page, "API": finalize(NUM, DEN, shape) -- out = RN32(RN64(NUM)/RN64(DEN)).
 * num [14][B][Hq][Sq][D], den [9][B][Hq][Sq] (device). */
int det_attn_finalize(const int64_t *num, const int64_t *den, int64_t B, int64_t Hq, int64_t Sq, int64_t D,
                      const det_out *o, void *stream);

/* det-attn page, "API": det_attn_sharded(Q, K, V, kv_splits, ...) -- the
 * KV-shard composition: rowmax per shard, combined by max; digits per shard
 * against the global max, combined by int64 add in `order` (NULL = 0,1,..);
 * finalize.  Bit-identical to det_attn for every split and order.
 * kv_splits: (host) n_splits shard lengths summing to Skv; order: (host)
 * permutation of 0..n_splits-1 or NULL. */
size_t det_attn_sharded_workspace_size(const det_tensor *q, const det_tensor *k, const det_tensor *v,
                                       const int64_t *kv_splits, int32_t n_splits, int32_t causal);
int det_attn_sharded(const det_tensor *q, const det_tensor *k, const det_tensor *v, const int64_t *kv_splits,
                     int32_t n_splits, const int32_t *order, int32_t causal, double scale, const det_out *o,
                     void *workspace, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------ cross-entropy */
/* det-cross-entropy page.  logits: (device) [N][V] of dtype DET_F32 or
 * DET_BF16, row i at logits + i*ld elements; targets: (device) int64 [N] in
 * [0, V).  A row whose target lies outside [0, V) reads no logit for it and
 * gets a NaN loss (det_debug_checks reports it).  Reduction codes: 0 none,
 * 1 mean, 2 sum. */

/* "API": rowmax(logits, v_lo, v_hi) -- per-token max over [v_lo, v_hi). rowmax: (device) f32 [N]. */
int det_ce_rowmax(const void *logits, int32_t dtype, int64_t N, int64_t ld, int64_t v_lo, int64_t v_hi,
                  float *rowmax, void *stream);

/* "API": denom_digits(logits, global_rowmax, v_lo, v_hi) -- exact
 * den_i = sum_v RN32(exp_det(x_iv - m_i)) over [v_lo, v_hi).
 * den: (device) int64 [9][N]; add_into as for det_attn_accumulate. */
int det_ce_denom_digits(const void *logits, int32_t dtype, int64_t N, int64_t ld, const float *rowmax,
                        int64_t v_lo, int64_t v_hi, int64_t *den, int32_t add_into, void *stream);

/* "API": finalize(den_digits, logits, targets, global_rowmax) -> (loss, denom):
 * denom_i = RN64(den_i); loss_i = RN32(RN64(RN64(m_i + log_det(denom_i)) - x_{i,t_i})),
 * log_det = 2*atanh((f-1)/(f+1)) series on f in (sqrt2/2, sqrt2] plus e*ln2.
 * loss: (device) f32 [N]; denom: (device) f64 [N]. */
int det_ce_finalize(const int64_t *den, const void *logits, int32_t dtype, int64_t N, int64_t V, int64_t ld,
                    const int64_t *targets, const float *rowmax, float *loss, double *denom, void *stream);

/* "API": forward(logits, targets) -> (loss [N], rowmax [N], denom [N]) over the
 * whole vocabulary.  Workspace: det_ce_forward_workspace_size() bytes. */
size_t det_ce_forward_workspace_size(int64_t N);
int det_ce_forward(const void *logits, int32_t dtype, int64_t N, int64_t V, int64_t ld, const int64_t *targets,
                   float *loss, float *rowmax, double *denom, void *workspace, size_t ws_bytes, void *stream);

/* Loss reduction ("reduction is mean, sum, or none"): none copies loss to out[N];
 * sum = RN32(RN64(S)), mean = RN32(RN64(RN64(S)/N)), S = exact sum of the f32
 * losses; out[0].  Workspace: det_ce_reduce_workspace_size() bytes. */
size_t det_ce_reduce_workspace_size(int64_t N);
int det_ce_reduce(const float *loss, int64_t N, int32_t reduction, float *out, void *workspace, size_t ws_bytes,
                  void *stream);

/* Gradient "softmax(x_i) - onehot(t_i)" scaled by the upstream gradient:
 * grad_iv = RN32(RN64(RN64(RN64(w_iv / denom_i) - [v == t_i]) * c_i)),
 * c_i = grad_loss[i] (none), grad_loss[0] (sum), RN64(grad_loss[0]/N) (mean).
 * A vocabulary shard (det-cross-entropy page, "Correctness": the same bytes on
 * one device or many): logits and grad hold the V columns [v0, v0 + V) of the
 * vocabulary, targets are whole-vocabulary indices, and rowmax / denom are the
 * composed global values; v0 = 0 with the whole vocabulary is the unsharded
 * call.  v0 < 0 gives DET_E_VALUE.
 * grad_loss: (device) f32 [N] or [1]; grad: (device) f32, row i at grad + i*grad_ld. */
int det_ce_backward(const void *logits, int32_t dtype, int64_t N, int64_t V, int64_t ld, int64_t v0,
                    const int64_t *targets, const float *rowmax, const double *denom, const float *grad_loss,
                    int32_t reduction, float *grad, int64_t grad_ld, void *stream);

#ifdef __cplusplus
}
#endif
#endif
