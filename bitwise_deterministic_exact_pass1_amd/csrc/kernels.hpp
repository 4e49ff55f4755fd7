// kernels.hpp -- host-side launchers shared by the C ABI (capi.cpp) and the
// kernel translation units.  Argument checking happens in capi.cpp before any
// of these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <functional>

#include "dev_math.hpp"

namespace det {

struct Tensor {  // mirrors det_tensor
    const void *data;
    int dtype;  // 0 f32, 1 bf16
    int64_t B, H, S, D;
    int64_t sB, sH, sS;
};

struct OutView {
    float *data;
    int64_t sB, sH, sS;
};

// Geometry shared by the attention launchers.
struct AttnGeom {
    int64_t B, Hq, Hkv, Sq, Skv, D;
    int64_t Dp;  // widened Q row length: D rounded up to 16, 32, 64, 128 or 256
    int causal;
    double scale;
};

constexpr int kRowTile = 32;    // query rows per score tile
constexpr int kKeyTile = 256;   // keys per score tile (4 waves x 64 lanes)

// Query rows of a chunk, padded to whole row tiles (padding rows are zero).
// The workgroup's logical grid position (x, y, z), its linear ids dealt so
// that each of the chip's 8 XCDs runs one contiguous range of z-major, then
// y-major positions: workgroups are handed to the XCDs round-robin by linear
// id, so without this every XCD would touch every head, and each XCD's L2
// would fetch every head's data from HBM.  A bijection of the grid, so any
// other dispatch order only loses the locality.
struct GridPos {
    uint32_t x, y, z;
};
__device__ __forceinline__ GridPos xcd_grouped_pos() {
    constexpr uint32_t kXcds = 8;
    // (computed by every lane and read back from the first: vector registers
    // are free at this point, scalar ones are not)
    uint32_t X = gridDim.x, Y = gridDim.y, N = X * Y * gridDim.z;
    uint32_t L = (blockIdx.z * Y + blockIdx.y) * X + blockIdx.x;
    asm volatile("" : "+v"(X), "+v"(Y), "+v"(N), "+v"(L));
    const uint32_t xcd = L % kXcds, r = L / kXcds, q = N / kXcds, rem = N % kXcds;
    const uint32_t M = (xcd < rem ? xcd * (q + 1) : rem * (q + 1) + (xcd - rem) * q) + r;
    return GridPos{(uint32_t)__builtin_amdgcn_readfirstlane((int)(M % X)),
                   (uint32_t)__builtin_amdgcn_readfirstlane((int)((M / X) % Y)),
                   (uint32_t)__builtin_amdgcn_readfirstlane((int)(M / (X * Y)))};
}

inline int64_t padded_rows(int64_t ni) { return (ni + kRowTile - 1) / kRowTile * kRowTile; }
inline int64_t padded_dim(int64_t D) {
    int64_t p = 16;
    while (p < D) p *= 2;
    return p;
}

// ---- per-kernel timing (tracing aid): when enabled, every launch below is
// bracketed by two HIP events on its own stream.
struct ProfScope {
    ProfScope(const char *name, hipStream_t s);
    ~ProfScope();
    int slot;
    hipStream_t stream;
};
void prof_enable(bool on);
// "name count total_ms" lines for the launches since prof_enable(true).
size_t prof_report(char *buf, size_t len);

// ---- the fixed device scratch of det_attn_noalloc (noalloc.hip): its size,
// and its device address on the current device (looked up once per device).
constexpr size_t kNoAllocBytes = (size_t)64 << 20;
hipError_t noalloc_scratch(void **ptr, size_t *bytes);

// ---- workspace carving (all offsets 256-byte aligned)
size_t align256(size_t n);

// Per-chunk scratch of the score path: widened Q rows, rowmax keys, scores.
size_t score_scratch_bytes(const AttnGeom &g, int64_t rows_i, int64_t kv_len);

// Launchers (return hipError_t of the first failing launch).
hipError_t launch_widen_q(const Tensor &q, const AttnGeom &g, int64_t i0, int64_t i1, double *q64,
                          hipStream_t s);
hipError_t launch_fill_u32(uint32_t *p, int64_t n, uint32_t v, hipStream_t s);
hipError_t launch_fill_i64(int64_t *p, int64_t n, int64_t v, hipStream_t s);

// Scores of query rows [i0,i1) (all b,hq) against keys [kv_lo,kv_hi); writes
// scores[bh][i-i0][j-kv_lo] when `scores` is non-null and folds the visible
// scores into rowmax_keys[bh*key_rows + (i - key_row0)] by atomic max.
hipError_t launch_scores(const Tensor &k, const AttnGeom &g, const double *q64, int64_t i0, int64_t i1,
                         int64_t kv_lo, int64_t kv_hi, float *scores, uint32_t *rowmax_keys, int64_t key_rows,
                         int64_t key_row0, hipStream_t s);

// adds to *bad the number of rows [row0, row0 + rows) of the BHq heads
// ([BHq][out_rows] layout) whose computed max exceeds the supplied rowmax
hipError_t launch_rowmax_below(const float *supplied, const float *computed, int64_t BHq, int64_t rows,
                               int64_t out_rows, int64_t row0, unsigned int *bad, hipStream_t s);
hipError_t launch_keys_to_f32(const uint32_t *keys, float *out, int64_t B_Hq, int64_t rows, int64_t out_rows,
                              int64_t out_row0, hipStream_t s);

// ---- pass-1 scores of bf16 inputs on the matrix cores (qk.hip)
constexpr int kQKmax = 4;  // balanced base-256 digits per Q or K digit row (32-bit integers)
bool qk_uses_mfma(const Tensor &q);
size_t qk_kprep_bytes(const AttnGeom &g, int64_t kv_len);
size_t qk_chunk_bytes(const AttnGeom &g, int64_t ni, int64_t kv_len);
hipError_t launch_qk_kprep(const Tensor &k, const AttnGeom &g, int64_t kv_lo, int64_t kv_hi, void *ws,
                           hipStream_t s);
// ---- attention backward (bwd.hip)
constexpr int kBwdDigits = 18;   // radix-2^32 digits of a gradient sum (products of two f32 values)
constexpr int kBwdElo = -298;    // their lsb exponent
// delta and the dK / dV digit planes (whole problem) / per chunk of ni query
// rows: p and ds, the exponent statistics, the right operands' digit slices and
// the per-tile flags
size_t bwd_fixed_bytes(const AttnGeom &g);
size_t bwd_chunk_bytes(const AttnGeom &g, int64_t ni);
hipError_t launch_zero_view(const OutView &o, int64_t B, int64_t H, int64_t S, int64_t D, hipStream_t s);
// scores (nullable): writes the scores of query rows [i0, i1) against every
// key into the given [B*Hq][i1-i0][Skv] array (the matrix-core score path);
// without it the chains kernel runs the score chain itself.
typedef std::function<hipError_t(int64_t i0, int64_t i1, float *scores)> ScoreFn;
hipError_t launch_attn_backward(const Tensor &q, const Tensor &k, const Tensor &v, const Tensor &o,
                                const Tensor &dout, const float *rowmax, const double *den64, const AttnGeom &g,
                                void *fixed_ws, void *chunk_ws, int64_t chunk, const OutView &dq,
                                const OutView &dk, const OutView &dv, int force_fallback, const ScoreFn *scores,
                                hipStream_t s);

// Capacity of the remainder list of one V preparation (entries of all heads);
// heads whose remainders do not fit take the generic exact path.
constexpr int kRareCap = 4096;
// All arguments of the V preparation of one key range (device code in
// vprep.hpp): V's strides, the group geometry and the prepared arrays.
struct VJob {
    const void *v;
    int dtype;
    int64_t vsB, vsH, vsS, Hkv, D, Dp32, nG, kv_lo, kv_hi, nKB, nbhk;
    void *stats;
    int *colgrid, *grpB;
    void *vsl;
    // entries whose low bits fall below their column's digit grid: a count, a
    // flag per (head, 32-column group) and the list of (head, key, column, remainder)
    int *rare_n, *rare_grp;
    int4 *rare;
};
// Scores of rows [i0, i1) against keys [kv_lo, kv_hi) on the matrix cores.
// prep_q: Q's digit rows of the chunk are prepared (and the chunk's rowmax
// keys started at "empty"); otherwise the chunk workspace still holds them from
// an earlier call, and the keys keep their values (the max accumulates).
// prep_k: K's digit rows are prepared into kprep in the same launch as Q's;
// vj (bf16 V, nullable): V's column statistics are computed in that launch and
// its digit slices in the score-fix launch.  Both need a nonempty range.
hipError_t launch_scores_qk(const Tensor &q, const Tensor &k, const AttnGeom &g, void *kprep, bool prep_k,
                            bool prep_q, const VJob *vj, void *chunk_ws, int64_t i0, int64_t i1, int64_t kv_lo, int64_t kv_hi,
                            float *scores, uint32_t *rowmax_keys, int64_t key_rows, int64_t key_row0,
                            hipStream_t s);

// ---- pass 2 on the matrix cores (pv.hip)

// Where pass 2 takes the scores of a block from.
struct PvSrc {
    // stored pass-1 scores [bh][ni][W] of the chunk's rows and the key range
    // (f32 inputs), or null: the scores are recomputed
    const float *scores;
    int64_t W;
    // recomputed (bf16 inputs): the chunk's Q digit rows and the key range's K
    // digit rows as the score path laid them out ([row][kQKmax][Dp64] bytes and
    // one int4 {grid, digit count, log2 bound} per row; Q rows bh * ni_pad + i - i0,
    // K rows bhk * kv_pad + j - kv_lo)
    const int8_t *qdig, *kdig;
    const int4 *qinfo, *kinfo;
    int64_t ni_pad, kv_pad, Dp64;
    double scale;
    // the bf16 rows themselves, for the fp64 chain of the pairs outside the
    // matrix cores' exactness bound
    const void *q, *k;
    int64_t qsB, qsH, qsS, ksB, ksH, ksS;
    // or null: query rows that need more digits than the digit rows hold have
    // their scores by the fp64 chain from pass 1 of the same chunk and key
    // range: qslot[Q row] >= 0 is the row's slot, slots[slot * kv_pad + j - kv_lo]
    const int *qslot;
    const float *slots;
    int64_t slot_bytes;
};
// The pass-2 layout forced by the testing switch (0: by key-range length).
int pass2_layout();

// The recomputed-score source of a chunk of ni query rows against a key range
// of kv_len keys, from the workspace parts the score path prepared; slots:
// pass 1 ran on this chunk and key range just before, and its score slots of
// rows with many digits are used.
PvSrc qk_pv_src(const Tensor &q, const Tensor &k, const AttnGeom &g, void *kprep, void *chunk_ws, int64_t ni,
                int64_t kv_len, bool slots);

// Prepared V of one key range: per-column grid exponents and balanced int8
// digits in MFMA lane order.
struct VPrep {
    void *stats;  // column statistics per key chunk
    int *colgrid, *grpB;
    void *slices;
    int *rare_n, *rare_grp;  // remainders below the column grids (see VJob)
    int4 *rare;
    int64_t Dp32, nKB;
};
VJob make_vjob(const Tensor &v, const AttnGeom &g, int64_t kv_lo, int64_t kv_hi, VPrep &vp);
size_t vprep_bytes(const AttnGeom &g, int64_t kv_len);
// bytes of the V digit slices / of the column statistics within vprep_bytes
size_t vslice_bytes(const AttnGeom &g, int64_t kv_len);
size_t vstats_bytes(const AttnGeom &g);
// bytes of the remainder count, group flags and list within vprep_bytes
size_t vrare_bytes(const AttnGeom &g);
size_t pv_fallback_bytes(const AttnGeom &g, int64_t rows_i);
hipError_t launch_vprep(const Tensor &v, const AttnGeom &g, int64_t kv_lo, int64_t kv_hi, VPrep &vp,
                        hipStream_t s);
// V's digit slices alone (after its column statistics).
hipError_t launch_vslice(const VJob &J, hipStream_t s);
// The digit rows pass 2 recomputes scores from, without computing any: K's
// for [kv_lo, kv_hi) (prep_k), the chunk's Q rows [i0, i1) (prep_q) and, with
// vp, V's column statistics in the same launch, then V's digit slices.
hipError_t launch_qkv_prep(const Tensor &q, const Tensor &k, const Tensor &v, const AttnGeom &g, void *kprep,
                           bool prep_k, bool prep_q, VPrep *vp, void *chunk_ws, int64_t i0, int64_t i1, int64_t kv_lo,
                           int64_t kv_hi, hipStream_t s);
// With `o`, stat_m / stat_den (both or neither) also receive each row's max
// and RN64(DEN) at [bh * stat_rows + i].
// Exact NUM/DEN of query rows [i0,i1) against keys [kv_lo,kv_hi), with scores
// from `src` and rowmax[bh*rm_rows + i - rm_row0] (or, when rowmax is null, the
// order keys rowmax_keys at the same place).  With `o` the tile is finalized
// into o; otherwise its exact values are added into the digit planes num/den
// (rows bh*rows_per_bh + i - row0).  Tiles the matrix-core path cannot
// represent exactly are redone by the generic path (a second launch).
hipError_t launch_pv(const Tensor &v, const AttnGeom &g, const VPrep &vp, const PvSrc &src, const float *rowmax,
                     const uint32_t *rowmax_keys, int64_t rm_rows, int64_t rm_row0, int64_t i0, int64_t i1, int64_t kv_lo, int64_t kv_hi,
                     int *flags, int64_t *fb_num, int64_t *fb_den, const OutView *o, int64_t *num, int64_t *den,
                     int64_t plane_rows, int64_t rows_per_bh, int64_t row0, int force_fallback, hipStream_t s,
                     float *stat_m = nullptr, double *stat_den = nullptr, int64_t stat_rows = 0);

hipError_t launch_normalize(int64_t *digits, int64_t n_values, int n_digits, hipStream_t s);
// Rows [i0, i1) of each of n_bh runs of `rows` rows (values of `width`
// consecutive int64 each) in planes of `plane` values: normalize to canonical
// form, or fill with v.
hipError_t launch_normalize_rows(int64_t *digits, int n_digits, int64_t plane, int64_t n_bh, int64_t rows,
                                 int64_t i0, int64_t i1, int64_t width, hipStream_t s);
hipError_t launch_fill_rows_i64(int64_t *p, int n_planes, int64_t plane, int64_t n_bh, int64_t rows, int64_t i0,
                                int64_t i1, int64_t width, int64_t v, hipStream_t s);
hipError_t launch_digits_combine(int64_t *acc, const int64_t *part, int64_t n_values, int n_digits,
                                 hipStream_t s);
hipError_t launch_rowmax_combine(float *acc, const float *part, int64_t n, hipStream_t s);

// out[b][hq][i][d] for rows i0..i1 from planes num [14][plane_rows][D], den [9][plane_rows].
hipError_t launch_finalize(const int64_t *num, const int64_t *den, int64_t plane_rows, int64_t rows_per_bh,
                           int64_t row0, int64_t B_Hq, int64_t Hq, int64_t i0, int64_t i1, int64_t D,
                           const OutView &o, hipStream_t s);

// ---- cross-entropy
hipError_t launch_ce_rowmax(const void *x, int dtype, int64_t N, int64_t ld, int64_t v_lo, int64_t v_hi,
                            float *rowmax, hipStream_t s);
hipError_t launch_ce_denom(const void *x, int dtype, int64_t N, int64_t ld, const float *rowmax, int64_t v_lo,
                           int64_t v_hi, int64_t *den, int add_into, hipStream_t s);
hipError_t launch_ce_finalize(const int64_t *den, const void *x, int dtype, int64_t N, int64_t V, int64_t ld,
                              const int64_t *targets, const float *rowmax, float *loss, double *denom,
                              hipStream_t s);
// rows given a target outside [0, V) since the last call (their loss is NaN),
// then cleared; waits for the stream
hipError_t ce_take_bad_targets(hipStream_t s, unsigned int *count);
hipError_t launch_ce_forward(const void *x, int dtype, int64_t N, int64_t V, int64_t ld, const int64_t *targets,
                             float *loss, float *rowmax, double *denom, hipStream_t s);
hipError_t launch_ce_reduce(const float *loss, int64_t N, int reduction, float *out, int64_t *scratch,
                            hipStream_t s);
// v0: the vocabulary index of column 0 of x and grad (a vocabulary shard);
// targets are indices into the whole vocabulary.
hipError_t launch_ce_backward(const void *x, int dtype, int64_t N, int64_t V, int64_t ld, int64_t v0,
                              const int64_t *targets, const float *rowmax, const double *denom,
                              const float *grad_loss, int reduction, float *grad, int64_t grad_ld, hipStream_t s);

}  // namespace det
