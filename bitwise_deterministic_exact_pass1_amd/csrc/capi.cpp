// capi.cpp -- the extern "C" entry points declared in include/det_attn.h.
//
// Every entry point validates its arguments on the host before the first HIP
// call (so the checks run without a GPU), then enqueues a fixed sequence of
// kernels on the caller's stream.  Work is split into query-row chunks sized by
// the caller's workspace; rows are independent, so the chunking never changes
// a result bit.
#include "det_attn.h"
#include "kernels.hpp"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

using namespace det;

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int ok() {
    g_err.clear();
    return DET_OK;
}

int hip_fail(hipError_t e, const char *what) {
    return fail(DET_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define HIP_TRY(expr, what)                        \
    do {                                           \
        hipError_t _e = (expr);                    \
        if (_e != hipSuccess) return hip_fail(_e, what); \
    } while (0)

constexpr size_t kDefaultBudget = (size_t)8 << 30;  // default workspace per call

Tensor to_t(const det_tensor *t) { return Tensor{t->data, t->dtype, t->B, t->H, t->S, t->D, t->sB, t->sH, t->sS}; }

int check_tensor(const det_tensor *t, const char *name) {
    if (!t) return fail(DET_E_NULL, "%s descriptor is NULL", name);
    if (t->dtype != DET_F32 && t->dtype != DET_BF16) return fail(DET_E_DTYPE, "%s dtype %d is not f32/bf16", name, t->dtype);
    if (t->B < 1 || t->H < 1 || t->S < 0) return fail(DET_E_SHAPE, "%s has B=%lld H=%lld S=%lld", name,
                                                      (long long)t->B, (long long)t->H, (long long)t->S);
    if (t->D < 1 || t->D > 256) return fail(DET_E_SHAPE, "%s head dim D=%lld outside [1,256]", name, (long long)t->D);
    if (t->sB < 0 || t->sH < 0 || t->sS < 0) return fail(DET_E_STRIDE, "%s has a negative stride", name);
    if (!t->data && t->S > 0) return fail(DET_E_NULL, "%s data is NULL", name);
    return DET_OK;
}

int check_qk(const det_tensor *q, const det_tensor *k, int causal) {
    int rc;
    if ((rc = check_tensor(q, "q")) || (rc = check_tensor(k, "k"))) return rc;
    if (q->dtype != k->dtype) return fail(DET_E_DTYPE, "q and k dtypes differ");
    if (q->B != k->B) return fail(DET_E_SHAPE, "q and k batch sizes differ");
    if (q->D != k->D) return fail(DET_E_SHAPE, "q and k head dims differ");
    if (q->H % k->H) return fail(DET_E_SHAPE, "Hq=%lld is not a multiple of Hkv=%lld", (long long)q->H, (long long)k->H);
    if (causal && q->S != k->S) return fail(DET_E_SHAPE, "causal attention needs Sq == Skv");
    return DET_OK;
}

int check_qkv(const det_tensor *q, const det_tensor *k, const det_tensor *v, int causal) {
    int rc;
    if ((rc = check_qk(q, k, causal)) || (rc = check_tensor(v, "v"))) return rc;
    if (v->dtype != k->dtype) return fail(DET_E_DTYPE, "v and k dtypes differ");
    if (v->B != k->B || v->H != k->H || v->S != k->S || v->D != k->D)
        return fail(DET_E_SHAPE, "v shape differs from k");
    return DET_OK;
}

int check_range(const det_tensor *k, int64_t lo, int64_t hi) {
    if (lo < 0 || hi < lo || hi > k->S)
        return fail(DET_E_SHAPE, "key range [%lld,%lld) outside [0,%lld]", (long long)lo, (long long)hi, (long long)k->S);
    return DET_OK;
}

int check_qrange(const det_tensor *q, int64_t lo, int64_t hi) {
    if (lo < 0 || hi < lo || hi > q->S)
        return fail(DET_E_SHAPE, "query range [%lld,%lld) outside [0,%lld]", (long long)lo, (long long)hi,
                    (long long)q->S);
    return DET_OK;
}

int check_out(const det_out *o) {
    if (!o) return fail(DET_E_NULL, "output descriptor is NULL");
    if (!o->data) return fail(DET_E_NULL, "output data is NULL");
    if (o->sB < 0 || o->sH < 0 || o->sS < 0) return fail(DET_E_STRIDE, "output has a negative stride");
    return DET_OK;
}

AttnGeom geom(const det_tensor *q, const det_tensor *k, int causal, double scale) {
    AttnGeom g;
    g.B = q->B;
    g.Hq = q->H;
    g.Hkv = k->H;
    g.Sq = q->S;
    g.Skv = k->S;
    g.D = q->D;
    g.Dp = padded_dim(q->D);
    g.causal = causal;
    g.scale = scale;
    return g;
}

// Bump allocator over the caller's workspace.
// Bump allocator over the caller's workspace.  Every region is checked
// against the workspace size on the host: a layout that outgrows the size the
// byte functions computed is reported (over) before any kernel could touch it.
struct Carver {
    char *p;
    size_t cap;
    size_t used = 0;
    bool over = false;
    template <typename T> T *take(size_t count) {
        T *r = (T *)(p + used);
        used += align256(count * sizeof(T));
        if (used > cap) over = true;
        return r;
    }
};

// ---- per-chunk workspace needs of each entry point (ni = query rows per chunk)

// ---- scores: bf16 on the matrix cores (qk.hip), f32 by the fp64 VALU chain (attn.hip)

size_t score_fixed_bytes(const AttnGeom &g, bool mfma, int64_t kv_len) {
    return mfma ? qk_kprep_bytes(g, kv_len) : 0;
}

size_t score_chunk_bytes(const AttnGeom &g, bool mfma, int64_t ni, int64_t kv_len) {
    return mfma ? qk_chunk_bytes(g, ni, kv_len) : align256((size_t)g.B * g.Hq * padded_rows(ni) * g.Dp * 8);
}

// Scores of rows [i0, i1) against keys [lo, hi), with the rowmax keys when
// `keys` is set.  prep_q: Q's part of the chunk is prepared and the rowmax
// keys of rows [i0, i1) start at "empty"; without it both are kept from an
// earlier call on the same chunk (the keys then accumulate the max over the
// calls).  prep_k: K's digits for the range are prepared first (the
// matrix-core path prepares them in the same launch as Q's); vp: V is prepared
// too (on the matrix-core path beside the score preparation and the score fix,
// otherwise by its own launches).
hipError_t run_scores(const Tensor &tq, const Tensor &tk, const Tensor &tv, const AttnGeom &g, bool mfma, void *kprep,
                      bool prep_k, bool prep_q, VPrep *vp, void *chunk_ws, int64_t i0, int64_t i1, int64_t lo,
                      int64_t hi, float *scores, uint32_t *keys, int64_t key_rows, int64_t key_row0, hipStream_t s) {
    hipError_t e;
    const bool host = mfma && hi > lo && i1 > i0;  // the score launches can carry the preparations
    if (vp && !host && (e = launch_vprep(tv, g, lo, hi, *vp, s)) != hipSuccess) return e;
    if (mfma) {
        if (!host) return hipSuccess;
        VJob vj{};
        if (vp) vj = make_vjob(tv, g, lo, hi, *vp);
        return launch_scores_qk(tq, tk, g, kprep, prep_k, prep_q, vp ? &vj : nullptr, chunk_ws, i0, i1, lo, hi, scores, keys,
                                key_rows, key_row0, s);
    }
    if (keys && prep_q) {  // keys[h * key_rows + i - key_row0]: one run per head, or one in all when contiguous
        const int64_t bh = g.B * g.Hq, n = i1 - i0;
        const bool whole = key_rows == n && key_row0 == i0;
        for (int64_t h = 0; h < (whole ? 1 : bh); ++h)
            if ((e = launch_fill_u32(keys + h * key_rows + (i0 - key_row0), whole ? bh * n : n, kKeyNegInf, s)) !=
                hipSuccess)
                return e;
    }
    if (prep_q && (e = launch_widen_q(tq, g, i0, i1, (double *)chunk_ws, s)) != hipSuccess) return e;
    return launch_scores(tk, g, (const double *)chunk_ws, i0, i1, lo, hi, scores, keys, key_rows, key_row0, s);
}

bool use_mfma_scores(const det_tensor *q) { return q->dtype == DET_BF16; }

size_t bytes_rowmax(const AttnGeom &g, bool mfma, int64_t ni, int64_t kv_len) {
    const int64_t bh = g.B * g.Hq;
    return score_fixed_bytes(g, mfma, kv_len) + score_chunk_bytes(g, mfma, ni, kv_len) + align256((size_t)bh * ni * 4);
}

// Set by det_debug_score_source (a testing aid): 0 chooses by workspace size,
// 1 keeps bf16 scores between the passes, 2 recomputes them in pass 2.
std::atomic<int> g_score_source{0};

// Scores kept between the passes (an f32 per row and key of the chunk), unless
// pass 2 recomputes them (rc: bf16 only, from the digit rows pass 1 prepared).
size_t stored_score_bytes(bool rc, int64_t rows, int64_t W) { return rc ? 0 : align256((size_t)rows * W * 4); }

size_t bytes_accumulate(const AttnGeom &g, bool mfma, bool rc, int64_t ni, int64_t W) {
    const int64_t bh = g.B * g.Hq;
    return vprep_bytes(g, W) + score_fixed_bytes(g, mfma, W) + score_chunk_bytes(g, mfma, ni, W) +
           stored_score_bytes(rc, bh * ni, W) + align256((size_t)bh * ((ni + 31) / 32) * 4);
}

size_t bytes_fused(const AttnGeom &g, bool mfma, bool rc, int64_t ni) {
    const int64_t bh = g.B * g.Hq, rows = bh * ni;
    return vprep_bytes(g, g.Skv) + score_fixed_bytes(g, mfma, g.Skv) + score_chunk_bytes(g, mfma, ni, g.Skv) +
           align256((size_t)rows * 4) + stored_score_bytes(rc, rows, g.Skv) + pv_fallback_bytes(g, ni);
}

size_t bytes_sharded(const AttnGeom &g, bool mfma, bool rc, int64_t ni, int64_t maxlen) {
    const int64_t bh = g.B * g.Hq, rows = bh * ni;
    return vprep_bytes(g, maxlen) + score_fixed_bytes(g, mfma, maxlen) + score_chunk_bytes(g, mfma, ni, maxlen) +
           align256((size_t)rows * 4) + stored_score_bytes(rc, rows, maxlen) + align256((size_t)rows * 4) +
           align256((size_t)bh * ((ni + 31) / 32) * 4) +
           align256((size_t)kNumDigits * rows * g.D * 8) + align256((size_t)kDenDigits * rows * 8);
}

// Whether pass 2 recomputes the bf16 scores instead of reading the ones pass 1
// kept.  Keeping them costs a round trip through HBM of 4 bytes per (row, key)
// and an O(rows x keys) workspace per row chunk; recomputing costs the score
// products and their exact composition a second time.  Measured on MI355X:
// keeping is faster up to a few thousand keys per row (1024 keys: 0.11 against
// 0.16 ms per call; 8192: 9.5 against 9.7 ms), recomputing beyond (37810
// keys, head dim 128: 0.71 against 0.75 s).  So the scores are recomputed for
// key ranges of kRecomputeKeys or more at head dims up to 128, or when one row
// tile's share of the kept buffer does not fit the workspace (a small fixed
// scratch; `need_kept_tile`: the layout's size for one tile with kept
// scores), and kept otherwise; f32 scores are always kept.
constexpr int64_t kRecomputeKeys = 16384;
template <typename F>
bool recompute_scores(bool mfma, const AttnGeom &g, int64_t kv_len, size_t ws_bytes, F need_kept_tile) {
    if (!mfma) return false;
    const int m = g_score_source.load(std::memory_order_relaxed);
    if (m == 1 || m == 2) return m == 2;
    return (kv_len >= kRecomputeKeys && g.D <= 128) || need_kept_tile() > ws_bytes;
}

// Pass 2's score source for rows [i0, i1) against [lo, hi): stored scores, or
// the digit rows in kprep / the chunk workspace (with pass 1's score slots when
// pass 1 ran on the same rows and range just before: `slots`).
PvSrc pv_src(const Tensor &tq, const Tensor &tk, const AttnGeom &g, bool rc, void *kprep, void *cws, float *sc,
             int64_t i0, int64_t i1, int64_t lo, int64_t hi, bool slots = false) {
    if (rc) return qk_pv_src(tq, tk, g, kprep, cws, i1 - i0, hi - lo, slots);
    PvSrc p{};
    p.scores = sc;
    p.W = hi - lo;
    return p;
}

VPrep carve_vprep(Carver &c, const AttnGeom &g, int64_t kv_len) {
    const int64_t bhk = g.B * g.Hkv, Dp32 = (g.D + 31) / 32 * 32, nG = Dp32 / 32;
    const int64_t nKB = std::max<int64_t>((kv_len + 31) / 32, 1);
    VPrep v;
    v.stats = c.take<char>(vstats_bytes(g));
    v.colgrid = c.take<int>(bhk * Dp32);
    v.grpB = c.take<int>(bhk * nG);
    v.slices = c.take<char>(vslice_bytes(g, kv_len));
    v.rare_n = c.take<int>(1);
    v.rare_grp = c.take<int>(bhk * nG);
    v.rare = c.take<int4>(kRareCap);
    v.Dp32 = Dp32;
    v.nKB = nKB;
    return v;
}

// Set by det_debug_force_generic (a testing aid): every tile then takes the
// generic exact path, so tests can check that both paths give the same bits.
std::atomic<int> g_force_generic{0};
int force_fallback() { return g_force_generic.load(std::memory_order_relaxed); }
// Set by det_debug_checks: entry points that take caller-supplied row maxima
// or targets verify them on the device and report violations (synchronizing).
std::atomic<int> g_checks{0};
bool checks_on() { return g_checks.load(std::memory_order_relaxed) != 0; }

// The cross-entropy target check around a launch: the count is cleared before
// and read after (both wait for the stream).
int ce_check_begin(hipStream_t s) {
    unsigned int c = 0;
    HIP_TRY(ce_take_bad_targets(s, &c), "input checks");
    return ok();
}
int ce_check_end(hipStream_t s) {
    unsigned int c = 0;
    HIP_TRY(ce_take_bad_targets(s, &c), "input checks");
    if (c) return fail(DET_E_VALUE, "%u rows have a target outside [0, V) (their loss is NaN)", c);
    return ok();
}

// Set by det_debug_pass2_layout (a testing aid): which pass-2 kernel takes
// recomputed scores (0: by key-range length).
std::atomic<int> g_pass2_layout{0};

// Largest chunk (a multiple of kRowTile, or all Sq rows) whose need fits `budget`;
// 0 if even one tile does not fit.
template <typename F> int64_t choose_chunk(int64_t Sq, size_t budget, F need) {
    if (Sq <= 0) return 0;
    if (need(Sq) <= budget) return Sq;
    int64_t lo = 0, hi = (Sq - 1) / kRowTile;  // in tiles
    // (Sq: the number of query rows to process)
    while (lo < hi) {
        const int64_t mid = (lo + hi + 1) / 2;
        if (need(mid * kRowTile) <= budget) lo = mid;
        else hi = mid - 1;
    }
    return lo * kRowTile;
}

template <typename F> size_t default_size(int64_t Sq, F need) {
    if (Sq <= 0) return 256;
    const int64_t ni = std::max<int64_t>(std::min<int64_t>(Sq, kRowTile), choose_chunk(Sq, kDefaultBudget, need));
    return need(ni);
}

int check_ws(void *ws, size_t have, size_t need_min) {
    if (need_min == 0) return DET_OK;
    if (!ws) return fail(DET_E_WORKSPACE, "workspace is NULL (need %zu bytes)", need_min);
    if (((uintptr_t)ws) & 255) return fail(DET_E_WORKSPACE, "workspace is not 256-byte aligned");
    if (have < need_min) return fail(DET_E_WORKSPACE, "workspace has %zu bytes, need at least %zu", have, need_min);
    return DET_OK;
}

}  // namespace

extern "C" {

const char *det_last_error(void) { return g_err.c_str(); }

int det_debug_force_generic(int32_t on) {
    g_force_generic.store(on ? 1 : 0, std::memory_order_relaxed);
    return ok();
}

int det_debug_checks(int32_t on) {
    g_checks.store(on ? 1 : 0, std::memory_order_relaxed);
    return ok();
}

int det_debug_score_source(int32_t mode) {
    if (mode < 0 || mode > 2) return fail(DET_E_VALUE, "score source %d is not 0, 1 or 2", (int)mode);
    g_score_source.store(mode, std::memory_order_relaxed);
    return ok();
}

int det_debug_pass2_layout(int32_t mode) {
    if (mode < 0 || mode > 2) return fail(DET_E_VALUE, "pass-2 layout %d is not 0, 1 or 2", (int)mode);
    g_pass2_layout.store(mode, std::memory_order_relaxed);
    return ok();
}

int det_profile_begin(void) {
    prof_enable(true);
    return ok();
}

size_t det_profile_end(char *buf, size_t len) {
    const size_t n = prof_report(buf, len);
    prof_enable(false);
    return n;
}

int det_digit_format(int32_t which, int32_t *n_digits, int32_t *lsb_exp2) {
    if (!n_digits || !lsb_exp2) return fail(DET_E_NULL, "output pointer is NULL");
    if (which == 0) {
        *n_digits = kNumDigits;
        *lsb_exp2 = kNumElo;
    } else if (which == 1) {
        *n_digits = kDenDigits;
        *lsb_exp2 = kDenElo;
    } else {
        return fail(DET_E_VALUE, "digit format %d is neither 0 (NUM) nor 1 (DEN)", which);
    }
    return ok();
}

// ------------------------------------------------------------------ rowmax

size_t det_attn_rowmax_workspace_size(const det_tensor *q, const det_tensor *k, int64_t q_lo, int64_t q_hi,
                                      int64_t kv_lo, int64_t kv_hi) {
    if (check_qk(q, k, 0) || check_qrange(q, q_lo, q_hi) || check_range(k, kv_lo, kv_hi)) return 0;
    const AttnGeom g = geom(q, k, 0, 1.0);
    const bool mf = use_mfma_scores(q);
    return default_size(q_hi - q_lo, [&](int64_t ni) { return bytes_rowmax(g, mf, ni, kv_hi - kv_lo); });
}

int det_attn_rowmax(const det_tensor *q, const det_tensor *k, int64_t q_lo, int64_t q_hi, int64_t kv_lo,
                    int64_t kv_hi, int32_t causal, double scale, float *rowmax, void *workspace, size_t ws_bytes,
                    void *stream) {
    int rc;
    if ((rc = check_qk(q, k, causal)) || (rc = check_qrange(q, q_lo, q_hi)) || (rc = check_range(k, kv_lo, kv_hi)))
        return rc;
    const int64_t nq = q_hi - q_lo;
    if (!rowmax && nq > 0) return fail(DET_E_NULL, "rowmax is NULL");
    const AttnGeom g = geom(q, k, causal, scale);
    const bool mf = use_mfma_scores(q);
    const int64_t W = kv_hi - kv_lo;
    auto need = [&](int64_t ni) { return bytes_rowmax(g, mf, ni, W); };
    if ((rc = check_ws(workspace, ws_bytes, nq > 0 ? need(std::min<int64_t>(nq, kRowTile)) : 0))) return rc;
    if (nq == 0) return ok();
    hipStream_t s = (hipStream_t)stream;
    const Tensor tq = to_t(q), tk = to_t(k);
    const int64_t chunk = choose_chunk(nq, ws_bytes, need), bh = g.B * g.Hq;
    Carver c0{(char *)workspace, ws_bytes};
    void *kprep = c0.take<char>(score_fixed_bytes(g, mf, W));
    // per-chunk regions, sized for the largest chunk and reused by every chunk
    void *cws = c0.take<char>(score_chunk_bytes(g, mf, chunk, W));
    uint32_t *keys = c0.take<uint32_t>(bh * chunk);
    if (c0.over) return fail(DET_E_WORKSPACE, "internal: workspace layout exceeds its computed size");
    for (int64_t i0 = q_lo; i0 < q_hi; i0 += chunk) {
        const int64_t i1 = std::min(q_hi, i0 + chunk), ni = i1 - i0;
        HIP_TRY(run_scores(tq, tk, tk, g, mf, kprep, i0 == q_lo, true, nullptr, cws, i0, i1, kv_lo, kv_hi, nullptr,
                           keys, ni, i0, s),
                "scores");
        HIP_TRY(launch_keys_to_f32(keys, rowmax, bh, ni, g.Sq, i0, s), "rowmax");
    }
    return ok();
}

// ------------------------------------------------------------------ accumulate

// The accumulate precondition under det_debug_checks: the range's own row
// maxima (det_attn_rowmax into scratch this check allocates) against the
// supplied ones; DET_E_VALUE when a visible score lies above its row's value.
static int check_rowmax_bound(const det_tensor *q, const det_tensor *k, const float *rowmax, int64_t q_lo, int64_t q_hi,
                       int64_t kv_lo, int64_t kv_hi, int32_t causal, double scale, hipStream_t s) {
    const AttnGeom g = geom(q, k, causal, scale);
    const int64_t bh = g.B * g.Hq;
    const size_t ws = det_attn_rowmax_workspace_size(q, k, q_lo, q_hi, kv_lo, kv_hi);
    const size_t mbytes = (size_t)(bh * g.Sq) * sizeof(float);
    char *buf = nullptr;
    HIP_TRY(hipMalloc((void **)&buf, align256(mbytes) + align256(sizeof(unsigned int)) + ws), "input checks");
    float *mx = (float *)buf;
    unsigned int *bad = (unsigned int *)(buf + align256(mbytes));
    void *wsp = buf + align256(mbytes) + align256(sizeof(unsigned int));
    unsigned int nbad = 0;
    hipError_t e = hipMemsetAsync(bad, 0, sizeof(unsigned int), s);
    int rc = e == hipSuccess ? det_attn_rowmax(q, k, q_lo, q_hi, kv_lo, kv_hi, causal, scale, mx, wsp, ws, s) : 0;
    if (e == hipSuccess && rc == 0) e = launch_rowmax_below(rowmax, mx, bh, q_hi - q_lo, g.Sq, q_lo, bad, s);
    if (e == hipSuccess && rc == 0) e = hipMemcpyAsync(&nbad, bad, sizeof(nbad), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess && rc == 0) e = hipStreamSynchronize(s);
    const hipError_t ef = hipFree(buf);
    if (rc) return rc;
    if (e != hipSuccess) return hip_fail(e, "input checks");
    if (ef != hipSuccess) return hip_fail(ef, "input checks");
    if (nbad) return fail(DET_E_VALUE, "%u rows have a visible score above the supplied rowmax", nbad);
    return ok();
}

size_t det_attn_accumulate_workspace_size(const det_tensor *q, const det_tensor *k, const det_tensor *v,
                                          int64_t q_lo, int64_t q_hi, int64_t kv_lo, int64_t kv_hi) {
    if (check_qkv(q, k, v, 0) || check_qrange(q, q_lo, q_hi) || check_range(k, kv_lo, kv_hi)) return 0;
    const AttnGeom g = geom(q, k, 0, 1.0);
    const bool mf = use_mfma_scores(q);
    const int64_t nq = q_hi - q_lo, W = kv_hi - kv_lo;
    const bool recomp = recompute_scores(mf, g, W, kDefaultBudget, [&] {
        return bytes_accumulate(g, mf, false, std::max<int64_t>(std::min<int64_t>(nq, kRowTile), 1), W);
    });
    return default_size(nq, [&](int64_t ni) { return bytes_accumulate(g, mf, recomp, ni, W); });
}

int det_attn_accumulate(const det_tensor *q, const det_tensor *k, const det_tensor *v, const float *rowmax,
                        int64_t q_lo, int64_t q_hi, int64_t kv_lo, int64_t kv_hi, int32_t causal, double scale,
                        int64_t *num, int64_t *den, int32_t add_into, void *workspace, size_t ws_bytes,
                        void *stream) {
    int rc;
    if ((rc = check_qkv(q, k, v, causal)) || (rc = check_qrange(q, q_lo, q_hi)) || (rc = check_range(k, kv_lo, kv_hi)))
        return rc;
    const int64_t nq = q_hi - q_lo;
    if (nq > 0 && (!rowmax || !num || !den)) return fail(DET_E_NULL, "rowmax, num or den is NULL");
    const AttnGeom g = geom(q, k, causal, scale);
    const bool mf = use_mfma_scores(q);
    const int64_t W = kv_hi - kv_lo;
    const bool recomp = recompute_scores(mf, g, W, ws_bytes, [&] {
        return bytes_accumulate(g, mf, false, std::max<int64_t>(std::min<int64_t>(nq, kRowTile), 1), W);
    });
    auto need = [&](int64_t ni) { return bytes_accumulate(g, mf, recomp, ni, W); };
    if ((rc = check_ws(workspace, ws_bytes, nq > 0 ? need(std::min<int64_t>(nq, kRowTile)) : 0))) return rc;
    if (nq == 0) return ok();
    hipStream_t s = (hipStream_t)stream;
    if (checks_on() && W > 0 && (rc = check_rowmax_bound(q, k, rowmax, q_lo, q_hi, kv_lo, kv_hi, causal, scale, s)))
        return rc;
    const Tensor tq = to_t(q), tk = to_t(k), tv = to_t(v);
    const int64_t bh = g.B * g.Hq, rows = bh * g.Sq;
    const int64_t chunk = choose_chunk(nq, ws_bytes, need);
    Carver c0{(char *)workspace, ws_bytes};
    VPrep vp = carve_vprep(c0, g, W);
    void *kprep = c0.take<char>(score_fixed_bytes(g, mf, W));
    // per-chunk regions, sized for the largest chunk and reused by every chunk
    void *cws = c0.take<char>(score_chunk_bytes(g, mf, chunk, W));
    float *sc = recomp ? nullptr : c0.take<float>(bh * chunk * W);
    int *flags = c0.take<int>(bh * ((chunk + 31) / 32));
    if (c0.over) return fail(DET_E_WORKSPACE, "internal: workspace layout exceeds its computed size");
    // only rows [q_lo, q_hi) of each head are touched
    if (!add_into) {
        HIP_TRY(launch_fill_rows_i64(num, kNumDigits, rows * g.D, bh, g.Sq, q_lo, q_hi, g.D, 0, s), "fill num");
        HIP_TRY(launch_fill_rows_i64(den, kDenDigits, rows, bh, g.Sq, q_lo, q_hi, 1, 0, s), "fill den");
    }
    const int ff = force_fallback();
    for (int64_t i0 = q_lo; i0 < q_hi && W > 0; i0 += chunk) {
        const int64_t i1 = std::min(q_hi, i0 + chunk);
        // the first chunk's launches also prepare K and V
        const bool first = i0 == q_lo;
        if (recomp)  // the digit rows pass 2 recomputes the scores from (and V's, on the first chunk)
            HIP_TRY(launch_qkv_prep(tq, tk, tv, g, kprep, first, true, first ? &vp : nullptr, cws, i0, i1, kv_lo, kv_hi,
                                    s),
                    "prepare");
        else
            HIP_TRY(run_scores(tq, tk, tv, g, mf, kprep, first, true, first ? &vp : nullptr, cws, i0, i1, kv_lo,
                               kv_hi, sc, nullptr, 0, 0, s),
                    "scores");
        HIP_TRY(launch_pv(tv, g, vp, pv_src(tq, tk, g, recomp, kprep, cws, sc, i0, i1, kv_lo, kv_hi), rowmax, nullptr, g.Sq,
                          0, i0, i1, kv_lo, kv_hi, flags, nullptr, nullptr, nullptr, num, den, rows, g.Sq, 0, ff, s),
                "deposit");
    }
    HIP_TRY(launch_normalize_rows(num, kNumDigits, rows * g.D, bh, g.Sq, q_lo, q_hi, g.D, s), "normalize num");
    HIP_TRY(launch_normalize_rows(den, kDenDigits, rows, bh, g.Sq, q_lo, q_hi, 1, s), "normalize den");
    return ok();
}

// ------------------------------------------------------------------ composition

int det_rowmax_combine(float *acc, const float *part, int64_t n, void *stream) {
    if (n < 0) return fail(DET_E_SHAPE, "negative count");
    if (n > 0 && (!acc || !part)) return fail(DET_E_NULL, "acc or part is NULL");
    HIP_TRY(launch_rowmax_combine(acc, part, n, (hipStream_t)stream), "rowmax combine");
    return ok();
}

int det_digits_normalize(int64_t *acc, int64_t n_values, int32_t n_digits, void *stream) {
    if (n_values < 0) return fail(DET_E_SHAPE, "negative count");
    if (n_digits != kNumDigits && n_digits != kDenDigits)
        return fail(DET_E_VALUE, "n_digits must be %d or %d", kNumDigits, kDenDigits);
    if (n_values > 0 && !acc) return fail(DET_E_NULL, "acc is NULL");
    HIP_TRY(launch_normalize(acc, n_values, n_digits, (hipStream_t)stream), "digits normalize");
    return ok();
}

int det_digits_combine(int64_t *acc, const int64_t *part, int64_t n_values, int32_t n_digits, void *stream) {
    if (n_values < 0) return fail(DET_E_SHAPE, "negative count");
    if (n_digits != kNumDigits && n_digits != kDenDigits)
        return fail(DET_E_VALUE, "n_digits must be %d or %d", kNumDigits, kDenDigits);
    if (n_values > 0 && (!acc || !part)) return fail(DET_E_NULL, "acc or part is NULL");
    HIP_TRY(launch_digits_combine(acc, part, n_values, n_digits, (hipStream_t)stream), "digits combine");
    return ok();
}

// ------------------------------------------------------------------ finalize

int det_attn_finalize(const int64_t *num, const int64_t *den, int64_t B, int64_t Hq, int64_t Sq, int64_t D,
                      const det_out *o, void *stream) {
    if (B < 1 || Hq < 1 || Sq < 0 || D < 1 || D > 256) return fail(DET_E_SHAPE, "bad finalize shape");
    int rc;
    if (Sq == 0) return ok();
    if ((rc = check_out(o))) return rc;
    if (!num || !den) return fail(DET_E_NULL, "num or den is NULL");
    const int64_t rows = B * Hq * Sq;
    HIP_TRY(launch_finalize(num, den, rows, Sq, 0, B * Hq, Hq, 0, Sq, D, OutView{o->data, o->sB, o->sH, o->sS},
                            (hipStream_t)stream),
            "finalize");
    return ok();
}

// ------------------------------------------------------------------ fused

size_t det_attn_workspace_size(const det_tensor *q, const det_tensor *k, const det_tensor *v, int32_t causal) {
    if (check_qkv(q, k, v, causal)) return 0;
    const AttnGeom g = geom(q, k, causal, 1.0);
    const bool mf = use_mfma_scores(q);
    const bool recomp = recompute_scores(mf, g, g.Skv, kDefaultBudget, [&] {
        return bytes_fused(g, mf, false, std::max<int64_t>(std::min<int64_t>(g.Sq, kRowTile), 1));
    });
    return default_size(g.Sq, [&](int64_t ni) { return bytes_fused(g, mf, recomp, ni); });
}

static int fused_attn(const det_tensor *q, const det_tensor *k, const det_tensor *v, int32_t causal, double scale,
                      const det_out *o, float *stat_m, double *stat_den, void *workspace, size_t ws_bytes,
                      void *stream) {
    int rc;
    if ((rc = check_qkv(q, k, v, causal))) return rc;
    if (q->S > 0 && (rc = check_out(o))) return rc;
    const AttnGeom g = geom(q, k, causal, scale);
    const bool mf = use_mfma_scores(q);
    const bool recomp = recompute_scores(mf, g, g.Skv, ws_bytes, [&] {
        return bytes_fused(g, mf, false, std::max<int64_t>(std::min<int64_t>(g.Sq, kRowTile), 1));
    });
    auto need = [&](int64_t ni) { return bytes_fused(g, mf, recomp, ni); };
    if ((rc = check_ws(workspace, ws_bytes, g.Sq > 0 ? need(std::min<int64_t>(g.Sq, kRowTile)) : 0))) return rc;
    if (g.Sq == 0) return ok();
    hipStream_t s = (hipStream_t)stream;
    const Tensor tq = to_t(q), tk = to_t(k), tv = to_t(v);
    const OutView ov{o->data, o->sB, o->sH, o->sS};
    const int64_t chunk = choose_chunk(g.Sq, ws_bytes, need), bh = g.B * g.Hq;
    Carver c0{(char *)workspace, ws_bytes};
    VPrep vp = carve_vprep(c0, g, g.Skv);
    void *kprep = c0.take<char>(score_fixed_bytes(g, mf, g.Skv));
    // per-chunk regions, sized for the largest chunk and reused by every chunk
    const int64_t crows = bh * chunk, ctiles = (chunk + 31) / 32;
    void *cws = c0.take<char>(score_chunk_bytes(g, mf, chunk, g.Skv));
    uint32_t *keys = c0.take<uint32_t>(crows);
    float *sc = recomp ? nullptr : c0.take<float>(crows * g.Skv);
    int *flags = c0.take<int>(bh * ctiles);
    int64_t *fnum = c0.take<int64_t>(kNumDigits * bh * ctiles * 32 * g.D);
    int64_t *fden = c0.take<int64_t>(kDenDigits * bh * ctiles * 32);
    if (c0.over) return fail(DET_E_WORKSPACE, "internal: workspace layout exceeds its computed size");
    const int ff = force_fallback();
    for (int64_t i0 = 0; i0 < g.Sq; i0 += chunk) {
        const int64_t i1 = std::min(g.Sq, i0 + chunk), ni = i1 - i0;
        // the first chunk's launches also prepare K and V
        // pass 1: the row maxima, and the scores when they are kept for pass 2
        HIP_TRY(run_scores(tq, tk, tv, g, mf, kprep, i0 == 0, true, i0 == 0 ? &vp : nullptr, cws, i0, i1, 0, g.Skv, sc,
                           keys, ni, i0, s),
                "scores");
        HIP_TRY(launch_pv(tv, g, vp, pv_src(tq, tk, g, recomp, kprep, cws, sc, i0, i1, 0, g.Skv, true), nullptr, keys, ni, i0, i0,
                          i1, 0, g.Skv, flags, fnum, fden, &ov, nullptr, nullptr, 0, 0, 0, ff, s, stat_m, stat_den,
                          g.Sq),
                "deposit");
    }
    return ok();
}

int det_attn(const det_tensor *q, const det_tensor *k, const det_tensor *v, int32_t causal, double scale,
             const det_out *o, void *workspace, size_t ws_bytes, void *stream) {
    return fused_attn(q, k, v, causal, scale, o, nullptr, nullptr, workspace, ws_bytes, stream);
}

int det_attn_noalloc(const det_tensor *q, const det_tensor *k, const det_tensor *v, int32_t causal, double scale,
                     const det_out *o, void *stream) {
    int rc;
    if ((rc = check_qkv(q, k, v, causal))) return rc;
    if (q->S > 0 && (rc = check_out(o))) return rc;
    const AttnGeom g = geom(q, k, causal, scale);
    const bool mf = use_mfma_scores(q);
    const int64_t tile_rows = std::max<int64_t>(std::min<int64_t>(g.Sq, kRowTile), 1);
    const bool recomp =
        recompute_scores(mf, g, g.Skv, kNoAllocBytes, [&] { return bytes_fused(g, mf, false, tile_rows); });
    const size_t need_min = g.Sq > 0 ? bytes_fused(g, mf, recomp, tile_rows) : 0;
    if (need_min > kNoAllocBytes)
        return fail(DET_E_WORKSPACE,
                    "det_attn_noalloc: one %d-row chunk of this problem needs %zu bytes of scratch; the fixed "
                    "scratch holds %zu (use det_attn with a workspace)",
                    kRowTile, need_min, kNoAllocBytes);
    if (g.Sq == 0) return ok();
    void *scratch = nullptr;
    size_t cap = 0;
    HIP_TRY(noalloc_scratch(&scratch, &cap), "noalloc scratch address");
    return fused_attn(q, k, v, causal, scale, o, nullptr, nullptr, scratch, cap, stream);
}

int det_attn_stats(const det_tensor *q, const det_tensor *k, const det_tensor *v, int32_t causal, double scale,
                   const det_out *o, float *rowmax, double *den64, void *workspace, size_t ws_bytes, void *stream) {
    if (q && q->S > 0 && (!rowmax || !den64)) return fail(DET_E_NULL, "rowmax or den64 is NULL");
    if (k && k->S == 0 && q && q->S > 0) return fail(DET_E_SHAPE, "det_attn_stats needs a nonempty key range");
    return fused_attn(q, k, v, causal, scale, o, rowmax, den64, workspace, ws_bytes, stream);
}

static int check_grad_operand(const det_tensor *t, const det_tensor *q, const char *name) {
    int rc;
    if ((rc = check_tensor(t, name))) return rc;
    if (t->dtype != DET_F32) return fail(DET_E_DTYPE, "%s must be DET_F32", name);
    if (t->B != q->B || t->H != q->H || t->S != q->S || t->D != q->D)
        return fail(DET_E_SHAPE, "%s shape differs from q", name);
    return DET_OK;
}

// With bf16 inputs the backward's scores come from the matrix-core score path,
// which needs its K preparation, its chunk part and rowmax keys (unused here).
static size_t bytes_backward(const AttnGeom &g, bool mf, int64_t ni) {
    const size_t sc = mf ? score_fixed_bytes(g, true, g.Skv) + score_chunk_bytes(g, true, ni, g.Skv) +
                               align256((size_t)g.B * g.Hq * ni * 4)
                         : 0;
    return bwd_fixed_bytes(g) + bwd_chunk_bytes(g, ni) + sc;
}

size_t det_attn_backward_workspace_size(const det_tensor *q, const det_tensor *k, const det_tensor *v,
                                        int32_t causal) {
    if (check_qkv(q, k, v, causal)) return 0;
    const AttnGeom g = geom(q, k, causal, 1.0);
    const bool mf = use_mfma_scores(q);
    return default_size(g.Sq, [&](int64_t ni) { return bytes_backward(g, mf, ni); });
}

int det_attn_backward(const det_tensor *q, const det_tensor *k, const det_tensor *v, const det_tensor *o,
                      const det_tensor *dout, const float *rowmax, const double *den64, int32_t causal,
                      double scale, const det_out *dq, const det_out *dk, const det_out *dv, void *workspace,
                      size_t ws_bytes, void *stream) {
    int rc;
    if ((rc = check_qkv(q, k, v, causal))) return rc;
    if ((rc = check_grad_operand(o, q, "o")) || (rc = check_grad_operand(dout, q, "dout"))) return rc;
    if (q->S > 0 && (rc = check_out(dq))) return rc;
    if (k->S > 0 && ((rc = check_out(dk)) || (rc = check_out(dv)))) return rc;
    if (q->S > 0 && k->S > 0 && (!rowmax || !den64)) return fail(DET_E_NULL, "rowmax or den64 is NULL");
    const AttnGeom g = geom(q, k, causal, scale);
    const bool mf = use_mfma_scores(q);
    auto need = [&](int64_t ni) { return bytes_backward(g, mf, ni); };
    const bool work = g.Sq > 0 && g.Skv > 0;
    if ((rc = check_ws(workspace, ws_bytes, work ? need(std::min<int64_t>(g.Sq, kRowTile)) : 0))) return rc;
    hipStream_t s = (hipStream_t)stream;
    if (!work) {  // no pair: every gradient is zero
        if (g.Sq > 0) HIP_TRY(launch_zero_view(OutView{dq->data, dq->sB, dq->sH, dq->sS}, g.B, g.Hq, g.Sq, g.D, s), "zero dq");
        if (g.Skv > 0) {
            HIP_TRY(launch_zero_view(OutView{dk->data, dk->sB, dk->sH, dk->sS}, g.B, g.Hkv, g.Skv, g.D, s), "zero dk");
            HIP_TRY(launch_zero_view(OutView{dv->data, dv->sB, dv->sH, dv->sS}, g.B, g.Hkv, g.Skv, g.D, s), "zero dv");
        }
        return ok();
    }
    const int64_t chunk = choose_chunk(g.Sq, ws_bytes, need);
    Carver c0{(char *)workspace, ws_bytes};
    void *fixed = c0.take<char>(bwd_fixed_bytes(g));
    void *cws = c0.take<char>(bwd_chunk_bytes(g, chunk));
    void *kprep = mf ? c0.take<char>(score_fixed_bytes(g, true, g.Skv)) : nullptr;
    void *sws = mf ? c0.take<char>(score_chunk_bytes(g, true, chunk, g.Skv)) : nullptr;
    uint32_t *keys = mf ? c0.take<uint32_t>(g.B * g.Hq * chunk) : nullptr;
    if (c0.over) return fail(DET_E_WORKSPACE, "internal: workspace layout exceeds its computed size");
    const Tensor tq = to_t(q), tk = to_t(k);
    const ScoreFn scores = [&](int64_t i0, int64_t i1, float *out) {
        return run_scores(tq, tk, tk, g, true, kprep, i0 == 0, true, nullptr, sws, i0, i1, 0, g.Skv, out, keys, i1 - i0,
                          i0, s);
    };
    HIP_TRY(launch_attn_backward(tq, tk, to_t(v), to_t(o), to_t(dout), rowmax, den64, g, fixed, cws, chunk,
                                 OutView{dq->data, dq->sB, dq->sH, dq->sS}, OutView{dk->data, dk->sB, dk->sH, dk->sS},
                                 OutView{dv->data, dv->sB, dv->sH, dv->sS}, force_fallback(), mf ? &scores : nullptr, s),
            "backward");
    return ok();
}

// ------------------------------------------------------------------ sharded

namespace {
int check_splits(const det_tensor *k, const int64_t *splits, int32_t n, const int32_t *order) {
    if (n < 1) return fail(DET_E_VALUE, "need at least one KV split");
    if (!splits) return fail(DET_E_NULL, "kv_splits is NULL");
    int64_t sum = 0;
    for (int32_t a = 0; a < n; ++a) {
        if (splits[a] < 0) return fail(DET_E_VALUE, "negative split length");
        sum += splits[a];
    }
    if (sum != k->S) return fail(DET_E_VALUE, "kv_splits sum to %lld, Skv is %lld", (long long)sum, (long long)k->S);
    if (order) {
        std::vector<char> seen(n, 0);
        for (int32_t a = 0; a < n; ++a) {
            if (order[a] < 0 || order[a] >= n || seen[order[a]]) return fail(DET_E_VALUE, "order is not a permutation");
            seen[order[a]] = 1;
        }
    }
    return DET_OK;
}
int64_t max_split(const int64_t *splits, int32_t n) {
    int64_t m = 0;
    for (int32_t a = 0; a < n; ++a) m = std::max(m, splits[a]);
    return m;
}
}  // namespace

size_t det_attn_sharded_workspace_size(const det_tensor *q, const det_tensor *k, const det_tensor *v,
                                       const int64_t *kv_splits, int32_t n_splits, int32_t causal) {
    if (check_qkv(q, k, v, causal) || check_splits(k, kv_splits, n_splits, nullptr)) return 0;
    const AttnGeom g = geom(q, k, causal, 1.0);
    const bool mf = use_mfma_scores(q);
    const int64_t ml = max_split(kv_splits, n_splits);
    const bool recomp = recompute_scores(mf, g, ml, kDefaultBudget, [&] {
        return bytes_sharded(g, mf, false, std::max<int64_t>(std::min<int64_t>(g.Sq, kRowTile), 1), ml);
    });
    return default_size(g.Sq, [&](int64_t ni) { return bytes_sharded(g, mf, recomp, ni, ml); });
}

int det_attn_sharded(const det_tensor *q, const det_tensor *k, const det_tensor *v, const int64_t *kv_splits,
                     int32_t n_splits, const int32_t *order, int32_t causal, double scale, const det_out *o,
                     void *workspace, size_t ws_bytes, void *stream) {
    int rc;
    if ((rc = check_qkv(q, k, v, causal)) || (rc = check_splits(k, kv_splits, n_splits, order))) return rc;
    if (q->S > 0 && (rc = check_out(o))) return rc;
    const AttnGeom g = geom(q, k, causal, scale);
    const bool mf = use_mfma_scores(q);
    const int64_t ml = max_split(kv_splits, n_splits);
    const bool recomp = recompute_scores(mf, g, ml, ws_bytes, [&] {
        return bytes_sharded(g, mf, false, std::max<int64_t>(std::min<int64_t>(g.Sq, kRowTile), 1), ml);
    });
    auto need = [&](int64_t ni) { return bytes_sharded(g, mf, recomp, ni, ml); };
    if ((rc = check_ws(workspace, ws_bytes, g.Sq > 0 ? need(std::min<int64_t>(g.Sq, kRowTile)) : 0))) return rc;
    if (g.Sq == 0) return ok();
    hipStream_t s = (hipStream_t)stream;
    const Tensor tq = to_t(q), tk = to_t(k), tv = to_t(v);
    const OutView ov{o->data, o->sB, o->sH, o->sS};
    std::vector<int64_t> lo(n_splits);
    int64_t run = 0;
    for (int32_t a = 0; a < n_splits; ++a) {
        lo[a] = run;
        run += kv_splits[a];
    }
    const int64_t chunk = choose_chunk(g.Sq, ws_bytes, need), bh = g.B * g.Hq;
    const int ff = force_fallback();
    for (int64_t i0 = 0; i0 < g.Sq; i0 += chunk) {
        const int64_t i1 = std::min(g.Sq, i0 + chunk), ni = i1 - i0, rows = bh * ni;
        Carver c{(char *)workspace, ws_bytes};
        VPrep vp = carve_vprep(c, g, ml);
        void *kprep = c.take<char>(score_fixed_bytes(g, mf, ml));
        void *cws = c.take<char>(score_chunk_bytes(g, mf, ni, ml));
        uint32_t *keys = c.take<uint32_t>(rows);
        float *sc = recomp ? nullptr : c.take<float>(rows * ml);
        float *rm_acc = c.take<float>(rows);
        int *flags = c.take<int>(bh * ((ni + 31) / 32));
        int64_t *num_acc = c.take<int64_t>(kNumDigits * rows * g.D);
        int64_t *den_acc = c.take<int64_t>(kDenDigits * rows);
        if (c.over) return fail(DET_E_WORKSPACE, "internal: workspace layout exceeds its computed size");
        // pass 1: the rowmax of each shard, composed by max: every shard's score
        // launch max-reduces its rows into the same order keys (an integer max,
        // so the result does not depend on the order); Q's digits are prepared by
        // the first shard's launch and kept for every later launch of this chunk
        bool any = false;
        for (int32_t a = 0; a < n_splits; ++a) {
            const int32_t sh = order ? order[a] : a;
            const int64_t l = lo[sh], h = l + kv_splits[sh];
            if (h <= l) continue;  // an empty shard has no scores: its max is -inf, the identity
            HIP_TRY(run_scores(tq, tk, tv, g, mf, kprep, true, !any, nullptr, cws, i0, i1, l, h, nullptr, keys, ni, i0,
                               s),
                    "scores");
            any = true;
        }
        if (any) HIP_TRY(launch_keys_to_f32(keys, rm_acc, bh, ni, ni, 0, s), "rowmax");
        else HIP_TRY(launch_fill_u32((uint32_t *)rm_acc, rows, 0xff800000u, s), "fill rowmax");  // -inf
        // pass 2: each shard's digits against the global max, composed by int64 add: the
        // deposit adds its limbs into the shared accumulator (integer atomics), and one
        // carry pass at the end makes the sum canonical
        HIP_TRY(launch_fill_i64(num_acc, kNumDigits * rows * g.D, 0, s), "fill num");
        HIP_TRY(launch_fill_i64(den_acc, kDenDigits * rows, 0, s), "fill den");
        for (int32_t a = 0; a < n_splits; ++a) {
            const int32_t sh = order ? order[a] : a;
            const int64_t l = lo[sh], h = l + kv_splits[sh];
            if (h <= l) continue;
            if (recomp)  // this shard's K and V digit rows; Q's are kept from pass 1
                HIP_TRY(launch_qkv_prep(tq, tk, tv, g, kprep, true, false, &vp, cws, i0, i1, l, h, s), "prepare");
            else
                HIP_TRY(run_scores(tq, tk, tv, g, mf, kprep, true, false, &vp, cws, i0, i1, l, h, sc, nullptr, 0, 0, s),
                        "scores");
            HIP_TRY(launch_pv(tv, g, vp, pv_src(tq, tk, g, recomp, kprep, cws, sc, i0, i1, l, h), rm_acc, nullptr, ni, i0,
                              i0, i1, l, h, flags, nullptr, nullptr, nullptr, num_acc, den_acc, rows, ni, i0, ff, s),
                    "deposit");
        }
        HIP_TRY(launch_normalize(num_acc, rows * g.D, kNumDigits, s), "normalize");
        HIP_TRY(launch_normalize(den_acc, rows, kDenDigits, s), "normalize");
        HIP_TRY(launch_finalize(num_acc, den_acc, rows, ni, i0, bh, g.Hq, i0, i1, g.D, ov, s), "finalize");
    }
    return ok();
}

// ------------------------------------------------------------------ cross-entropy

namespace {
int check_logits(const void *x, int32_t dtype, int64_t N, int64_t V, int64_t ld) {
    if (dtype != DET_F32 && dtype != DET_BF16) return fail(DET_E_DTYPE, "logits dtype %d is not f32/bf16", dtype);
    if (N < 0 || V < 1) return fail(DET_E_SHAPE, "bad logits shape N=%lld V=%lld", (long long)N, (long long)V);
    if (ld < V) return fail(DET_E_STRIDE, "row stride %lld < V=%lld", (long long)ld, (long long)V);
    if (N > 0 && !x) return fail(DET_E_NULL, "logits is NULL");
    return DET_OK;
}
// Range form used by rowmax / denom_digits, where V itself is not passed.
int check_logits_range(const void *x, int32_t dtype, int64_t N, int64_t ld, int64_t lo, int64_t hi) {
    if (dtype != DET_F32 && dtype != DET_BF16) return fail(DET_E_DTYPE, "logits dtype %d is not f32/bf16", dtype);
    if (N < 0 || ld < 1) return fail(DET_E_SHAPE, "bad logits shape N=%lld ld=%lld", (long long)N, (long long)ld);
    if (lo < 0 || hi < lo || hi > ld)
        return fail(DET_E_SHAPE, "vocab range [%lld,%lld) outside the row of %lld", (long long)lo, (long long)hi,
                    (long long)ld);
    if (N > 0 && !x) return fail(DET_E_NULL, "logits is NULL");
    return DET_OK;
}
int check_vrange(int64_t V, int64_t lo, int64_t hi) {
    if (lo < 0 || hi < lo || hi > V) return fail(DET_E_SHAPE, "vocab range [%lld,%lld) outside [0,%lld]", (long long)lo,
                                                 (long long)hi, (long long)V);
    return DET_OK;
}
}  // namespace

int det_ce_rowmax(const void *logits, int32_t dtype, int64_t N, int64_t ld, int64_t v_lo, int64_t v_hi,
                  float *rowmax, void *stream) {
    int rc;
    if ((rc = check_logits_range(logits, dtype, N, ld, v_lo, v_hi))) return rc;
    if (N > 0 && !rowmax) return fail(DET_E_NULL, "rowmax is NULL");
    HIP_TRY(launch_ce_rowmax(logits, dtype, N, ld, v_lo, v_hi, rowmax, (hipStream_t)stream), "ce rowmax");
    return ok();
}

int det_ce_denom_digits(const void *logits, int32_t dtype, int64_t N, int64_t ld, const float *rowmax,
                        int64_t v_lo, int64_t v_hi, int64_t *den, int32_t add_into, void *stream) {
    int rc;
    if ((rc = check_logits_range(logits, dtype, N, ld, v_lo, v_hi))) return rc;
    if (N > 0 && (!rowmax || !den)) return fail(DET_E_NULL, "rowmax or den is NULL");
    HIP_TRY(launch_ce_denom(logits, dtype, N, ld, rowmax, v_lo, v_hi, den, add_into, (hipStream_t)stream),
            "ce denom");
    return ok();
}

int det_ce_finalize(const int64_t *den, const void *logits, int32_t dtype, int64_t N, int64_t V, int64_t ld,
                    const int64_t *targets, const float *rowmax, float *loss, double *denom, void *stream) {
    int rc;
    if ((rc = check_logits(logits, dtype, N, V, ld))) return rc;
    if (N > 0 && (!den || !targets || !rowmax || !loss || !denom)) return fail(DET_E_NULL, "a required pointer is NULL");
    hipStream_t s = (hipStream_t)stream;
    const bool chk = checks_on() && N > 0;
    if (chk && (rc = ce_check_begin(s))) return rc;
    HIP_TRY(launch_ce_finalize(den, logits, dtype, N, V, ld, targets, rowmax, loss, denom, s), "ce finalize");
    return chk ? ce_check_end(s) : ok();
}

size_t det_ce_forward_workspace_size(int64_t) { return 0; }

int det_ce_forward(const void *logits, int32_t dtype, int64_t N, int64_t V, int64_t ld, const int64_t *targets,
                   float *loss, float *rowmax, double *denom, void *, size_t, void *stream) {
    int rc;
    if ((rc = check_logits(logits, dtype, N, V, ld))) return rc;
    if (N > 0 && (!targets || !loss || !rowmax || !denom)) return fail(DET_E_NULL, "a required pointer is NULL");
    hipStream_t s = (hipStream_t)stream;
    const bool chk = checks_on() && N > 0;
    if (chk && (rc = ce_check_begin(s))) return rc;
    HIP_TRY(launch_ce_forward(logits, dtype, N, V, ld, targets, loss, rowmax, denom, s), "ce forward");
    return chk ? ce_check_end(s) : ok();
}

size_t det_ce_reduce_workspace_size(int64_t) { return 0; }

int det_ce_reduce(const float *loss, int64_t N, int32_t reduction, float *out, void *, size_t, void *stream) {
    if (N < 0) return fail(DET_E_SHAPE, "negative N");
    if (reduction < 0 || reduction > 2) return fail(DET_E_VALUE, "reduction %d is not 0/1/2", reduction);
    if (!out || (N > 0 && !loss)) return fail(DET_E_NULL, "loss or out is NULL");
    hipStream_t s = (hipStream_t)stream;
    if (reduction == 0) {
        if (N > 0) HIP_TRY(hipMemcpyAsync(out, loss, N * sizeof(float), hipMemcpyDeviceToDevice, s), "copy");
        return ok();
    }
    HIP_TRY(launch_ce_reduce(loss, N, reduction, out, nullptr, s), "ce reduce");
    return ok();
}

int det_ce_backward(const void *logits, int32_t dtype, int64_t N, int64_t V, int64_t ld, int64_t v0,
                    const int64_t *targets, const float *rowmax, const double *denom, const float *grad_loss,
                    int32_t reduction, float *grad, int64_t grad_ld, void *stream) {
    int rc;
    if ((rc = check_logits(logits, dtype, N, V, ld))) return rc;
    if (v0 < 0) return fail(DET_E_VALUE, "vocabulary offset %lld is negative", (long long)v0);
    if (reduction < 0 || reduction > 2) return fail(DET_E_VALUE, "reduction %d is not 0/1/2", reduction);
    if (grad_ld < V) return fail(DET_E_STRIDE, "grad row stride %lld < V", (long long)grad_ld);
    if (N > 0 && (!targets || !rowmax || !denom || !grad_loss || !grad))
        return fail(DET_E_NULL, "a required pointer is NULL");
    HIP_TRY(launch_ce_backward(logits, dtype, N, V, ld, v0, targets, rowmax, denom, grad_loss, reduction, grad,
                               grad_ld, (hipStream_t)stream),
            "ce backward");
    return ok();
}

}  // extern "C"

namespace det {
int pass2_layout() { return g_pass2_layout.load(std::memory_order_relaxed); }
}  // namespace det
