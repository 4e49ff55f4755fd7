// attn.hip -- attention kernels for gfx950.
//
// Pass 1 (det-attn page, "Method": the global row max) and the score rule:
//   s_ij = RN32(RN64(scale * dot_ij)), dot_ij = fp64 fma chain over d ascending.
// One lane owns one key j and keeps kRowTile chains (one per query row) in
// VGPRs; the query rows come in through scalar loads of a widened fp64 copy of
// Q, so every FMA takes its q operand from an SGPR pair and its k operand from
// a VGPR.  Scores are stored for pass 2 (the chain is not recomputed).
//
// Pass 2 lives in pv.hip; this file also holds the digit compose, carry and
// finalize kernels.
#include "dev_math.hpp"
#include "kernels.hpp"

#include <algorithm>
#include <climits>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

namespace det {

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// ---------------------------------------------------------------- per-kernel timing

namespace {
struct ProfRec {
    const char *name;
    hipEvent_t a, b;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfRec> g_prof;
std::vector<hipEvent_t> g_event_pool;

hipEvent_t pooled_event() {
    if (!g_event_pool.empty()) {
        hipEvent_t e = g_event_pool.back();
        g_event_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}
}  // namespace

ProfScope::ProfScope(const char *name, hipStream_t s) : slot(-1), stream(s) {
    if (!g_prof_on) return;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    ProfRec r{name, pooled_event(), pooled_event()};
    if (!r.a || !r.b) return;
    (void)hipEventRecord(r.a, s);
    slot = (int)g_prof.size();
    g_prof.push_back(r);
}

ProfScope::~ProfScope() {
    if (slot < 0) return;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    (void)hipEventRecord(g_prof[slot].b, stream);
}

void prof_enable(bool on) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    for (auto &r : g_prof) {
        g_event_pool.push_back(r.a);
        g_event_pool.push_back(r.b);
    }
    g_prof.clear();
    g_prof_on = on;
}

size_t prof_report(char *buf, size_t len) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    std::vector<std::string> names;
    std::vector<double> tot;
    std::vector<long> cnt;
    for (auto &r : g_prof) {
        (void)hipEventSynchronize(r.b);
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) continue;
        size_t k = 0;
        while (k < names.size() && names[k] != r.name) ++k;
        if (k == names.size()) {
            names.push_back(r.name);
            tot.push_back(0.0);
            cnt.push_back(0);
        }
        tot[k] += ms;
        cnt[k] += 1;
    }
    std::string out;
    for (size_t k = 0; k < names.size(); ++k) {
        char line[160];
        snprintf(line, sizeof line, "%s %ld %.6f\n", names[k].c_str(), cnt[k], tot[k]);
        out += line;
    }
    if (buf && len) {
        const size_t n = std::min(len - 1, out.size());
        memcpy(buf, out.data(), n);
        buf[n] = 0;
    }
    return out.size() + 1;
}

size_t score_scratch_bytes(const AttnGeom &g, int64_t rows_i, int64_t kv_len) {
    const int64_t bh = g.B * g.Hq;
    return align256((size_t)bh * padded_rows(rows_i) * g.Dp * sizeof(double)) +  // widened Q rows
           align256((size_t)bh * rows_i * sizeof(uint32_t)) +       // rowmax keys
           align256((size_t)bh * rows_i * kv_len * sizeof(float));  // scores / weights
}

// ---------------------------------------------------------------- small kernels

__global__ void k_fill_u32(uint32_t *p, int64_t n, uint32_t v) {
    for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < n; t += (int64_t)gridDim.x * blockDim.x)
        p[t] = v;
}
__global__ void k_fill_i64(int64_t *p, int64_t n, int64_t v) {
    for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < n; t += (int64_t)gridDim.x * blockDim.x)
        p[t] = v;
}

static dim3 grid_for(int64_t n, int block = 256) {
    int64_t g = (n + block - 1) / block;
    return dim3((unsigned)std::max<int64_t>(1, std::min<int64_t>(g, 1 << 20)));
}

hipError_t launch_fill_u32(uint32_t *p, int64_t n, uint32_t v, hipStream_t s) {
    ProfScope prof_("fill", s);
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_fill_u32, grid_for(n), dim3(256), 0, s, p, n, v);
    return hipGetLastError();
}
hipError_t launch_fill_i64(int64_t *p, int64_t n, int64_t v, hipStream_t s) {
    ProfScope prof_("fill", s);
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_fill_i64, grid_for(n), dim3(256), 0, s, p, n, v);
    return hipGetLastError();
}

// Widen query rows [i0,i1) of every (b,hq) to fp64, rows padded with zeros to
// Dp (a zero k and zero q add exactly +0 to a chain that is never -0).
template <typename T>
__global__ void k_widen_q(const T *__restrict__ q, int64_t sB, int64_t sH, int64_t sS, int64_t Hq, int64_t D,
                          int64_t Dp, int64_t i0, int64_t ni, int64_t ni_pad, int64_t total,
                          double *__restrict__ out) {
    for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total; t += (int64_t)gridDim.x * blockDim.x) {
        const int64_t d = t % Dp;
        const int64_t r = t / Dp;
        const int64_t ii = r % ni_pad;
        const int64_t bh = r / ni_pad;
        const int64_t b = bh / Hq, h = bh % Hq;
        double x = 0.0;
        if (d < D && ii < ni) x = (double)elem<T>::to_f32(q[b * sB + h * sH + (i0 + ii) * sS + d]);
        out[t] = x;
    }
}

hipError_t launch_widen_q(const Tensor &q, const AttnGeom &g, int64_t i0, int64_t i1, double *q64,
                          hipStream_t s) {
    ProfScope prof_("widen_q", s);
    const int64_t ni = i1 - i0, ni_pad = padded_rows(ni), total = g.B * g.Hq * ni_pad * g.Dp;
    if (total <= 0) return hipSuccess;
    if (q.dtype == 0)
        hipLaunchKernelGGL(k_widen_q<float>, grid_for(total), dim3(256), 0, s, (const float *)q.data, q.sB, q.sH,
                           q.sS, g.Hq, g.D, g.Dp, i0, ni, ni_pad, total, q64);
    else
        hipLaunchKernelGGL(k_widen_q<bf16_t>, grid_for(total), dim3(256), 0, s, (const bf16_t *)q.data, q.sB,
                           q.sH, q.sS, g.Hq, g.D, g.Dp, i0, ni, ni_pad, total, q64);
    return hipGetLastError();
}

// ---------------------------------------------------------------- pass 1: scores

// The widened query tile (kRowTile rows x DP doubles, zero-padded rows and
// columns) is staged once per block in LDS; every lane of a wave reads the same
// address there (a broadcast, no bank conflicts), so no query value is held in
// scalar registers and the tile loop carries no spills.
template <typename TK, int DP>
__global__ __launch_bounds__(256) void k_scores(const double *__restrict__ q64, const TK *__restrict__ kp,
                                                int64_t ksB, int64_t ksH, int64_t ksS, int64_t Hq, int64_t group,
                                                int64_t D, int causal, double scale, int64_t i0, int64_t i1,
                                                int64_t ni_pad, int64_t kv_lo, int64_t kv_hi,
                                                float *__restrict__ scores, uint32_t *__restrict__ rowmax_keys,
                                                int64_t key_rows, int64_t key_row0) {
    constexpr int RT = kRowTile;
    constexpr int DC = 8;  // head-dim slice per step
    __shared__ double qs[RT * DP];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t bh = blockIdx.z;
    const int64_t b = bh / Hq, hq = bh % Hq, hk = hq / group;
    const int64_t ni = i1 - i0;
    const int64_t ir0 = i0 + (int64_t)blockIdx.y * RT;
    if (ir0 >= i1) return;
    const int nrows = (int)min64(RT, i1 - ir0);
    const int64_t W = kv_hi - kv_lo;
    const double *qtile = q64 + (bh * ni_pad + (ir0 - i0)) * DP;
    for (int t = threadIdx.x; t < RT * DP; t += blockDim.x) qs[t] = qtile[t];
    __syncthreads();
    const TK *kbase = kp + b * ksB + hk * ksH;

    uint32_t mkey[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) mkey[r] = kKeyNegInf;

    for (int64_t tile = blockIdx.x;; tile += gridDim.x) {
        const int64_t jt0 = kv_lo + tile * kKeyTile;
        if (jt0 >= kv_hi) break;
        if (causal && jt0 > ir0 + nrows - 1) break;  // this and later tiles are masked
        const int64_t j = jt0 + wave * 64 + lane;
        const bool jv = j < kv_hi;
        const TK *krow = kbase + (jv ? j : kv_lo) * ksS;
        double acc[RT];
#pragma unroll
        for (int r = 0; r < RT; ++r) acc[r] = 0.0;
#pragma unroll 1
        for (int dc = 0; dc < DP; dc += DC) {
            double kv[DC];
#pragma unroll
            for (int u = 0; u < DC; ++u)
                kv[u] = (jv && dc + u < D) ? (double)elem<TK>::to_f32(krow[dc + u]) : 0.0;
            const double *qd = qs + dc;
#pragma unroll
            for (int r = 0; r < RT; ++r) {
#pragma unroll
                for (int u = 0; u < DC; ++u) acc[r] = fma(qd[r * DP + u], kv[u], acc[r]);
            }
        }
        // one running address for the tile's score rows (a per-row address
        // for each of the RT rows would be RT scalar pairs live at once)
        float *srow = scores ? scores + (bh * ni + (ir0 - i0)) * W + (j - kv_lo) : nullptr;
        // the key's offset from the tile's first row, clamped to [-1, RT]:
        // key j is visible to row ir0 + r under the causal mask iff dj <= r
        const int dj = (int)max64(-1, min64(RT, j - ir0));
        // rows past the chunk's end are zero padding: their scores are not
        // stored and their maxima never leave the kernel (a per-lane bound,
        // so the row tests are made where they are used)
        int nrows_v;  // (a vector copy the compiler cannot split back into 32 scalar tests)
        asm volatile("v_mov_b32 %0, %1" : "=v"(nrows_v) : "s"(nrows));
        const int lim = jv ? nrows_v : 0;
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            const float sc = (float)(scale * acc[r]);
            if (srow && r < lim) *srow = sc;
            if (jv && (!causal || dj <= r)) mkey[r] = max(mkey[r], order_key(sc));
            if (srow) srow += W;
        }
    }
    if (!rowmax_keys) return;
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        if (r < nrows) {
            uint32_t m = mkey[r];
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
            if (lane == 0) atomicMax(&rowmax_keys[bh * key_rows + (ir0 + r - key_row0)], m);
        }
    }
}

template <typename TK, int DP>
static void launch_scores_dp(dim3 grid, const Tensor &k, const AttnGeom &g, const double *q64, int64_t i0,
                             int64_t i1, int64_t kv_lo, int64_t kv_hi, float *scores, uint32_t *rowmax_keys,
                             int64_t key_rows, int64_t key_row0, hipStream_t s) {
    hipLaunchKernelGGL((k_scores<TK, DP>), grid, dim3(256), 0, s, q64, (const TK *)k.data, k.sB, k.sH, k.sS, g.Hq,
                       g.Hq / g.Hkv, g.D, g.causal, g.scale, i0, i1, padded_rows(i1 - i0), kv_lo, kv_hi, scores,
                       rowmax_keys, key_rows, key_row0);
}

template <typename TK>
static void launch_scores_t(dim3 grid, const Tensor &k, const AttnGeom &g, const double *q64, int64_t i0,
                            int64_t i1, int64_t kv_lo, int64_t kv_hi, float *scores, uint32_t *rowmax_keys,
                            int64_t key_rows, int64_t key_row0, hipStream_t s) {
    switch (g.Dp) {
    case 16: launch_scores_dp<TK, 16>(grid, k, g, q64, i0, i1, kv_lo, kv_hi, scores, rowmax_keys, key_rows, key_row0, s); break;
    case 32: launch_scores_dp<TK, 32>(grid, k, g, q64, i0, i1, kv_lo, kv_hi, scores, rowmax_keys, key_rows, key_row0, s); break;
    case 64: launch_scores_dp<TK, 64>(grid, k, g, q64, i0, i1, kv_lo, kv_hi, scores, rowmax_keys, key_rows, key_row0, s); break;
    case 128: launch_scores_dp<TK, 128>(grid, k, g, q64, i0, i1, kv_lo, kv_hi, scores, rowmax_keys, key_rows, key_row0, s); break;
    default: launch_scores_dp<TK, 256>(grid, k, g, q64, i0, i1, kv_lo, kv_hi, scores, rowmax_keys, key_rows, key_row0, s); break;
    }
}

hipError_t launch_scores(const Tensor &k, const AttnGeom &g, const double *q64, int64_t i0, int64_t i1,
                         int64_t kv_lo, int64_t kv_hi, float *scores, uint32_t *rowmax_keys, int64_t key_rows,
                         int64_t key_row0, hipStream_t s) {
    ProfScope prof_("scores", s);
    const int64_t ni = i1 - i0;
    if (ni <= 0 || kv_hi <= kv_lo) return hipSuccess;
    const int64_t ktiles = (kv_hi - kv_lo + kKeyTile - 1) / kKeyTile;
    const int64_t parts = std::min<int64_t>(ktiles, 8);
    dim3 grid((unsigned)parts, (unsigned)((ni + kRowTile - 1) / kRowTile), (unsigned)(g.B * g.Hq));
    if (k.dtype == 0)
        launch_scores_t<float>(grid, k, g, q64, i0, i1, kv_lo, kv_hi, scores, rowmax_keys, key_rows, key_row0, s);
    else
        launch_scores_t<bf16_t>(grid, k, g, q64, i0, i1, kv_lo, kv_hi, scores, rowmax_keys, key_rows, key_row0, s);
    return hipGetLastError();
}

__global__ void k_keys_to_f32(const uint32_t *__restrict__ keys, float *__restrict__ out, int64_t BHq, int64_t rows,
                              int64_t out_rows, int64_t out_row0) {
    const int64_t n = BHq * rows;
    for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < n; t += (int64_t)gridDim.x * blockDim.x) {
        const int64_t bh = t / rows, r = t % rows;
        out[bh * out_rows + out_row0 + r] = key_value(keys[t]);
    }
}

__global__ void k_rowmax_below(const float *__restrict__ supplied, const float *__restrict__ computed, int64_t BHq,
                               int64_t rows, int64_t out_rows, int64_t row0, unsigned int *bad) {
    const int64_t n = BHq * rows;
    for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < n; t += (int64_t)gridDim.x * blockDim.x) {
        const int64_t at = (t / rows) * out_rows + row0 + t % rows;
        if (computed[at] > supplied[at]) atomicAdd(bad, 1u);
    }
}

hipError_t launch_rowmax_below(const float *supplied, const float *computed, int64_t BHq, int64_t rows,
                               int64_t out_rows, int64_t row0, unsigned int *bad, hipStream_t s) {
    if (BHq * rows <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_rowmax_below, grid_for(BHq * rows), dim3(256), 0, s, supplied, computed, BHq, rows,
                       out_rows, row0, bad);
    return hipGetLastError();
}

hipError_t launch_keys_to_f32(const uint32_t *keys, float *out, int64_t BHq, int64_t rows, int64_t out_rows,
                              int64_t out_row0, hipStream_t s) {
    ProfScope prof_("keys_to_f32", s);
    if (BHq * rows <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_keys_to_f32, grid_for(BHq * rows), dim3(256), 0, s, keys, out, BHq, rows, out_rows,
                       out_row0);
    return hipGetLastError();
}

// ---------------------------------------------------------------- digits

template <int K>
__global__ void k_normalize(int64_t *__restrict__ dg, int64_t n) {
    for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < n; t += (int64_t)gridDim.x * blockDim.x) {
        int64_t d[K];
#pragma unroll
        for (int k = 0; k < K; ++k) d[k] = dg[k * n + t];
        canonicalize<K>(d);
#pragma unroll
        for (int k = 0; k < K; ++k) dg[k * n + t] = d[k];
    }
}

template <int K>
__global__ void k_digits_combine(int64_t *__restrict__ acc, const int64_t *__restrict__ part, int64_t n) {
    for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < n; t += (int64_t)gridDim.x * blockDim.x) {
        int64_t d[K];
#pragma unroll
        for (int k = 0; k < K; ++k) d[k] = acc[k * n + t] + part[k * n + t];
        canonicalize<K>(d);
#pragma unroll
        for (int k = 0; k < K; ++k) acc[k * n + t] = d[k];
    }
}

// Rows [i0, i1) of head blockIdx.y: values bh*rows*width + i0*width + t,
// t < (i1 - i0) * width, digit k at k * plane.
template <int K>
__global__ void k_normalize_rows(int64_t *__restrict__ dg, int64_t plane, int64_t rows, int64_t i0, int64_t run,
                                 int64_t width) {
    const int64_t base = (int64_t)blockIdx.y * rows * width + i0 * width;
    for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < run; t += (int64_t)gridDim.x * blockDim.x) {
        int64_t d[K];
#pragma unroll
        for (int k = 0; k < K; ++k) d[k] = dg[k * plane + base + t];
        canonicalize<K>(d);
#pragma unroll
        for (int k = 0; k < K; ++k) dg[k * plane + base + t] = d[k];
    }
}

__global__ void k_fill_rows_i64(int64_t *__restrict__ p, int64_t plane, int64_t rows, int64_t i0, int64_t run,
                                int64_t width, int64_t v) {
    int64_t *q = p + (int64_t)blockIdx.z * plane + (int64_t)blockIdx.y * rows * width + i0 * width;
    for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < run; t += (int64_t)gridDim.x * blockDim.x)
        q[t] = v;
}

static dim3 grid_rows(int64_t run, int64_t n_bh, int64_t nz = 1) {
    const int64_t g = std::min<int64_t>((run + 255) / 256, 4096);
    return dim3((unsigned)std::max<int64_t>(g, 1), (unsigned)n_bh, (unsigned)nz);
}

hipError_t launch_normalize_rows(int64_t *digits, int n_digits, int64_t plane, int64_t n_bh, int64_t rows,
                                 int64_t i0, int64_t i1, int64_t width, hipStream_t s) {
    ProfScope prof_("normalize", s);
    const int64_t run = (i1 - i0) * width;
    if (run <= 0 || n_bh <= 0) return hipSuccess;
    for (int64_t b0 = 0; b0 < n_bh; b0 += 65535) {  // grid y holds at most 65535 heads per launch
        const int64_t nb = std::min<int64_t>(65535, n_bh - b0);
        int64_t *dg = digits + b0 * rows * width;
        if (n_digits == kNumDigits)
            hipLaunchKernelGGL(k_normalize_rows<kNumDigits>, grid_rows(run, nb), dim3(256), 0, s, dg, plane, rows, i0,
                               run, width);
        else
            hipLaunchKernelGGL(k_normalize_rows<kDenDigits>, grid_rows(run, nb), dim3(256), 0, s, dg, plane, rows, i0,
                               run, width);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_fill_rows_i64(int64_t *p, int n_planes, int64_t plane, int64_t n_bh, int64_t rows, int64_t i0,
                                int64_t i1, int64_t width, int64_t v, hipStream_t s) {
    ProfScope prof_("fill", s);
    const int64_t run = (i1 - i0) * width;
    if (run <= 0 || n_bh <= 0 || n_planes <= 0) return hipSuccess;
    for (int64_t b0 = 0; b0 < n_bh; b0 += 65535) {  // grid y holds at most 65535 heads per launch
        const int64_t nb = std::min<int64_t>(65535, n_bh - b0);
        hipLaunchKernelGGL(k_fill_rows_i64, grid_rows(run, nb, n_planes), dim3(256), 0, s, p + b0 * rows * width,
                           plane, rows, i0, run, width, v);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_normalize(int64_t *digits, int64_t n_values, int n_digits, hipStream_t s) {
    ProfScope prof_("normalize", s);
    if (n_values <= 0) return hipSuccess;
    if (n_digits == kNumDigits)
        hipLaunchKernelGGL(k_normalize<kNumDigits>, grid_for(n_values), dim3(256), 0, s, digits, n_values);
    else
        hipLaunchKernelGGL(k_normalize<kDenDigits>, grid_for(n_values), dim3(256), 0, s, digits, n_values);
    return hipGetLastError();
}

hipError_t launch_digits_combine(int64_t *acc, const int64_t *part, int64_t n_values, int n_digits,
                                 hipStream_t s) {
    ProfScope prof_("digits_combine", s);
    if (n_values <= 0) return hipSuccess;
    if (n_digits == kNumDigits)
        hipLaunchKernelGGL(k_digits_combine<kNumDigits>, grid_for(n_values), dim3(256), 0, s, acc, part,
                           n_values);
    else
        hipLaunchKernelGGL(k_digits_combine<kDenDigits>, grid_for(n_values), dim3(256), 0, s, acc, part,
                           n_values);
    return hipGetLastError();
}

__global__ void k_rowmax_combine(float *__restrict__ acc, const float *__restrict__ part, int64_t n) {
    for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < n; t += (int64_t)gridDim.x * blockDim.x)
        acc[t] = key_value(max(order_key(acc[t]), order_key(part[t])));
}

hipError_t launch_rowmax_combine(float *acc, const float *part, int64_t n, hipStream_t s) {
    ProfScope prof_("rowmax_combine", s);
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_rowmax_combine, grid_for(n), dim3(256), 0, s, acc, part, n);
    return hipGetLastError();
}

// ---------------------------------------------------------------- finalize

// One block of 64 threads per output row (blockIdx.x = bh * ni + ii), its
// threads striding over the head dim: the row's indices are wave-uniform and
// computed once, not per element.
__global__ __launch_bounds__(64) void k_finalize(const int64_t *__restrict__ num, const int64_t *__restrict__ den,
                                                 int64_t plane_rows, int64_t rows_per_bh, int64_t row0, int64_t Hq,
                                                 int64_t i0, int64_t ni, int64_t D, float *__restrict__ o,
                                                 int64_t osB, int64_t osH, int64_t osS) {
    const int64_t r = blockIdx.x;
    const int64_t ii = r % ni, bh = r / ni;
    const int64_t i = i0 + ii;
    const int64_t prow = bh * rows_per_bh + (i - row0);
    const int64_t b = bh / Hq, h = bh % Hq;
    int64_t dd[kDenDigits];
#pragma unroll
    for (int k = 0; k < kDenDigits; ++k) dd[k] = den[k * plane_rows + prow];
    canonicalize<kDenDigits>(dd);
    const double d64 = digits_to_f64<kDenDigits>(dd, kDenElo);
    const int64_t nplane = plane_rows * D;
    const int64_t *nrow = num + prow * D;
    float *orow = o + b * osB + h * osH + i * osS;
    for (int64_t d = threadIdx.x; d < D; d += 64) {
        int64_t nd[kNumDigits];
#pragma unroll
        for (int k = 0; k < kNumDigits; ++k) nd[k] = nrow[k * nplane + d];
        canonicalize<kNumDigits>(nd);
        orow[d] = (float)(digits_to_f64<kNumDigits>(nd, kNumElo) / d64);
    }
}

hipError_t launch_finalize(const int64_t *num, const int64_t *den, int64_t plane_rows, int64_t rows_per_bh,
                           int64_t row0, int64_t B_Hq, int64_t Hq, int64_t i0, int64_t i1, int64_t D,
                           const OutView &o, hipStream_t s) {
    ProfScope prof_("finalize", s);
    const int64_t ni = i1 - i0, rows = B_Hq * ni;
    if (rows <= 0 || D <= 0) return hipSuccess;
    if (rows > INT32_MAX) return hipErrorInvalidValue;  // one block per row
    hipLaunchKernelGGL(k_finalize, dim3((unsigned)rows), dim3(64), 0, s, num, den, plane_rows, rows_per_bh, row0, Hq,
                       i0, ni, D, o.data, o.sB, o.sH, o.sS);
    return hipGetLastError();
}

}  // namespace det
