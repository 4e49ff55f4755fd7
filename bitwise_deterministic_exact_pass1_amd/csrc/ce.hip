// ce.hip -- deterministic cross-entropy kernels for gfx950 (det-cross-entropy
// page, "Method": global row max m_i, exact den_i = sum_v exp(x_iv - m_i) in a
// long accumulator, loss = logsumexp - x_{i,t_i}, gradient softmax - onehot).
//
// One workgroup owns one token row.  Each thread keeps an exact binary64
// window over its strided share of the vocabulary and flushes it into nine
// radix-2^32 digits held in LDS with integer atomics; thread 0 then carries the
// digits to canonical form.  Integer addition is associative, so the digits
// are a fixed function of the row however the threads interleave.
#include "dev_math.hpp"
#include "kernels.hpp"

#include <algorithm>

namespace det {

constexpr int kCeThreads = 256;

// Rows whose target lies outside [0, V): their logit is not read and their
// loss is NaN.  Counted here (per device) for the library's optional checks.
__device__ unsigned int g_ce_bad_targets;

static dim3 ce_grid(int64_t n) {
    return dim3((unsigned)std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, 1 << 20)));
}

template <typename T>
__device__ __forceinline__ float ce_load(const void *x, int64_t ld, int64_t i, int64_t v) {
    return elem<T>::to_f32(((const T *)x)[i * ld + v]);
}

// Block-wide max of order keys (sh holds one word per wave); every thread gets the result.
__device__ __forceinline__ uint32_t block_max_key(uint32_t k, uint32_t *sh) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) k = max(k, (uint32_t)__shfl_xor((int)k, off, 64));
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) sh[wave] = k;
    __syncthreads();
    uint32_t r = sh[0];
    for (int w = 1; w < (int)(blockDim.x / 64); ++w) r = max(r, sh[w]);
    __syncthreads();
    return r;
}

template <typename T>
__device__ __forceinline__ float row_max(const void *x, int64_t ld, int64_t i, int64_t v_lo, int64_t v_hi,
                                         uint32_t *sh) {
    uint32_t k = kKeyNegInf;
    for (int64_t v = v_lo + threadIdx.x; v < v_hi; v += kCeThreads) k = max(k, order_key(ce_load<T>(x, ld, i, v)));
    return key_value(block_max_key(k, sh));
}

// Exact den digits of one row into the 9 LDS digits `sd` (zeroed by the caller).
template <typename T>
__device__ __forceinline__ void row_denom(const void *x, int64_t ld, int64_t i, float m, int64_t v_lo, int64_t v_hi,
                                          int64_t *sd) {
    Window win;
    win.init();
    for (int64_t v = v_lo + threadIdx.x; v < v_hi; v += kCeThreads) {
        const float w = weight(ce_load<T>(x, ld, i, v), m);
        if (w != 0.0f) {
            const int ew = f32_exp(w);
            win.add<kDenDigits>((double)w, max(ew, -126) - 23, ew + 1, kDenGcap, kDenElo, sd, 1);
        }
    }
    win.flush<kDenDigits>(kDenElo, sd, 1);
}

template <typename T>
__global__ __launch_bounds__(kCeThreads) void k_ce_rowmax(const void *x, int64_t ld, int64_t v_lo, int64_t v_hi,
                                                          float *rowmax) {
    __shared__ uint32_t sh[kCeThreads / 64];
    const int64_t i = blockIdx.x;
    const float m = row_max<T>(x, ld, i, v_lo, v_hi, sh);
    if (threadIdx.x == 0) rowmax[i] = m;
}

template <typename T>
__global__ __launch_bounds__(kCeThreads) void k_ce_denom(const void *x, int64_t N, int64_t ld,
                                                         const float *rowmax, int64_t v_lo, int64_t v_hi,
                                                         int64_t *den, int add_into) {
    __shared__ int64_t sd[kDenDigits];
    const int64_t i = blockIdx.x;
    if (threadIdx.x < kDenDigits) sd[threadIdx.x] = 0;
    __syncthreads();
    row_denom<T>(x, ld, i, rowmax[i], v_lo, v_hi, sd);
    __syncthreads();
    if (threadIdx.x == 0) {
        int64_t d[kDenDigits];
#pragma unroll
        for (int k = 0; k < kDenDigits; ++k) d[k] = sd[k] + (add_into ? den[k * N + i] : 0);
        canonicalize<kDenDigits>(d);
#pragma unroll
        for (int k = 0; k < kDenDigits; ++k) den[k * N + i] = d[k];
    }
}

// loss_i = RN32(RN64(RN64(m + log_det(RN64(den))) - x_t)); denom_i = RN64(den).
template <typename T>
__device__ __forceinline__ void ce_loss(const int64_t (&dd)[kDenDigits], const void *x, int64_t ld, int64_t i,
                                        int64_t V, int64_t t, float m, float *loss, double *denom) {
    const double d64 = digits_to_f64<kDenDigits>(dd, kDenElo);
    const double lse = (double)m + log_det(d64);
    double xt = __builtin_nan("");
    if (t >= 0 && t < V) xt = (double)ce_load<T>(x, ld, i, t);
    else atomicAdd(&g_ce_bad_targets, 1u);
    loss[i] = (float)(lse - xt);
    denom[i] = d64;
}

// The same loss from a target logit already loaded (xt, exact in f32).
__device__ __forceinline__ void ce_loss_of(const int64_t (&dd)[kDenDigits], float xt, float m, int64_t i,
                                           float *loss, double *denom) {
    const double d64 = digits_to_f64<kDenDigits>(dd, kDenElo);
    const double lse = (double)m + log_det(d64);
    loss[i] = (float)(lse - (double)xt);
    denom[i] = d64;
}

template <typename T>
__global__ void k_ce_finalize(const int64_t *den, const void *x, int64_t N, int64_t V, int64_t ld,
                              const int64_t *targets, const float *rowmax, float *loss, double *denom) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < N; i += (int64_t)gridDim.x * blockDim.x) {
        int64_t d[kDenDigits];
#pragma unroll
        for (int k = 0; k < kDenDigits; ++k) d[k] = den[k * N + i];
        canonicalize<kDenDigits>(d);
        ce_loss<T>(d, x, ld, i, V, targets[i], rowmax[i], loss, denom);
    }
}

// Fused forward over the whole vocabulary: max, exact den, loss in one block per row.
template <typename T>
__global__ __launch_bounds__(kCeThreads) void k_ce_forward(const void *x, int64_t V, int64_t ld,
                                                           const int64_t *targets, float *loss, float *rowmax,
                                                           double *denom) {
    __shared__ uint32_t sh[kCeThreads / 64];
    __shared__ int64_t sd[kDenDigits];
    const int64_t i = blockIdx.x;
    if (threadIdx.x < kDenDigits) sd[threadIdx.x] = 0;
    const float m = row_max<T>(x, ld, i, 0, V, sh);  // contains __syncthreads
    row_denom<T>(x, ld, i, m, 0, V, sd);
    __syncthreads();
    if (threadIdx.x == 0) {
        int64_t d[kDenDigits];
#pragma unroll
        for (int k = 0; k < kDenDigits; ++k) d[k] = sd[k];
        canonicalize<kDenDigits>(d);
        rowmax[i] = m;
        ce_loss<T>(d, x, ld, i, V, targets[i], m, loss, denom);
    }
}

// S = exact sum of the f32 losses; sum -> RN32(RN64(S)), mean -> RN32(RN64(RN64(S)/N)).
__global__ __launch_bounds__(1024) void k_ce_reduce(const float *loss, int64_t N, int reduction, float *out) {
    __shared__ int64_t sd[kDenDigits];
    if (threadIdx.x < kDenDigits) sd[threadIdx.x] = 0;
    __syncthreads();
    Window win;
    win.init();
    for (int64_t i = threadIdx.x; i < N; i += blockDim.x) {
        const float l = loss[i];
        if (l != 0.0f) {
            const int e = f32_exp(l);
            win.add<kDenDigits>((double)l, max(e, -126) - 23, e + 1, kDenGcap, kDenElo, sd, 1);
        }
    }
    win.flush<kDenDigits>(kDenElo, sd, 1);
    __syncthreads();
    if (threadIdx.x == 0) {
        int64_t d[kDenDigits];
#pragma unroll
        for (int k = 0; k < kDenDigits; ++k) d[k] = sd[k];
        canonicalize<kDenDigits>(d);
        const double s = digits_to_f64<kDenDigits>(d, kDenElo);
        out[0] = reduction == 1 ? (float)(s / (double)N) : (float)s;
    }
}

template <typename T>
__global__ void k_ce_backward(const void *x, int64_t N, int64_t V, int64_t ld, int64_t v0, const int64_t *targets,
                              const float *rowmax, const double *denom, const float *grad_loss, int reduction,
                              float *grad, int64_t grad_ld) {
    const int64_t total = N * V;
    for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total; t += (int64_t)gridDim.x * blockDim.x) {
        const int64_t i = t / V, v = t % V;
        double c;
        if (reduction == 0) c = (double)grad_loss[i];
        else if (reduction == 1) c = (double)grad_loss[0] / (double)N;
        else c = (double)grad_loss[0];
        const float w = weight(ce_load<T>(x, ld, i, v), rowmax[i]);
        const double p = (double)w / denom[i];
        const double g = p - (v == targets[i] - v0 ? 1.0 : 0.0);
        grad[i * grad_ld + v] = (float)(g * c);
    }
}

// ---------------------------------------------------------------- bf16 pattern tables
//
// A bf16 logit is one of 2^16 bit patterns and its weight depends on nothing
// else in the row, so the exact sum over a row equals the exact sum over
// patterns of count(pattern) * w(pattern), and a gradient row is a lookup of
// g(pattern) (plus the target column).  The tables cover a window of 32
// binades of |x|, both signs (8192 patterns), placed per row from a sample of
// its values with four times headroom above the largest sampled magnitude;
// patterns outside the window take the per-element rules instead.  Both forms
// give the same bits: integer counts times exact f32 weights, summed exactly.

constexpr int kTT = 512;                   // threads of a row workgroup
constexpr int kHalf = 32 * 128;            // patterns per sign: 32 binades x 128 mantissas
constexpr int kTab = 2 * kHalf;            // table slots
constexpr int kSlots = kTab / kTT;         // slots per thread (16)
constexpr int kPipe = 4;                  // vectors per thread in flight while the previous ones are binned
constexpr int kQcap = 2048;                // out-of-window patterns kept per row
constexpr int64_t kTabMinLen = kTab;       // shorter ranges use the per-element kernels
constexpr int64_t kCountMax = (int64_t)1 << 29;  // count * w stays exact in binary64

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_value(uint32_t c) { return __uint_as_float(c << 16); }

// Slot of pattern c in the window starting at magnitude pattern `base`, or a
// value >= kTab when c lies outside it.  Slot bit 12 is the sign.
__device__ __forceinline__ uint32_t tab_slot(uint32_t c, uint32_t base) {
    const uint32_t a = (c & 0x7fffu) - base;
    return a < (uint32_t)kHalf ? (a | ((c >> 3) & 0x1000u)) : 0xffffffffu;
}
__device__ __forceinline__ uint32_t slot_code(uint32_t s, uint32_t base) {
    return ((s & (kHalf - 1)) + base) | ((s & kHalf) << 3);
}

// Split [v_lo, v_hi) of one row into a scalar head (up to the first 16-byte
// boundary), whole 16-byte vectors of 8 patterns, and a scalar tail.
struct RowSplit {
    int64_t head, nvec, tail0, len;
    __device__ RowSplit(const uint16_t *p0, int64_t len_) : len(len_) {
        head = min((int64_t)((((uintptr_t)0 - (uintptr_t)p0) & 15) >> 1), len);
        nvec = (len - head) >> 3;
        tail0 = head + nvec * 8;
    }
    // offset (from v_lo) of the j-th scalar element, j < nscalar()
    __device__ int64_t scalar_at(int64_t j) const { return j < head ? j : tail0 + (j - head); }
    __device__ int64_t nscalar() const { return head + (len - tail0); }
};

// Window base from each thread's largest sampled magnitude pattern: four
// times headroom above the workgroup's largest, 32 binades down.
__device__ __forceinline__ uint32_t window_of_sample_max(uint32_t mag, uint32_t *red) {
    const uint32_t top = block_max_key(mag, red) >> 7;  // exponent field of the largest sample
    const int lo = max(0, (int)top + 2 - 31);
    return (uint32_t)lo << 7;
}

// Window base for a row: the largest magnitude among the first vector of each
// thread (or its first scalar), reduced over the workgroup.
__device__ __forceinline__ uint32_t pick_window(const uint16_t *p0, const RowSplit &rs, uint32_t *red) {
    const int tid = threadIdx.x;
    uint32_t mag = 0;
    if (tid < rs.nvec) {
        const uint4 u = ((const uint4 *)(p0 + rs.head))[tid];
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) mag = max(mag, max(w[k] & 0x7fffu, (w[k] >> 16) & 0x7fffu));
    } else if (tid < rs.nscalar()) {
        mag = p0[rs.scalar_at(tid)] & 0x7fffu;
    }
    return window_of_sample_max(mag, red);
}

// The same placement from one vector per thread that every thread holds
// (rows with at least 8 vectors per thread).
__device__ __forceinline__ uint32_t window_from_sample(const uint4 u, uint32_t *red) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
    uint32_t mag = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) mag = max(mag, max(w[k] & 0x7fffu, (w[k] >> 16) & 0x7fffu));
    return window_of_sample_max(mag, red);
}

struct HistShared {
    uint32_t hist[kTab];
    uint16_t q[kQcap];
    int64_t sd[kTT / 64][kDenDigits];  // one digit set per wave (fewer lanes per LDS atomic address)
    uint32_t red[kTT / 64];
    uint32_t qn;
};

__device__ __forceinline__ void hist_put(HistShared &S, uint32_t c, uint32_t base) {
    const uint32_t s = tab_slot(c, base);
    if (s < (uint32_t)kTab) {
        atomicAdd(&S.hist[s], 1u);
    } else {
        const uint32_t pos = atomicAdd(&S.qn, 1u);
        if (pos < (uint32_t)kQcap) S.q[pos] = (uint16_t)c;
    }
}

// Eight patterns of one 16-byte vector.  Both patterns of a 32-bit word are
// placed at once in 16-bit lanes: a = (c & 0x7fff) - base modulo 2^16 is below
// kHalf exactly when the pattern lies in the window (a difference below zero
// wraps to 2^16 - 32767 or more), so one mask of the OR over the vector decides
// whether all eight are in it; then each lane's byte offset 4 slot =
// 4 a + (sign << 14) is below 2^15, so both fit their halves.
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void hist_put8(HistShared &S, const uint4 u, uint32_t base) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
    const u16x2 b2 = {(uint16_t)base, (uint16_t)base};
    uint32_t a[4], any = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        a[k] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, w[k] & 0x7fff7fffu) - b2);
        any |= a[k];
    }
    if ((any & 0xf000f000u) == 0) {
        const u16x2 two = {2, 2};
        char *h = (char *)S.hist;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t o = __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, a[k]) << two) |
                               ((w[k] >> 1) & 0x40004000u);
            atomicAdd((uint32_t *)(h + (o & 0xffffu)), 1u);
            atomicAdd((uint32_t *)(h + (o >> 16)), 1u);
        }
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            hist_put(S, w[k] & 0xffffu, base);
            hist_put(S, w[k] >> 16, base);
        }
    }
}

// Exact weight sum of one row range through the pattern histogram.  FWD: the
// range is the whole row, the row max comes from the histogram, and the loss,
// max and RN64(den) are written; otherwise the caller's max is used and the
// digits go to den[k*N + i] (added to what is there when add_into).
template <bool FWD>
__global__ __launch_bounds__(kTT, 6) void k_ce_hist(const uint16_t *x, int64_t N, int64_t ld, int64_t v_lo,
                                                    int64_t v_hi, const int64_t *targets, const float *rowmax_in,
                                                    float *loss, float *rowmax_out, double *denom, int64_t *den,
                                                    int add_into) {
    __shared__ HistShared S;
    const int tid = threadIdx.x, wave = tid >> 6;
    const int64_t i = blockIdx.x;
    const uint16_t *p0 = x + i * ld + v_lo;
    const RowSplit rs(p0, v_hi - v_lo);
    for (int k = tid; k < kTab / 4; k += kTT) ((uint4 *)S.hist)[k] = make_uint4(0u, 0u, 0u, 0u);
    if (tid < kDenDigits * (kTT / 64)) (&S.sd[0][0])[tid] = 0;
    if (tid == 0) S.qn = 0;

    // The first batch of loads is issued before the window is placed: the
    // window comes from each thread's first vector, which is that batch's
    // first element, so the placement waits for one load round trip that
    // the rest of the batch overlaps.
    // the target's column is read now and its logit once the window is
    // placed, so both round trips overlap the streaming (the value is used at
    // the very end)
    int64_t tcol = 0;
    if (FWD && tid == 0) tcol = targets[i];
    const uint4 *vp = (const uint4 *)(p0 + rs.head);
    int64_t k = tid;
    uint32_t base;
    if (8 * kTT <= rs.nvec) {  // (a workgroup-uniform test: both branches hold a barrier)
        uint4 u[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) u[j] = vp[k + j * kTT];
        base = window_from_sample(u[0], S.red);  // synchronizes
#pragma unroll
        for (int j = 0; j < 8; ++j) hist_put8(S, u[j], base);
        k += 8 * kTT;
    } else {
        base = pick_window(p0, rs, S.red);  // synchronizes
    }
    // (a target outside [0, V) reads no logit: the bf16 quiet NaN stands in)
    const bool tok = tcol >= 0 && tcol < v_hi - v_lo;
    uint32_t xraw = 0x7fc0u;
    if (FWD && tid == 0 && tok) xraw = x[i * ld + tcol];
    // software-pipelined: the next four vectors are in flight while the
    // current four are binned
    if (k + (kPipe - 1) * kTT < rs.nvec) {
        uint4 a[kPipe];
#pragma unroll
        for (int j = 0; j < kPipe; ++j) a[j] = vp[k + j * kTT];
        k += kPipe * kTT;
        for (; k + (kPipe - 1) * kTT < rs.nvec; k += kPipe * kTT) {
            uint4 b[kPipe];
#pragma unroll
            for (int j = 0; j < kPipe; ++j) b[j] = vp[k + j * kTT];
#pragma unroll
            for (int j = 0; j < kPipe; ++j) hist_put8(S, a[j], base);
#pragma unroll
            for (int j = 0; j < kPipe; ++j) a[j] = b[j];
        }
#pragma unroll
        for (int j = 0; j < kPipe; ++j) hist_put8(S, a[j], base);
    }
    for (; k < rs.nvec; k += kTT) hist_put8(S, vp[k], base);
    for (int64_t j = tid; j < rs.nscalar(); j += kTT) hist_put(S, p0[rs.scalar_at(j)], base);
    __syncthreads();

    const uint32_t qn = S.qn;
    const bool over = qn > (uint32_t)kQcap;  // some outside patterns were not kept: rescan for them
    // thread tid takes the runs of four slots 4 (tid + q kTT), q < kSlots / 4:
    // the patterns a row holds most of (a few binades) spread over four times
    // as many threads as whole runs of kSlots would, while each run's weights
    // stay close in exponent for the window
    uint32_t cnt[kSlots];
#pragma unroll
    for (int j = 0; j < kSlots / 4; ++j) {
        const uint4 c4 = ((const uint4 *)S.hist)[tid + kTT * j];
        cnt[4 * j] = c4.x;
        cnt[4 * j + 1] = c4.y;
        cnt[4 * j + 2] = c4.z;
        cnt[4 * j + 3] = c4.w;
    }
    auto slot_at = [&](int j) { return 4u * ((uint32_t)tid + (uint32_t)kTT * (uint32_t)(j >> 2)) + (uint32_t)(j & 3); };

    float m;
    if (FWD) {
        uint32_t key = kKeyNegInf;
#pragma unroll
        for (int j = 0; j < kSlots; ++j)
            if (cnt[j]) key = max(key, order_key(bf16_value(slot_code(slot_at(j), base))));
        if (!over) {
            for (uint32_t q = tid; q < qn; q += kTT) key = max(key, order_key(bf16_value(S.q[q])));
        } else {
            for (int64_t j = tid; j < rs.len; j += kTT) {
                const uint32_t c = p0[j];
                if (tab_slot(c, base) >= (uint32_t)kTab) key = max(key, order_key(bf16_value(c)));
            }
        }
        m = key_value(block_max_key(key, S.red));
    } else {
        m = rowmax_in[i];
    }

    int64_t *sd = S.sd[wave];
    Window win;
    win.init();
#pragma unroll
    for (int j = 0; j < kSlots; ++j) {
        if (cnt[j]) {
            const float w = weight(bf16_value(slot_code(slot_at(j), base)), m);
            if (w != 0.0f) {
                const double t = (double)w * (double)cnt[j];  // exact: 24 x 29 bits
                const int ew = f32_exp(w);
                win.add<kDenDigits>(t, max(ew, -126) - 23, f64_exp(t) + 1, kDenGcap, kDenElo, sd, 1);
            }
        }
    }
    auto add_one = [&](uint32_t c) {
        const float w = weight(bf16_value(c), m);
        if (w != 0.0f) {
            const int ew = f32_exp(w);
            win.add<kDenDigits>((double)w, max(ew, -126) - 23, ew + 1, kDenGcap, kDenElo, sd, 1);
        }
    };
    if (!over) {
        for (uint32_t q = tid; q < qn; q += kTT) add_one(S.q[q]);
    } else {
        for (int64_t j = tid; j < rs.len; j += kTT) {
            const uint32_t c = p0[j];
            if (tab_slot(c, base) >= (uint32_t)kTab) add_one(c);
        }
    }
    win.flush<kDenDigits>(kDenElo, sd, 1);
    __syncthreads();
    if (tid < kDenDigits) {  // the waves' digit sets, added as integers (any order gives the same sum)
        int64_t acc = 0;
        for (int w = 1; w < kTT / 64; ++w) acc += S.sd[w][tid];
        S.sd[0][tid] += acc;
    }
    __syncthreads();
    if (tid == 0) {
        int64_t d[kDenDigits];
#pragma unroll
        for (int q = 0; q < kDenDigits; ++q) d[q] = S.sd[0][q] + ((!FWD && add_into) ? den[q * N + i] : 0);
        canonicalize<kDenDigits>(d);
        if (FWD) {
            rowmax_out[i] = m;
            if (!tok) atomicAdd(&g_ce_bad_targets, 1u);
            ce_loss_of(d, bf16_value(xraw), m, i, loss, denom);
        } else {
#pragma unroll
            for (int q = 0; q < kDenDigits; ++q) den[q * N + i] = d[q];
        }
    }
}

// Row max of bf16 logits over [v_lo, v_hi): as signed 16-bit integers the
// non-negative patterns order like their values (+0 above -0) and the negative
// ones in reverse, so the max is the largest integer when it is >= 0 and the
// smallest integer otherwise.
__global__ __launch_bounds__(kTT) void k_ce_rowmax_bf16(const uint16_t *x, int64_t ld, int64_t v_lo, int64_t v_hi,
                                                        float *rowmax) {
    __shared__ uint32_t red[kTT / 64];
    const int tid = threadIdx.x;
    const int64_t i = blockIdx.x;
    const uint16_t *p0 = x + i * ld + v_lo;
    const RowSplit rs(p0, v_hi - v_lo);
    int hi = -32769, lo = 32768;
    const uint4 *vp = (const uint4 *)(p0 + rs.head);
    auto take = [&](uint32_t w) {
        const int a = (int)(int16_t)(w & 0xffffu), b = (int)(int16_t)(w >> 16);
        hi = max(hi, max(a, b));
        lo = min(lo, min(a, b));
    };
    int64_t k = tid;
    for (; k + 3 * kTT < rs.nvec; k += 4 * kTT) {
        const uint4 u0 = vp[k], u1 = vp[k + kTT], u2 = vp[k + 2 * kTT], u3 = vp[k + 3 * kTT];
        take(u0.x); take(u0.y); take(u0.z); take(u0.w);
        take(u1.x); take(u1.y); take(u1.z); take(u1.w);
        take(u2.x); take(u2.y); take(u2.z); take(u2.w);
        take(u3.x); take(u3.y); take(u3.z); take(u3.w);
    }
    for (; k < rs.nvec; k += kTT) {
        const uint4 u = vp[k];
        take(u.x); take(u.y); take(u.z); take(u.w);
    }
    for (int64_t j = tid; j < rs.nscalar(); j += kTT) {
        const int a = (int)(int16_t)p0[rs.scalar_at(j)];
        hi = max(hi, a);
        lo = min(lo, a);
    }
    // keys: order_key of the candidate values (an empty range keeps -inf)
    uint32_t key = kKeyNegInf;
    if (hi >= 0) key = order_key(bf16_value((uint32_t)hi));
    else if (lo <= 32767) key = order_key(bf16_value((uint32_t)(uint16_t)(int16_t)lo));
    const float m = key_value(block_max_key(key, red));
    if (tid == 0) rowmax[i] = m;
}

// g = RN32(RN64(RN64(w / den64) - [target]) * c)
__device__ __forceinline__ float grad_value(float x, float m, double d64, double c, bool target) {
    const double p = (double)weight(x, m) / d64;
    return (float)((p - (target ? 1.0 : 0.0)) * c);
}

__device__ __forceinline__ double grad_scale(const float *grad_loss, int reduction, int64_t N, int64_t i) {
    if (reduction == 0) return (double)grad_loss[i];
    if (reduction == 1) return (double)grad_loss[0] / (double)N;
    return (double)grad_loss[0];
}

// Gradient rows of bf16 logits: one workgroup per row builds g(pattern) for the
// window's 8192 patterns, then streams the row through the table.
__global__ __launch_bounds__(kTT) void k_ce_backward_tab(const uint16_t *x, int64_t N, int64_t V, int64_t ld,
                                                         int64_t v0, const int64_t *targets, const float *rowmax,
                                                         const double *denom, const float *grad_loss,
                                                         int reduction, float *grad, int64_t grad_ld) {
    __shared__ float tab[kTab];
    __shared__ uint32_t red[kTT / 64];
    const int tid = threadIdx.x;
    const int64_t i = blockIdx.x;
    const uint16_t *p0 = x + i * ld;
    float *o = grad + i * grad_ld;
    const RowSplit rs(p0, V);
    const float m = rowmax[i];
    const double d64 = denom[i];
    const double c = grad_scale(grad_loss, reduction, N, i);
    const int64_t t = targets[i] - v0;  // the target's column in this shard (outside [0, V): none)
    const uint32_t base = pick_window(p0, rs, red);
    for (int s = tid; s < kTab; s += kTT) tab[s] = grad_value(bf16_value(slot_code(s, base)), m, d64, c, false);
    __syncthreads();

    // Four patterns per lane and step: 8-byte loads and 16-byte stores, both
    // contiguous over the wave; the gradient is written with streaming stores.
    const bool vec_out = (((uintptr_t)(o + rs.head)) & 15) == 0;
    auto one = [&](uint32_t code, int64_t v) {
        const uint32_t s = tab_slot(code, base);
        if (s < (uint32_t)kTab && v != t) return tab[s];
        return grad_value(bf16_value(code), m, d64, c, v == t);
    };
    const uint2 *vp = (const uint2 *)(p0 + rs.head);
    const int64_t n4 = rs.nvec * 2;
    auto row4 = [&](const uint2 u, int64_t k) {
        const int64_t v0 = rs.head + 4 * k;
        const uint32_t w[2] = {u.x, u.y};
        float g[4];
        uint32_t s[4];
        bool slow = (uint64_t)(t - v0) < 4;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            s[2 * q] = tab_slot(w[q] & 0xffffu, base);
            s[2 * q + 1] = tab_slot(w[q] >> 16, base);
            slow |= (s[2 * q] | s[2 * q + 1]) >= (uint32_t)kTab;
        }
        if (!slow) {
#pragma unroll
            for (int q = 0; q < 4; ++q) g[q] = tab[s[q]];
        } else {
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                g[2 * q] = one(w[q] & 0xffffu, v0 + 2 * q);
                g[2 * q + 1] = one(w[q] >> 16, v0 + 2 * q + 1);
            }
        }
        if (vec_out) {
            __builtin_nontemporal_store(f32x4{g[0], g[1], g[2], g[3]}, (f32x4 *)(o + v0));
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) o[v0 + q] = g[q];
        }
    };
    int64_t k = tid;
    for (; k + 7 * kTT < n4; k += 8 * kTT) {
        uint2 u[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) u[j] = vp[k + j * kTT];
#pragma unroll
        for (int j = 0; j < 8; ++j) row4(u[j], k + j * kTT);
    }
    for (; k < n4; k += kTT) row4(vp[k], k);
    for (int64_t j = tid; j < rs.nscalar(); j += kTT) {
        const int64_t v = rs.scalar_at(j);
        o[v] = one(p0[v], v);
    }
}

// The pattern-table kernels need 2-byte aligned rows and pay off from a range of
// about a table's size; counts must stay below 2^29 for exact products.
static bool bf16_rows_ok(const void *x) { return ((uintptr_t)x & 1) == 0; }
static bool use_tables(int64_t len) { return len >= kTabMinLen && len < kCountMax; }

hipError_t launch_ce_rowmax(const void *x, int dtype, int64_t N, int64_t ld, int64_t v_lo, int64_t v_hi,
                            float *rowmax, hipStream_t s) {
    ProfScope prof_("ce_rowmax", s);
    if (N <= 0) return hipSuccess;
    if (dtype == 0)
        hipLaunchKernelGGL(k_ce_rowmax<float>, dim3((unsigned)N), dim3(kCeThreads), 0, s, x, ld, v_lo, v_hi, rowmax);
    else if (bf16_rows_ok(x))
        hipLaunchKernelGGL(k_ce_rowmax_bf16, dim3((unsigned)N), dim3(kTT), 0, s, (const uint16_t *)x, ld, v_lo, v_hi,
                           rowmax);
    else
        hipLaunchKernelGGL(k_ce_rowmax<bf16_t>, dim3((unsigned)N), dim3(kCeThreads), 0, s, x, ld, v_lo, v_hi,
                           rowmax);
    return hipGetLastError();
}

hipError_t launch_ce_denom(const void *x, int dtype, int64_t N, int64_t ld, const float *rowmax, int64_t v_lo,
                           int64_t v_hi, int64_t *den, int add_into, hipStream_t s) {
    ProfScope prof_("ce_denom", s);
    if (N <= 0) return hipSuccess;
    if (dtype == 0)
        hipLaunchKernelGGL(k_ce_denom<float>, dim3((unsigned)N), dim3(kCeThreads), 0, s, x, N, ld, rowmax, v_lo,
                           v_hi, den, add_into);
    else if (bf16_rows_ok(x) && use_tables(v_hi - v_lo))
        hipLaunchKernelGGL(k_ce_hist<false>, dim3((unsigned)N), dim3(kTT), 0, s, (const uint16_t *)x, N, ld, v_lo,
                           v_hi, nullptr, rowmax, nullptr, nullptr, nullptr, den, add_into);
    else
        hipLaunchKernelGGL(k_ce_denom<bf16_t>, dim3((unsigned)N), dim3(kCeThreads), 0, s, x, N, ld, rowmax, v_lo,
                           v_hi, den, add_into);
    return hipGetLastError();
}

hipError_t launch_ce_finalize(const int64_t *den, const void *x, int dtype, int64_t N, int64_t V, int64_t ld,
                              const int64_t *targets, const float *rowmax, float *loss, double *denom,
                              hipStream_t s) {
    ProfScope prof_("ce_finalize", s);
    if (N <= 0) return hipSuccess;
    if (dtype == 0)
        hipLaunchKernelGGL(k_ce_finalize<float>, ce_grid(N), dim3(256), 0, s, den, x, N, V, ld, targets, rowmax,
                           loss, denom);
    else
        hipLaunchKernelGGL(k_ce_finalize<bf16_t>, ce_grid(N), dim3(256), 0, s, den, x, N, V, ld, targets, rowmax,
                           loss, denom);
    return hipGetLastError();
}

hipError_t launch_ce_forward(const void *x, int dtype, int64_t N, int64_t V, int64_t ld, const int64_t *targets,
                             float *loss, float *rowmax, double *denom, hipStream_t s) {
    ProfScope prof_("ce_forward", s);
    if (N <= 0) return hipSuccess;
    if (dtype == 0)
        hipLaunchKernelGGL(k_ce_forward<float>, dim3((unsigned)N), dim3(kCeThreads), 0, s, x, V, ld, targets, loss,
                           rowmax, denom);
    else if (bf16_rows_ok(x) && use_tables(V))
        hipLaunchKernelGGL(k_ce_hist<true>, dim3((unsigned)N), dim3(kTT), 0, s, (const uint16_t *)x, N, ld, (int64_t)0,
                           V, targets, nullptr, loss, rowmax, denom, nullptr, 0);
    else
        hipLaunchKernelGGL(k_ce_forward<bf16_t>, dim3((unsigned)N), dim3(kCeThreads), 0, s, x, V, ld, targets,
                           loss, rowmax, denom);
    return hipGetLastError();
}

hipError_t launch_ce_reduce(const float *loss, int64_t N, int reduction, float *out, int64_t *, hipStream_t s) {
    ProfScope prof_("ce_reduce", s);
    hipLaunchKernelGGL(k_ce_reduce, dim3(1), dim3(1024), 0, s, loss, N, reduction, out);
    return hipGetLastError();
}

hipError_t launch_ce_backward(const void *x, int dtype, int64_t N, int64_t V, int64_t ld, int64_t v0,
                              const int64_t *targets, const float *rowmax, const double *denom,
                              const float *grad_loss, int reduction, float *grad, int64_t grad_ld, hipStream_t s) {
    ProfScope prof_("ce_backward", s);
    if (N * V <= 0) return hipSuccess;
    if (dtype == 0)
        hipLaunchKernelGGL(k_ce_backward<float>, ce_grid(N * V), dim3(256), 0, s, x, N, V, ld, v0, targets, rowmax,
                           denom, grad_loss, reduction, grad, grad_ld);
    else if (bf16_rows_ok(x) && use_tables(V))
        hipLaunchKernelGGL(k_ce_backward_tab, dim3((unsigned)N), dim3(kTT), 0, s, (const uint16_t *)x, N, V, ld,
                           v0, targets, rowmax, denom, grad_loss, reduction, grad, grad_ld);
    else
        hipLaunchKernelGGL(k_ce_backward<bf16_t>, ce_grid(N * V), dim3(256), 0, s, x, N, V, ld, v0, targets, rowmax,
                           denom, grad_loss, reduction, grad, grad_ld);
    return hipGetLastError();
}

}  // namespace det

namespace det {

// The count of rows given a target outside [0, V) since the last call, then
// cleared (waits for the stream first).
hipError_t ce_take_bad_targets(hipStream_t s, unsigned int *count) {
    hipError_t e;
    if ((e = hipStreamSynchronize(s)) != hipSuccess) return e;
    if ((e = hipMemcpyFromSymbol(count, HIP_SYMBOL(g_ce_bad_targets), sizeof(unsigned int), 0,
                                 hipMemcpyDeviceToHost)) != hipSuccess)
        return e;
    const unsigned int zero = 0;
    return hipMemcpyToSymbol(HIP_SYMBOL(g_ce_bad_targets), &zero, sizeof(zero), 0, hipMemcpyHostToDevice);
}

}  // namespace det
