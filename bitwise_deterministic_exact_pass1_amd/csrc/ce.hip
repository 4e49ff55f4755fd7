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

static dim3 ce_grid(int64_t n) {
    return dim3((unsigned)std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, 1 << 20)));
}

template <typename T>
__device__ __forceinline__ float ce_load(const void *x, int64_t ld, int64_t i, int64_t v) {
    return elem<T>::to_f32(((const T *)x)[i * ld + v]);
}

// Block-wide max of order keys; every thread gets the result.
__device__ __forceinline__ uint32_t block_max_key(uint32_t k, uint32_t *sh) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) k = max(k, (uint32_t)__shfl_xor((int)k, off, 64));
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) sh[wave] = k;
    __syncthreads();
    uint32_t r = sh[0];
    for (int w = 1; w < kCeThreads / 64; ++w) r = max(r, sh[w]);
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
                                        int64_t t, float m, float *loss, double *denom) {
    const double d64 = digits_to_f64<kDenDigits>(dd, kDenElo);
    const double lse = (double)m + log_det(d64);
    loss[i] = (float)(lse - (double)ce_load<T>(x, ld, i, t));
    denom[i] = d64;
}

template <typename T>
__global__ void k_ce_finalize(const int64_t *den, const void *x, int64_t N, int64_t ld, const int64_t *targets,
                              const float *rowmax, float *loss, double *denom) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < N; i += (int64_t)gridDim.x * blockDim.x) {
        int64_t d[kDenDigits];
#pragma unroll
        for (int k = 0; k < kDenDigits; ++k) d[k] = den[k * N + i];
        canonicalize<kDenDigits>(d);
        ce_loss<T>(d, x, ld, i, targets[i], rowmax[i], loss, denom);
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
        ce_loss<T>(d, x, ld, i, targets[i], m, loss, denom);
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
__global__ void k_ce_backward(const void *x, int64_t N, int64_t V, int64_t ld, const int64_t *targets,
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
        const double g = p - (v == targets[i] ? 1.0 : 0.0);
        grad[i * grad_ld + v] = (float)(g * c);
    }
}

hipError_t launch_ce_rowmax(const void *x, int dtype, int64_t N, int64_t ld, int64_t v_lo, int64_t v_hi,
                            float *rowmax, hipStream_t s) {
    ProfScope prof_("ce_rowmax", s);
    if (N <= 0) return hipSuccess;
    if (dtype == 0)
        hipLaunchKernelGGL(k_ce_rowmax<float>, dim3((unsigned)N), dim3(kCeThreads), 0, s, x, ld, v_lo, v_hi, rowmax);
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
    else
        hipLaunchKernelGGL(k_ce_denom<bf16_t>, dim3((unsigned)N), dim3(kCeThreads), 0, s, x, N, ld, rowmax, v_lo,
                           v_hi, den, add_into);
    return hipGetLastError();
}

hipError_t launch_ce_finalize(const int64_t *den, const void *x, int dtype, int64_t N, int64_t ld,
                              const int64_t *targets, const float *rowmax, float *loss, double *denom,
                              hipStream_t s) {
    ProfScope prof_("ce_finalize", s);
    if (N <= 0) return hipSuccess;
    if (dtype == 0)
        hipLaunchKernelGGL(k_ce_finalize<float>, ce_grid(N), dim3(256), 0, s, den, x, N, ld, targets, rowmax, loss,
                           denom);
    else
        hipLaunchKernelGGL(k_ce_finalize<bf16_t>, ce_grid(N), dim3(256), 0, s, den, x, N, ld, targets, rowmax,
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

hipError_t launch_ce_backward(const void *x, int dtype, int64_t N, int64_t V, int64_t ld, const int64_t *targets,
                              const float *rowmax, const double *denom, const float *grad_loss, int reduction,
                              float *grad, int64_t grad_ld, hipStream_t s) {
    ProfScope prof_("ce_backward", s);
    if (N * V <= 0) return hipSuccess;
    if (dtype == 0)
        hipLaunchKernelGGL(k_ce_backward<float>, ce_grid(N * V), dim3(256), 0, s, x, N, V, ld, targets, rowmax,
                           denom, grad_loss, reduction, grad, grad_ld);
    else
        hipLaunchKernelGGL(k_ce_backward<bf16_t>, ce_grid(N * V), dim3(256), 0, s, x, N, V, ld, targets, rowmax,
                           denom, grad_loss, reduction, grad, grad_ld);
    return hipGetLastError();
}

}  // namespace det
