// bwd.hip -- gradients of the exact two-pass attention.
//
// No page gives a backward rule; the one computed here keeps every sum over
// the sequence axes exact, as the forward's sums are (det-attn page,
// "Method": order-invariant reductions, so any sharding of queries or keys
// gives the same bits).  Per row and pair:
//
//   delta_i = fp64 fma chain over d of dO_id * O_id
//   dp_ij   = fp64 fma chain over d of dO_id * V_jd
//   p_ij    = RN32(RN64(w_ij / den64_i)),  w and den64 as in the forward
//   ds_ij   = RN32(RN64(p_ij * RN64(dp_ij - delta_i)))
//
// and the three gradients are exact sums of f32 x f32 products (each exact in
// binary64, a multiple of 2^-298 below 2^256), rounded once:
//
//   dV_jd = RN32(RN64(sum p_ij dO_id)),  dK_jd = RN32(RN64(scale RN64(sum ds_ij Q_id))),
//   dQ_id = RN32(RN64(scale RN64(sum ds_ij K_jd)))
//
// The sums are kept as 18 radix-2^32 digits from 2^-298: a workgroup owns a
// 16 x 16 tile of outputs, each thread one output, whose digits live in LDS;
// every product is split into three 32-bit limbs added to the digits it
// spans (no carries until the end: 2^30 limbs of at most 2^32 stay below
// 2^62), so the result does not depend on the order of the terms.
#include "dev_math.hpp"
#include "kernels.hpp"

namespace det {

constexpr int kBT = 16;         // rows (or keys) and columns of a tile
constexpr int kBStep = 32;      // reduction steps staged per barrier

struct BwdArgs {
    const void *q, *k, *v;
    int64_t qsB, qsH, qsS, ksB, ksH, ksS, vsB, vsH, vsS;
    const float *o, *dout;
    int64_t osB, osH, osS, dsB, dsH, dsS;
    const float *rowmax;
    const double *den64;
    double *delta;  // [bh * Sq + i]
    int64_t Hq, Hkv, group, Sq, Skv, D;
    int causal;
    double scale;
    // query-row chunk [i0, i0 + ni)
    int64_t i0, ni, nbh;
    float *P, *DS;                      // [bh][ni][Skv]
    int64_t *dq_dig;                    // [kBwdDigits][nbh * ni][D]
    int64_t *dk_dig, *dv_dig;           // [kBwdDigits][B * Hkv * Skv][D]
};

template <typename T>
__device__ __forceinline__ float ld(const void *base, int64_t off) {
    return elem<T>::to_f32(((const T *)base)[off]);
}

// delta_i, one thread per row.
__global__ __launch_bounds__(256) void k_bwd_delta(BwdArgs A, int64_t rows) {
    const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= rows) return;
    const int64_t b = r / (A.Hq * A.Sq), hq = (r / A.Sq) % A.Hq, i = r % A.Sq;
    const float *o = A.o + b * A.osB + hq * A.osH + i * A.osS;
    const float *g = A.dout + b * A.dsB + hq * A.dsH + i * A.dsS;
    double acc = 0.0;
    for (int64_t d = 0; d < A.D; ++d) acc = fma((double)g[d], (double)o[d], acc);
    A.delta[r] = acc;
}

// p and ds of a 16 x 16 tile of pairs (rows of the chunk x keys): the 16 rows
// of Q and dO and the 16 rows of K and V staged in LDS as f32 (exact), then
// one thread per pair runs the two chains.  Tiles wholly above the causal
// diagonal are skipped (the sums never read them); invisible pairs of the
// other tiles get p = ds = 0.  Grid (key tiles, row tiles, heads).
template <typename T>
__global__ __launch_bounds__(256) void k_bwd_pds(BwdArgs A) {
    __shared__ float sq[kBT][257], sk[kBT][257], sg[kBT][257], sv[kBT][257];
    const int tid = threadIdx.x, r = tid >> 4, c = tid & 15;
    const int64_t kb = blockIdx.x, tile = blockIdx.y, bh = blockIdx.z;
    const int64_t b = bh / A.Hq, hq = bh % A.Hq, hk = hq / A.group;
    const int64_t ia = A.i0 + tile * kBT, ja = kb * kBT, iend = A.i0 + A.ni;
    const int64_t ilast = min64(iend, ia + kBT) - 1;
    if (A.causal && ja > ilast) return;
    for (int64_t d = tid; d < A.D; d += 256) {
#pragma unroll 4
        for (int rr = 0; rr < kBT; ++rr) {
            const int64_t iq = min64(ia + rr, iend - 1), jk = min64(ja + rr, A.Skv - 1);  // clamped: in range
            sq[rr][d] = ld<T>(A.q, b * A.qsB + hq * A.qsH + iq * A.qsS + d);
            sg[rr][d] = A.dout[b * A.dsB + hq * A.dsH + iq * A.dsS + d];
            sk[rr][d] = ld<T>(A.k, b * A.ksB + hk * A.ksH + jk * A.ksS + d);
            sv[rr][d] = ld<T>(A.v, b * A.vsB + hk * A.vsH + jk * A.vsS + d);
        }
    }
    __syncthreads();
    const int64_t i = ia + r, j = ja + c;
    if (i >= iend || j >= A.Skv) return;
    const int64_t row = bh * A.Sq + i;
    float p = 0.0f, ds = 0.0f;
    if (!A.causal || j <= i) {
        const int D = (int)A.D;
        double acc = 0.0;
        for (int d = 0; d < D; ++d) acc = fma((double)sq[r][d], (double)sk[c][d], acc);
        const float s = (float)(A.scale * acc);
        const float w = weight(s, A.rowmax[row]);
        p = (float)((double)w / A.den64[row]);
        double dp = 0.0;
        for (int d = 0; d < D; ++d) dp = fma((double)sg[r][d], (double)sv[c][d], dp);
        ds = (float)((double)p * (dp - A.delta[row]));
    }
    const int64_t at = (bh * A.ni + (i - A.i0)) * A.Skv + j;
    A.P[at] = p;
    A.DS[at] = ds;
}

// Adds the exact product of the f32 values with bit patterns ua and ub into
// the calling thread's digits.  The product is m 2^s with m = ma mb < 2^48
// (the significands) and s = ea + eb - 2 counted from 2^-298 (ea, eb the
// biased exponents, 1 for subnormals); its three 32-bit limbs go to digits
// s/32 .. s/32 + 2 by LDS atomic adds, which need no result and so do not
// wait on one another (the digits are the thread's own: no contention).
__device__ __forceinline__ void bwd_term(uint32_t ua, uint32_t ub, int64_t (*dig)[256], int tid) {
    const uint32_t ea = (ua >> 23) & 0xffu, eb = (ub >> 23) & 0xffu;
    const uint64_t ma = (ua & 0x7fffffu) | (ea ? 0x800000u : 0u), mb = (ub & 0x7fffffu) | (eb ? 0x800000u : 0u);
    const uint64_t m = ma * mb;
    if (m == 0) return;
    const int s = (int)max(ea, 1u) + (int)max(eb, 1u) - 2;
    // s <= 506 for finite values: k0 + 2 <= 17 (the clamp keeps inf / nan in the array)
    const int k0 = min(s >> 5, kBwdDigits - 3), sh = s & 31;
    const uint64_t lo = m << sh;            // bits 0..63 of m 2^sh (m 2^sh < 2^79)
    const uint64_t hi = m >> (32 - sh) >> 32;  // bits 64..78
    const bool neg = ((ua ^ ub) >> 31) != 0;
    int64_t c0 = (int64_t)(lo & 0xffffffffull), c1 = (int64_t)(lo >> 32), c2 = (int64_t)hi;
    if (neg) {
        c0 = -c0;
        c1 = -c1;
        c2 = -c2;
    }
    unsigned long long *d = (unsigned long long *)&dig[k0][tid];
    atomicAdd(d, (unsigned long long)c0);
    atomicAdd(d + 256, (unsigned long long)c1);
    if (c2) atomicAdd(d + 512, (unsigned long long)c2);
}

// Exact sums for a 16 x 16 tile of outputs, one thread per output.
//   MODE 0 (dQ): rows = chunk rows i of head bh, terms ds_ij K_jd over keys j
//   MODE 1 (dK): rows = keys j of key head bhk, terms ds_ij Q_id over (query head, row)
//   MODE 2 (dV): the same with p_ij dO_id
// Grid (column tiles, row tiles, heads).  Per step 32 terms of the tile's
// rows and columns are staged in LDS.
template <int MODE, typename T>
__global__ __launch_bounds__(256) void k_bwd_sum(BwdArgs A) {
    __shared__ int64_t dig[kBwdDigits][256];
    __shared__ float sa[kBT][kBStep + 1], sb[kBStep][kBT + 1];
    const int tid = threadIdx.x, r = tid >> 4, c = tid & 15;
    const int64_t da = (int64_t)blockIdx.x * kBT, ra = (int64_t)blockIdx.y * kBT, hh = blockIdx.z;
#pragma unroll
    for (int k = 0; k < kBwdDigits; ++k) dig[k][tid] = 0;
    const int64_t iend = A.i0 + A.ni;
    if (MODE == 0) {
        const int64_t bh = hh, b = bh / A.Hq, hk = (bh % A.Hq) / A.group;
        const int64_t ia = A.i0 + ra, ilast = min64(iend, ia + kBT) - 1;
        const int64_t jend = A.causal ? min64(A.Skv, ilast + 1) : A.Skv;
        for (int64_t t0 = 0; t0 < jend; t0 += kBStep) {
            __syncthreads();
            for (int e = tid; e < kBT * kBStep; e += 256) {
                const int rr = e / kBStep, tt = e % kBStep;
                const int64_t i = ia + rr, j = t0 + tt;
                sa[rr][tt] = (i < iend && j < jend) ? A.DS[(bh * A.ni + (i - A.i0)) * A.Skv + j] : 0.0f;
                const int cc = e % kBT, st = e / kBT;
                const int64_t jj = t0 + st, d = da + cc;
                sb[st][cc] = (jj < jend && d < A.D) ? ld<T>(A.k, b * A.ksB + hk * A.ksH + jj * A.ksS + d) : 0.0f;
            }
            __syncthreads();
#pragma unroll 4
            for (int tt = 0; tt < kBStep; ++tt)
                bwd_term(__float_as_uint(sa[r][tt]), __float_as_uint(sb[tt][c]), dig, tid);
        }
        const int64_t i = ia + r, d = da + c;
        if (i < iend && d < A.D) {
            const int64_t plane = A.nbh * A.ni * A.D, at = (bh * A.ni + (i - A.i0)) * A.D + d;
#pragma unroll
            for (int k = 0; k < kBwdDigits; ++k) A.dq_dig[k * plane + at] = dig[k][tid];
        }
        return;
    }
    const int64_t bhk = hh, b = bhk / A.Hkv, hk = bhk % A.Hkv;
    const int64_t ja = ra;
    const float *X = MODE == 1 ? A.DS : A.P;
    const int64_t istart = A.causal ? max64(A.i0, ja) : A.i0;
    for (int64_t g = 0; g < A.group; ++g) {
        const int64_t hq = hk * A.group + g, bh = b * A.Hq + hq;
        for (int64_t t0 = istart; t0 < iend; t0 += kBStep) {
            __syncthreads();
            for (int e = tid; e < kBT * kBStep; e += 256) {
                const int rr = e % kBT, tt = e / kBT;  // 16 consecutive keys of one query row
                const int64_t j = ja + rr, i = t0 + tt;
                sa[rr][tt] = (i < iend && j < A.Skv) ? X[(bh * A.ni + (i - A.i0)) * A.Skv + j] : 0.0f;
                const int cc = e % kBT;
                const int64_t d = da + cc;
                float x = 0.0f;
                if (i < iend && d < A.D) {
                    if (MODE == 1) x = ld<T>(A.q, b * A.qsB + hq * A.qsH + i * A.qsS + d);
                    else x = A.dout[b * A.dsB + hq * A.dsH + i * A.dsS + d];
                }
                sb[tt][cc] = x;
            }
            __syncthreads();
#pragma unroll 4
            for (int tt = 0; tt < kBStep; ++tt)
                bwd_term(__float_as_uint(sa[r][tt]), __float_as_uint(sb[tt][c]), dig, tid);
        }
    }
    const int64_t j = ja + r, d = da + c;
    if (j < A.Skv && d < A.D) {
        int64_t *out = MODE == 1 ? A.dk_dig : A.dv_dig;
        const int64_t plane = A.nbh / A.group * A.Skv * A.D, at = (bhk * A.Skv + j) * A.D + d;
#pragma unroll
        for (int k = 0; k < kBwdDigits; ++k) out[k * plane + at] += dig[k][tid];  // chunks run in stream order
    }
}

// out = RN32(RN64(f * RN64(X))) of each digit sum X (f = scale or 1); row R
// of the planes is (head, s) = (R / S, R % S) of the output view.
__global__ __launch_bounds__(256) void k_bwd_finalize(const int64_t *dig, int64_t rows, int64_t D, int64_t S,
                                                      int64_t s_off, int64_t H, double f, OutView o) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= rows * D) return;
    const int64_t R = t / D, d = t % D;
    int64_t x[kBwdDigits];
#pragma unroll
    for (int k = 0; k < kBwdDigits; ++k) x[k] = dig[k * rows * D + t];
    canonicalize<kBwdDigits>(x);
    const double v = digits_to_f64<kBwdDigits>(x, kBwdElo);
    const int64_t head = R / S, s = s_off + R % S;
    o.data[(head / H) * o.sB + (head % H) * o.sH + s * o.sS + d] = (float)(f * v);
}

__global__ __launch_bounds__(256) void k_bwd_zero(OutView o, int64_t H, int64_t S, int64_t D, int64_t n) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= n) return;
    const int64_t d = t % D, s = (t / D) % S, h = (t / (D * S)) % H, b = t / (D * S * H);
    o.data[b * o.sB + h * o.sH + s * o.sS + d] = 0.0f;
}

// ---------------------------------------------------------------- launchers

static unsigned blocks_of(int64_t n) { return (unsigned)((n + 255) / 256); }

size_t bwd_fixed_bytes(const AttnGeom &g) {
    return align256((size_t)g.B * g.Hq * g.Sq * 8) + 2 * align256((size_t)kBwdDigits * g.B * g.Hkv * g.Skv * g.D * 8);
}

size_t bwd_chunk_bytes(const AttnGeom &g, int64_t ni) {
    const int64_t bh = g.B * g.Hq;
    return 2 * align256((size_t)bh * ni * g.Skv * 4) + align256((size_t)kBwdDigits * bh * ni * g.D * 8);
}

hipError_t launch_zero_view(const OutView &o, int64_t B, int64_t H, int64_t S, int64_t D, hipStream_t s) {
    const int64_t n = B * H * S * D;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_bwd_zero, dim3(blocks_of(n)), dim3(256), 0, s, o, H, S, D, n);
    return hipGetLastError();
}

hipError_t launch_attn_backward(const Tensor &q, const Tensor &k, const Tensor &v, const Tensor &o,
                                const Tensor &dout, const float *rowmax, const double *den64, const AttnGeom &g,
                                void *fixed_ws, void *chunk_ws, int64_t chunk, const OutView &dq,
                                const OutView &dk, const OutView &dv, hipStream_t s) {
    const int64_t bh = g.B * g.Hq, bhk = g.B * g.Hkv, rows = bh * g.Sq;
    if (bh > 65535 || bhk > 65535 || (chunk + kBT - 1) / kBT > 65535 || (g.Skv + kBT - 1) / kBT > 65535)
        return hipErrorInvalidValue;  // grid y / z limits
    BwdArgs A{};
    A.q = q.data;
    A.k = k.data;
    A.v = v.data;
    A.qsB = q.sB; A.qsH = q.sH; A.qsS = q.sS;
    A.ksB = k.sB; A.ksH = k.sH; A.ksS = k.sS;
    A.vsB = v.sB; A.vsH = v.sH; A.vsS = v.sS;
    A.o = (const float *)o.data;
    A.osB = o.sB; A.osH = o.sH; A.osS = o.sS;
    A.dout = (const float *)dout.data;
    A.dsB = dout.sB; A.dsH = dout.sH; A.dsS = dout.sS;
    A.rowmax = rowmax;
    A.den64 = den64;
    A.Hq = g.Hq;
    A.Hkv = g.Hkv;
    A.group = g.Hq / g.Hkv;
    A.Sq = g.Sq;
    A.Skv = g.Skv;
    A.D = g.D;
    A.causal = g.causal;
    A.scale = g.scale;
    A.nbh = bh;
    char *f = (char *)fixed_ws;
    A.delta = (double *)f;
    f += align256((size_t)rows * 8);
    const size_t kvdig = align256((size_t)kBwdDigits * bhk * g.Skv * g.D * 8);
    A.dk_dig = (int64_t *)f;
    A.dv_dig = (int64_t *)(f + kvdig);
    char *c = (char *)chunk_ws;
    A.P = (float *)c;
    A.DS = (float *)(c + align256((size_t)bh * chunk * g.Skv * 4));
    A.dq_dig = (int64_t *)(c + 2 * align256((size_t)bh * chunk * g.Skv * 4));
    hipError_t e;
    const int64_t kvn = kBwdDigits * bhk * g.Skv * g.D;
    if ((e = launch_fill_i64(A.dk_dig, kvn, 0, s)) != hipSuccess) return e;
    if ((e = launch_fill_i64(A.dv_dig, kvn, 0, s)) != hipSuccess) return e;
    {
        ProfScope prof_("bwd_delta", s);
        hipLaunchKernelGGL(k_bwd_delta, dim3(blocks_of(rows)), dim3(256), 0, s, A, rows);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const bool bf = q.dtype == 1;
    const dim3 cols((unsigned)((g.D + kBT - 1) / kBT));
    for (int64_t i0 = 0; i0 < g.Sq; i0 += chunk) {
        A.i0 = i0;
        A.ni = std::min(chunk, g.Sq - i0);
        const int64_t rt = (A.ni + kBT - 1) / kBT;
        {
            ProfScope prof_("bwd_pds", s);
            dim3 grid((unsigned)((g.Skv + kBT - 1) / kBT), (unsigned)rt, (unsigned)bh);
            if (bf) hipLaunchKernelGGL(k_bwd_pds<bf16_t>, grid, dim3(256), 0, s, A);
            else hipLaunchKernelGGL(k_bwd_pds<float>, grid, dim3(256), 0, s, A);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        {
            ProfScope prof_("bwd_sum", s);
            dim3 gq(cols.x, (unsigned)rt, (unsigned)bh), gk(cols.x, (unsigned)((g.Skv + kBT - 1) / kBT), (unsigned)bhk);
            if (bf) {
                hipLaunchKernelGGL((k_bwd_sum<0, bf16_t>), gq, dim3(256), 0, s, A);
                hipLaunchKernelGGL((k_bwd_sum<1, bf16_t>), gk, dim3(256), 0, s, A);
                hipLaunchKernelGGL((k_bwd_sum<2, bf16_t>), gk, dim3(256), 0, s, A);
            } else {
                hipLaunchKernelGGL((k_bwd_sum<0, float>), gq, dim3(256), 0, s, A);
                hipLaunchKernelGGL((k_bwd_sum<1, float>), gk, dim3(256), 0, s, A);
                hipLaunchKernelGGL((k_bwd_sum<2, float>), gk, dim3(256), 0, s, A);
            }
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        {
            ProfScope prof_("bwd_finalize", s);
            const int64_t n = bh * A.ni;  // rows (head, i) of the chunk, i from i0
            hipLaunchKernelGGL(k_bwd_finalize, dim3(blocks_of(n * g.D)), dim3(256), 0, s, A.dq_dig, n, g.D, A.ni,
                               i0, g.Hq, g.scale, dq);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
    }
    ProfScope prof_("bwd_finalize", s);
    const int64_t nk = bhk * g.Skv;
    hipLaunchKernelGGL(k_bwd_finalize, dim3(blocks_of(nk * g.D)), dim3(256), 0, s, A.dk_dig, nk, g.D, g.Skv,
                       (int64_t)0, g.Hkv, g.scale, dk);
    hipLaunchKernelGGL(k_bwd_finalize, dim3(blocks_of(nk * g.D)), dim3(256), 0, s, A.dv_dig, nk, g.D, g.Skv,
                       (int64_t)0, g.Hkv, 1.0, dv);
    return hipGetLastError();
}

}  // namespace det
