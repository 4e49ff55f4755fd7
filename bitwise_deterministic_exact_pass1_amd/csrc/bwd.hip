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
// The sums run on the int8 matrix cores where an exactness argument holds
// (k_bwd_colstats, k_bwd_slice, k_bwd_mma below: integer grids, balanced
// base-256 digits, exact int32 class sums).  An output tile outside it takes
// the per-term digit sums (k_bwd_sum): 18 radix-2^32 digits from 2^-298 per
// output, each f32 x f32 product split into three 32-bit limbs added to the
// digits it spans (no carries until the end: 2^30 limbs of at most 2^32 stay
// below 2^62).  Both give the same bits, whatever the order of the terms.
// dK and dV sums of all tiles end in digit planes (k_bwd_finalize rounds
// them); dQ tiles own every key and are rounded where they are summed.
#include "dev_math.hpp"
#include "kernels.hpp"

namespace det {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kBT = 16;         // rows (or keys) and columns of a tile
constexpr int kBStep = 32;      // reduction steps staged per barrier
constexpr int kXA = 10;         // matrix-core sums: A digits at most (an 80-bit row span)
constexpr int kXB = 7;          // B digits at most
constexpr int kXC = 13;         // digit classes s = a + b; a tile needs na + nb <= kXC + 1
constexpr int64_t kXMaxT = (int64_t)1 << 17;  // reduction length bound of the int32 class sums

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
    int64_t *dk_dig, *dv_dig;           // [kBwdDigits][B * Hkv * Skv][D]
    // matrix-core sums of the chunk.  Statistics {largest exponent, smallest
    // lsb exponent} of the nonzero entries: of each ds row over keys, of each
    // ds / p column over (query head, row), of each column of K over keys and
    // of Q / dO over (query head, row) (these three with the exponent of each
    // entry's lowest set bit as its lsb).
    int2 *st_rds, *st_cds, *st_cp, *st_k, *st_q, *st_o;
    v4i *xb[3];           // digit blocks of the right operands of dQ, dK, dV (K, Q, dO)
    int *xf[3];           // per (row tile, column group): 1 = left to k_bwd_sum
    int64_t nIB, nJB, nG;          // 32-row tiles, 32-key tiles, 32-column groups (flags, per-term sums)
    int64_t nIB64, nJB64, nG16;    // 64-step blocks and 16-column groups of the matrix-core sums
    int force_fallback;
    OutView dq;
};

constexpr int64_t kStatEmpty = (int64_t)0x7fffffff80000000ll;  // int2 {INT_MIN, INT_MAX}

// Exponent statistics of one f32 value: its exponent and its lsb exponent
// (subnormals: -127 and -149); a zero is empty.
__device__ __forceinline__ void stat_of(float x, int &emax, int &lmin) {
    const int e = f32_exp(x);
    emax = x != 0.0f ? e : INT_MIN;
    lmin = x != 0.0f ? max(e, -126) - 23 : INT_MAX;
}

// The same with the exponent of the lowest set bit as lsb exponent: a value
// whose significand ends in c zero bits sits on a grid 2^c times coarser (a
// bf16 value widened to f32 ends in at least 16).  Used for the right
// operands, whose digits are made with shifts both ways (k_bwd_slice).
__device__ __forceinline__ void stat_of_exact(float x, int &emax, int &lmin) {
    const uint32_t bits = __float_as_uint(x), be = (bits >> 23) & 0xffu;
    const uint32_t m = (bits & 0x7fffffu) | (be ? 0x800000u : 0u);
    emax = m ? (int)be - 127 : INT_MIN;
    lmin = m ? (int)(be ? be : 1u) - 150 + __builtin_ctz(m) : INT_MAX;
}

// Grid exponent g and balanced base-256 digit count n of a row (or column)
// with statistics st: every entry is an integer multiple of 2^g, |entry| <
// 2^(emax + 1), so |entry 2^-g| < 2^(8n - 2) holds n balanced digits.
__device__ __forceinline__ void grid_of(int2 st, int &g, int &n) {
    g = st.x == INT_MIN ? 0 : st.y;
    n = st.x == INT_MIN ? 0 : (st.x + 1 - st.y + 2 + 7) >> 3;
}

__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) v = max(v, __shfl_xor(v, off, 64));
    return v;
}

template <typename T>
__device__ __forceinline__ float ld(const void *base, int64_t off) {
    return elem<T>::to_f32(((const T *)base)[off]);
}

// delta_i of 16 rows per 64-thread block: the rows of dO and O are read
// into LDS by all lanes along d (coalesced), then lanes 0..15 each run one
// row's chain over d from LDS (the row stride D + 1 keeps the 16 rows on
// distinct banks).  D <= 256.
constexpr int kDeltaRows = 16;
__global__ __launch_bounds__(64) void k_bwd_delta(BwdArgs A, int64_t rows) {
    __shared__ float sg[kDeltaRows * 257 + 1], so[kDeltaRows * 257 + 1];  // + a slot for unused lanes
    const int tid = threadIdx.x, D = (int)A.D;
    const int64_t r0 = (int64_t)blockIdx.x * kDeltaRows;
    const int nr = (int)min64(kDeltaRows, rows - r0);
    int64_t gb = 0, ob = 0;  // lane l < nr: offsets of row r0 + l
    if (tid < nr) {
        const int64_t r = r0 + tid, b = r / (A.Hq * A.Sq), hq = (r / A.Sq) % A.Hq, i = r % A.Sq;
        gb = b * A.dsB + hq * A.dsH + i * A.dsS;
        ob = b * A.osB + hq * A.osH + i * A.osS;
    }
#pragma unroll
    for (int rr = 0; rr < kDeltaRows; ++rr) {
        const int64_t g0 = __shfl(gb, min(rr, nr - 1), 64), o0 = __shfl(ob, min(rr, nr - 1), 64);
        float gv[4], ov[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int d = min(tid + 64 * u, D - 1);
            gv[u] = A.dout[g0 + d];
            ov[u] = A.o[o0 + d];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {  // stores without a branch (a guarded store drew its load into the branch)
            const int d = tid + 64 * u, at = (rr < nr && d < D) ? rr * (D + 1) + d : kDeltaRows * 257;
            sg[at] = gv[u];
            so[at] = ov[u];
        }
    }
    __syncthreads();
    if (tid >= nr) return;
    const float *g = sg + tid * (D + 1), *o = so + tid * (D + 1);
    double acc = 0.0;
    for (int d = 0; d < D; ++d) acc = fma((double)g[d], (double)o[d], acc);
    A.delta[r0 + tid] = acc;
}

// p and ds of a 64 x 64 tile of pairs (rows of the chunk x keys); with SC the
// scores were stored in P by the matrix-core score path (bf16 inputs; the
// same s, see qk.hip) and only the dp chain runs here:
//   s = RN32(RN64(scale * chain(q, k))), w = RN32(exp_det(RN64(s - m))),
//   p = RN32(RN64(w / den64)), ds = RN32(RN64(p * RN64(chain(dO, v) - delta))),
// invisible pairs 0, with register blocking: thread (tr, tc) = (tid / 16,
// tid % 16) owns rows 4 tr .. 4 tr + 3 and keys 4 tc .. 4 tc + 3 and runs both
// chains of its 16 pairs, d ascending.  Q, K, dO and V are staged in LDS as
// binary64 (exact widening) in chunks of kPdsDc dimensions, transposed to
// [d][row] so a thread reads its four rows' operands with two 16-byte loads
// (K and V with their keys interleaved so those loads are contiguous over
// the lanes); wave w fills array w, lane = row.  Grid (key tiles, row tiles, heads);
// tiles wholly above the causal diagonal are skipped.
constexpr int kPdsT = 64;   // rows and keys of a tile
constexpr int kPdsDc = 32;  // dimensions per LDS stage
constexpr int kPdsLd = kPdsT + 2;  // row stride of the staged arrays (16-byte aligned rows of doubles)

template <typename T, bool SC>
__global__ __launch_bounds__(256) void k_bwd_pds64(BwdArgs A) {
    constexpr int AO = SC ? 2 : 0;  // first staged array: Q, K, dO, V (with stored scores dO, V)
    constexpr int NR = SC ? 16 : 32;  // staged rows per lane and stage
    __shared__ __align__(16) double sm[4 - AO][kPdsDc][kPdsLd];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int tr = tid >> 4, tc = tid & 15;
    const int64_t kt = blockIdx.x, rt = blockIdx.y, bh = blockIdx.z;
    const int64_t b = bh / A.Hq, hq = bh % A.Hq, hk = hq / A.group;
    const int64_t iend = A.i0 + A.ni, ia = A.i0 + rt * kPdsT, ja = kt * kPdsT;
    const int64_t ilast = min64(iend, ia + kPdsT) - 1;
    if (A.causal && ja > ilast) return;
    // wave wv stages array wv (with stored scores: array 2 + wv / 2, rows
    // 32 (wv % 2) ..): lane handles dimension d0 + lane % 32 of rows
    // 2 r2 + lane / 32 (clamped into range; such rows are never stored), so
    // each load instruction reads two rows' contiguous dimensions; the next
    // stage's values are fetched into registers while this stage computes
    const void *src;
    int64_t base, rs;
    int64_t r0, rmax;
    bool isf32 = false;
    const int arr = SC ? 2 + (wv >> 1) : wv, rofs = SC ? 32 * (wv & 1) : 0;
    switch (arr) {
        case 0: src = A.q; base = b * A.qsB + hq * A.qsH; rs = A.qsS; r0 = ia; rmax = iend - 1; break;
        case 1: src = A.k; base = b * A.ksB + hk * A.ksH; rs = A.ksS; r0 = ja; rmax = A.Skv - 1; break;
        case 2: src = A.dout; base = b * A.dsB + hq * A.dsH; rs = A.dsS; r0 = ia; rmax = iend - 1; isf32 = true; break;
        default: src = A.v; base = b * A.vsB + hk * A.vsH; rs = A.vsS; r0 = ja; rmax = A.Skv - 1; break;
    }
    r0 += rofs;
    const int D = (int)A.D, dl = lane & 31, rh = lane >> 5;
    // all 32 loads of a stage are issued before any is used: in-range
    // (clamped) addresses, one element width per wave, no branches
    const bool w32 = __builtin_amdgcn_readfirstlane((int)(isf32 || sizeof(T) == 4)) != 0;
    uint32_t nx[NR];
    auto gload = [&](int d0) {
        const int64_t d = min(d0 + dl, D - 1);
        if (w32) {
            const uint32_t *p = (const uint32_t *)src + base + d;
#pragma unroll
            for (int r2 = 0; r2 < NR; ++r2) nx[r2] = p[min64(r0 + 2 * r2 + rh, rmax) * rs];
        } else {
            const uint16_t *p = (const uint16_t *)src + base + d;
#pragma unroll
            for (int r2 = 0; r2 < NR; ++r2) nx[r2] = (uint32_t)p[min64(r0 + 2 * r2 + rh, rmax) * rs] << 16;
        }
    };
    double as[4][4], ap[4][4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int t = 0; t < 4; ++t) as[u][t] = ap[u][t] = 0.0;
    gload(0);
    for (int d0 = 0; d0 < D; d0 += kPdsDc) {
        const int dn = min(kPdsDc, D - d0);
        __syncthreads();  // the previous stage's readers are done
        const bool dok = d0 + dl < D;
#pragma unroll
        for (int r2 = 0; r2 < NR; ++r2) {
            // K and V keys j = 4 tc + t sit at 32 (t / 2) + 2 tc + t % 2, so the
            // sixteen tc of a read touch one contiguous 256-byte run
            const int j = rofs + 2 * r2 + rh;
            const int col = (arr & 1) ? ((j & 2) << 4) + ((j >> 2) << 1) + (j & 1) : j;
            sm[arr - AO][dl][col] = dok ? (double)__uint_as_float(nx[r2]) : 0.0;
        }
        __syncthreads();
        if (d0 + kPdsDc < D) gload(d0 + kPdsDc);
        for (int dd = 0; dd < dn; ++dd) {
            const double2 *ro = (const double2 *)&sm[2 - AO][dd][4 * tr], *rv = (const double2 *)&sm[3 - AO][dd][2 * tc];
            const double2 o01 = ro[0], o23 = ro[1], v01 = rv[0], v23 = rv[16];
            const double ov[4] = {o01.x, o01.y, o23.x, o23.y}, vv[4] = {v01.x, v01.y, v23.x, v23.y};
            if (!SC) {
                const double2 *rq = (const double2 *)&sm[0][dd][4 * tr], *rk = (const double2 *)&sm[1][dd][2 * tc];
                const double2 q01 = rq[0], q23 = rq[1], k01 = rk[0], k23 = rk[16];
                const double qv[4] = {q01.x, q01.y, q23.x, q23.y}, kv[4] = {k01.x, k01.y, k23.x, k23.y};
#pragma unroll
                for (int u = 0; u < 4; ++u)
#pragma unroll
                    for (int t = 0; t < 4; ++t) as[u][t] = fma(qv[u], kv[t], as[u][t]);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int t = 0; t < 4; ++t) ap[u][t] = fma(ov[u], vv[t], ap[u][t]);
        }
    }
    // p, ds and the exponent statistics for the matrix-core sums.  The row
    // statistics and (SC) the 16 stored scores are loaded together first, from
    // in-range (clamped) addresses, so their latencies overlap.
    float rm[4], sv[4][4];
    double rden[4], rdelta[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int64_t ic = min64(ia + 4 * tr + u, iend - 1);
        const int64_t row = bh * A.Sq + ic;
        rm[u] = A.rowmax[row];
        rden[u] = A.den64[row];
        rdelta[u] = A.delta[row];
        if (SC) {
            const float *sp = A.P + (bh * A.ni + (ic - A.i0)) * A.Skv;
#pragma unroll
            for (int t = 0; t < 4; ++t) sv[u][t] = sp[min64(ja + 4 * tc + t, A.Skv - 1)];
        }
    }
    int re[4], rl[4], ce[4], cl[4], pe[4], pl[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        ce[t] = pe[t] = INT_MIN;
        cl[t] = pl[t] = INT_MAX;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int64_t i = ia + 4 * tr + u;
        const bool rowok = i < iend;
        const float m = rm[u];
        const double den = rden[u], delta = rdelta[u];
        re[u] = INT_MIN;
        rl[u] = INT_MAX;
        float pv[4], dv[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int64_t j = ja + 4 * tc + t;
            float p = 0.0f, ds = 0.0f;
            if (rowok && j < A.Skv && (!A.causal || j <= i)) {
                // the stored score (the matrix-core score path wrote it into P) or the chain's
                const float s = SC ? sv[u][t] : (float)(A.scale * as[u][t]);
                const float w = weight(s, m);
                p = (float)((double)w / den);
                ds = (float)((double)p * (ap[u][t] - delta));
            }
            pv[t] = p;
            dv[t] = ds;
            int e, l;
            stat_of(ds, e, l);
            re[u] = max(re[u], e);
            rl[u] = min(rl[u], l);
            ce[t] = max(ce[t], e);
            cl[t] = min(cl[t], l);
            stat_of(p, e, l);
            pe[t] = max(pe[t], e);
            pl[t] = min(pl[t], l);
        }
        if (rowok) {
            const int64_t at = (bh * A.ni + (i - A.i0)) * A.Skv + ja + 4 * tc;
#pragma unroll
            for (int t = 0; t < 4; ++t)
                if (ja + 4 * tc + t < A.Skv) {
                    A.P[at + t] = pv[t];
                    A.DS[at + t] = dv[t];
                }
        }
    }
    // ds row statistics over the tile's keys: lanes of one tr differ in tc (xor 1..8)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
            re[u] = max(re[u], __shfl_xor(re[u], o, 64));
            rl[u] = min(rl[u], __shfl_xor(rl[u], o, 64));
        }
        const int64_t i = ia + 4 * tr + u;
        if (tc == 0 && i < iend && re[u] != INT_MIN) {
            int2 *st = A.st_rds + bh * A.ni + (i - A.i0);
            atomicMax(&st->x, re[u]);
            atomicMin(&st->y, rl[u]);
        }
    }
    // ds and p key statistics over the wave's 16 rows (xor 16, 32), then over
    // the four waves in LDS (the staging arrays are free after the barrier):
    // one atomic per key and value from the workgroup
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int o = 16; o < 64; o <<= 1) {
            ce[t] = max(ce[t], __shfl_xor(ce[t], o, 64));
            cl[t] = min(cl[t], __shfl_xor(cl[t], o, 64));
            pe[t] = max(pe[t], __shfl_xor(pe[t], o, 64));
            pl[t] = min(pl[t], __shfl_xor(pl[t], o, 64));
        }
    }
    __syncthreads();  // every wave is done with the staged operands
    int4 *ks = (int4 *)&sm[0][0][0];  // [wave][key] {ds emax, ds lmin, p emax, p lmin}
    if (lane < 16) {
#pragma unroll
        for (int t = 0; t < 4; ++t) ks[wv * kPdsT + 4 * tc + t] = int4{ce[t], cl[t], pe[t], pl[t]};
    }
    __syncthreads();
    if (tid < kPdsT && ja + tid < A.Skv) {
        int4 v = ks[tid];
#pragma unroll
        for (int w = 1; w < 4; ++w) {
            const int4 u = ks[w * kPdsT + tid];
            v.x = max(v.x, u.x);
            v.y = min(v.y, u.y);
            v.z = max(v.z, u.z);
            v.w = min(v.w, u.w);
        }
        const int64_t at = (b * A.Hkv + hk) * A.Skv + ja + tid;
        if (v.x != INT_MIN) {
            atomicMax(&A.st_cds[at].x, v.x);
            atomicMin(&A.st_cds[at].y, v.y);
        }
        if (v.z != INT_MIN) {
            atomicMax(&A.st_cp[at].x, v.z);
            atomicMin(&A.st_cp[at].y, v.w);
        }
    }
}

// Column statistics of a B operand over rows [s0, s1) of the heads h = hk *
// ng + g, g < ng, of a [B, H, S, D] view (K: ng = 1 and all keys; Q and dO:
// ng = the group and the chunk's rows), into st[bhk * D + d].  Grid (column
// groups of 32, row blocks of 256, bhk * ng).
template <typename T>
__global__ __launch_bounds__(256) void k_bwd_colstats(const void *src, int64_t sB, int64_t sH, int64_t sS,
                                                      int64_t ng, int64_t Hkv, int64_t s0, int64_t s1, int64_t D,
                                                      int2 *st) {
    __shared__ int se[8][32], sl[8][32];
    const int t = threadIdx.x, c = t & 31, s8 = t >> 5;
    const int64_t z = blockIdx.z, bhk = z / ng, g = z % ng;
    const int64_t b = bhk / Hkv, hk = bhk % Hkv, h = hk * ng + g;
    const int64_t d = (int64_t)blockIdx.x * 32 + c;
    const int64_t r0 = s0 + (int64_t)blockIdx.y * 256, r1 = min64(s1, r0 + 256);
    int emax = INT_MIN, lmin = INT_MAX;
    if (d < D) {
        const T *col = (const T *)src + b * sB + h * sH + d;
#pragma unroll 4
        for (int64_t s = r0 + s8; s < r1; s += 8) {
            int e, l;
            stat_of_exact(elem<T>::to_f32(col[s * sS]), e, l);
            emax = max(emax, e);
            lmin = min(lmin, l);
        }
    }
    se[s8][c] = emax;
    sl[s8][c] = lmin;
    __syncthreads();
    if (t >= 32) return;
#pragma unroll
    for (int k = 1; k < 8; ++k) {
        emax = max(emax, se[k][c]);
        lmin = min(lmin, sl[k][c]);
    }
    if (d < D && emax != INT_MIN) {
        atomicMax(&st[bhk * D + d].x, emax);
        atomicMin(&st[bhk * D + d].y, lmin);
    }
}

// Digit blocks of the right operands of the matrix-core sums (K, Q, dO), one
// wave per block of 16 operand columns d by 64 reduction steps t.  Lane l
// holds column x = l % 16 at steps 16 (l / 16) + 0..15, the int8 operand
// order of v_mfma_i32_16x16x64_i8.  Each column is an integer on its grid,
// Xi = X 2^-g_x, written as n balanced base-256 digits (n of the block = the
// largest of its columns): the bytes of Xi + 0x80..80 with their top bit
// flipped.  Blocks whose columns need more digits than the kernel holds are
// not written (their tiles take the per-term sums).
//   MODE 3: B of dQ, unit (bhk, 16-column group, 64-key block): K[j][d]
//   MODE 4, 5: B of dK, dV, unit (bhk, 16-column group, g, 64-row block): Q / dO [i][d]
template <int MODE, typename T>
__global__ __launch_bounds__(256) void k_bwd_slice(BwdArgs A, int64_t nunits) {
    const int lane = threadIdx.x & 63;
    const int64_t u = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (u >= nunits) return;  // wave-uniform
    const int xr = lane & 15, tb = 16 * (lane >> 4);
    float val[16];
    int2 st = int2{INT_MIN, INT_MAX};
    int kmax;
    v4i *out;
    if (MODE == 3) {
        const int64_t jb = u % A.nJB64, G = (u / A.nJB64) % A.nG16, bhk = u / (A.nJB64 * A.nG16);
        const int64_t b = bhk / A.Hkv, hk = bhk % A.Hkv, d = G * 16 + xr;
        if (d < A.D) st = A.st_k[bhk * A.D + d];
        const int64_t base = b * A.ksB + hk * A.ksH + (d < A.D ? d : 0);
        float x[16];
#pragma unroll
        for (int p = 0; p < 16; ++p) x[p] = ld<T>(A.k, base + min64(jb * 64 + tb + p, A.Skv - 1) * A.ksS);
#pragma unroll
        for (int p = 0; p < 16; ++p) {
            const float xp = keep(x[p]);
            val[p] = (d < A.D && jb * 64 + tb + p < A.Skv) ? xp : 0.0f;
        }
        kmax = kXB;
        out = A.xb[0] + u * kXB * 64;
    } else {
        const int64_t ib = u % A.nIB64, g = (u / A.nIB64) % A.group, G = (u / (A.nIB64 * A.group)) % A.nG16,
                      bhk = u / (A.nIB64 * A.group * A.nG16);
        const int64_t b = bhk / A.Hkv, hk = bhk % A.Hkv, hq = hk * A.group + g, d = G * 16 + xr;
        if (d < A.D) st = (MODE == 4 ? A.st_q : A.st_o)[bhk * A.D + d];
        const int64_t dd = d < A.D ? d : 0;
        float x[16];
#pragma unroll
        for (int p = 0; p < 16; ++p) {
            const int64_t i = A.i0 + min64(ib * 64 + tb + p, A.ni - 1);
            x[p] = MODE == 4 ? ld<T>(A.q, b * A.qsB + hq * A.qsH + i * A.qsS + dd)
                             : A.dout[b * A.dsB + hq * A.dsH + i * A.dsS + dd];
        }
#pragma unroll
        for (int p = 0; p < 16; ++p) {
            const float xp = keep(x[p]);
            val[p] = (d < A.D && ib * 64 + tb + p < A.ni) ? xp : 0.0f;
        }
        kmax = kXB;
        out = A.xb[MODE - 3] + u * kXB * 64;
    }
    int g, n;
    grid_of(st, g, n);
    const int nt = __builtin_amdgcn_readfirstlane(wave_max(n));
    if (nt == 0 || nt > kmax) return;
    // Xi + 0x80..80 (nt bytes) for the 16 values, as 128-bit integers
    unsigned __int128 off = 0;
    for (int a = 0; a < nt; ++a) off = (off << 8) | 0x80u;
    unsigned __int128 U[16];
#pragma unroll
    for (int p = 0; p < 16; ++p) {
        const uint32_t bits = __float_as_uint(val[p]);
        const uint32_t be = (bits >> 23) & 0xffu;
        const uint64_t m = (bits & 0x7fffffu) | (be ? 0x800000u : 0u);
        // m 2^sh on the column's grid; sh < 0 only where m ends in at least -sh zero bits
        const int sh = (int)(be ? be : 1u) - 150 - g;
        const unsigned __int128 mag = !m ? 0 : sh >= 0 ? ((unsigned __int128)m << (sh & 127))
                                                       : (unsigned __int128)(m >> min(-sh, 63));
        U[p] = ((bits >> 31) ? off - mag : off + mag);
    }
    for (int a = 0; a < nt; ++a) {
        uint32_t wv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint32_t pack = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) pack |= ((uint32_t)(U[4 * q + e] >> (8 * a)) & 255u) << (8 * e);
            wv[q] = pack ^ 0x80808080u;
        }
        out[a * 64 + lane] = v4i{(int)wv[0], (int)wv[1], (int)wv[2], (int)wv[3]};
    }
}

// The matrix-core sums.  A workgroup of eight waves owns 32 rows x 64
// columns of one head's outputs; wave w takes the 16 x 16 tile of row half
// w & 1 and 16-column group w >> 1.  C_s += A_a x B_b (s = a + b) over the
// 64-step reduction blocks on v_mfma_i32_16x16x64_i8, exact in int32
// (|a_a b_b| <= 2^14, at most seven pairs per class and step, classes carried
// every 8192 steps; the top class only ever holds the product of the two top
// digits, each at most 2^6), then the exact sum X = sum_s 256^s C_s
// (|X| < 2^125) times 2^(ga_x + gb_d):
//   MODE 0 (dQ): grid (64-column groups, 32-row tiles, bh); the tile owns every
//     key, so dQ = RN32(RN64(scale RN64(X 2^e))) is stored directly;
//   MODE 1, 2 (dK, dV): grid (64-column groups, 32-key tiles, bhk * group);
//     the workgroup covers one query head's rows of the chunk and adds X 2^e
//     into the digit planes (integer atomics: any order gives the same digits).
// The left operand's digits are made here from the f32 ds / p of each block
// and shared by the eight waves through LDS (double buffered, one barrier per
// block); each wave keeps its B digits in registers, fetched one block ahead.
// Thirteen classes of a 16 x 16 tile take 52 registers, so two waves share a
// SIMD.  A tile whose rows or 32-column group need more digits than the kernel
// holds is flagged for k_bwd_sum (flags per 32 x 32 tile) and left alone.
constexpr int kT16 = 64;                 // reduction steps per block
constexpr int kXCarry16 = 8192 / kT16;   // blocks between class carries

template <int MODE>
__global__ __launch_bounds__(512, 4) void k_bwd_mma(BwdArgs A) {
    __shared__ v4i sA[2][kXA][2][64];  // [slot][digit][row half][lane]
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int rh = wv & 1;
    const int64_t G16 = (int64_t)blockIdx.x * 4 + (wv >> 1), G32 = G16 >> 1;
    const int64_t y = blockIdx.y, z = blockIdx.z;
    const int64_t d = G16 * 16 + (lane & 15);
    int2 sa = int2{INT_MIN, INT_MAX}, sb = int2{INT_MIN, INT_MAX}, sb32 = int2{INT_MIN, INT_MAX};
    int64_t bh = 0, bhk, g = 0, nblk, k0;
    const v4i *pb;
    int *flag;
    {
        const int x32 = lane & 31;  // rows 0..31 of the tile, for the tile's digit count
        if (MODE == 0) {
            bh = z;
            const int64_t b = bh / A.Hq, hk = (bh % A.Hq) / A.group, ir = y * 32 + x32;
            bhk = b * A.Hkv + hk;
            if (ir < A.ni) sa = A.st_rds[bh * A.ni + ir];
            k0 = 0;
            nblk = A.causal ? min64(A.nJB64, (A.i0 + y * 32 + 31) / kT16 + 1) : A.nJB64;
            pb = A.xb[0] + (bhk * A.nG16 + G16) * A.nJB64 * kXB * 64;
            flag = A.xf[0] + (bh * A.nIB + y) * A.nG + G32;
        } else {
            bhk = z / A.group;
            g = z % A.group;
            const int64_t j = y * 32 + x32;
            if (j < A.Skv) sa = (MODE == 1 ? A.st_cds : A.st_cp)[bhk * A.Skv + j];
            k0 = (A.causal && y * 32 > A.i0) ? (y * 32 - A.i0) / kT16 : 0;
            nblk = A.nIB64;
            pb = A.xb[MODE] + ((bhk * A.nG16 + G16) * A.group + g) * A.nIB64 * kXB * 64;
            flag = A.xf[MODE] + (bhk * A.nJB + y) * A.nG + G32;
        }
    }
    const int2 *stb = MODE == 0 ? A.st_k : MODE == 1 ? A.st_q : A.st_o;
    const bool mine = G16 < A.nG16;  // wave-uniform: the wave has columns
    if (mine && d < A.D) sb = stb[bhk * A.D + d];
    const int64_t d32 = G32 * 32 + (lane & 31);
    if (G32 < A.nG && d32 < A.D) sb32 = stb[bhk * A.D + d32];
    int ga, na, gb, nb, gb32, nb32;
    grid_of(sa, ga, na);
    grid_of(sb, gb, nb);
    grid_of(sb32, gb32, nb32);
    const int nat = __builtin_amdgcn_readfirstlane(wave_max(na));  // the same in every wave
    const int nbt = __builtin_amdgcn_readfirstlane(wave_max(nb));
    const int nbg = __builtin_amdgcn_readfirstlane(wave_max(nb32));  // the 32-column group's count
    const bool abad = A.force_fallback || nat > kXA || (MODE == 0 ? A.Skv : A.ni) > kXMaxT;
    const bool bad = abad || nbg > kXB || nat + nbg > kXC + 1;
    if (G32 < A.nG && (G16 & 1) == 0 && rh == 0 && (MODE == 0 || g == 0) && lane == 0) *flag = bad ? 1 : 0;
    if (abad) return;  // workgroup-uniform
    const bool run = mine && !bad && nbt > 0;  // wave-uniform
    if (nat == 0) nblk = k0;  // a zero operand: X = 0

    v4i C[kXC];
#pragma unroll
    for (int s = 0; s < kXC; ++s) C[s] = v4i{0, 0, 0, 0};
    // The left operand's digits, made from the f32 ds / p of each block:
    // thread tid holds 4 consecutive steps t0..t0+3 of operand row xa,
    // converts them on the row's grid and writes its 32-bit word of every
    // digit plane of the LDS operand image (half xa / 16, lane xa % 16 +
    // 16 (t0 / 16), bytes t0 % 16 ..).  A wave takes one row half and one
    // 16-step group (wave w: half w & 1, group w >> 1), its lane l row
    // xa % 16 = l / 4 and word l % 4, so the wave's 64 words of a plane are
    // consecutive (no two lanes on one LDS bank line).
    const int xa = 16 * (wv & 1) + (lane >> 2), t0 = 16 * (wv >> 1) + 4 * (lane & 3);
    int gx;
    const float *srow;
    int64_t sstep;
    bool xok;
    {
        int2 st = int2{INT_MIN, INT_MAX};
        if (MODE == 0) {
            const int64_t ir = y * 32 + xa;
            xok = ir < A.ni;
            if (xok) st = A.st_rds[bh * A.ni + ir];
            srow = A.DS + (bh * A.ni + (xok ? ir : 0)) * A.Skv;
            sstep = 1;
        } else {
            const int64_t j = y * 32 + xa, b = bhk / A.Hkv, hk = bhk % A.Hkv;
            xok = j < A.Skv;
            if (xok) st = (MODE == 1 ? A.st_cds : A.st_cp)[bhk * A.Skv + j];
            srow = (MODE == 1 ? A.DS : A.P) + (b * A.Hq + hk * A.group + g) * A.ni * A.Skv + (xok ? j : 0);
            sstep = A.Skv;
        }
        int nx_;
        grid_of(st, gx, nx_);
    }
    // (step counts are below 2^17: 32-bit step arithmetic, one 64-bit offset per block)
    const int tmax = (int)(MODE == 0 ? A.Skv - 1 : A.ni - 1);
    // the operand row's visible steps: t <= tlast (dQ: keys up to the query row)
    // and t >= tfirst (dK, dV: query rows from the key on)
    const int tlast = (A.causal && MODE == 0) ? (int)min64(tmax, A.i0 + y * 32 + xa) : tmax;
    const int tfirst = (A.causal && MODE != 0) ? (int)max64(0, y * 32 + xa - A.i0) : 0;
    // Steps tb .. tb + 3 of block kb: keys (dQ) or chunk rows (dK, dV).  The
    // loads (clamped, in range) are issued here and the values masked only in
    // stash_a, after the products: masking them here let the compiler move
    // each load into the branch of its select, with a wait per load.
    auto fetch_a = [&](int64_t kb, float (&av)[4]) {
        const int tb = (int)kb * kT16 + t0, tc = min(tb, tmax);
        const float *p = srow + (int64_t)tc * sstep;
#pragma unroll
        for (int e = 0; e < 4; ++e) av[e] = p[(min(tb + e, tmax) - tc) * (int)sstep];
    };
    auto mask_a = [&](int64_t kb, float (&av)[4]) {
        const int tb = (int)kb * kT16 + t0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int t = tb + e;
            const float x = keep(av[e]);
            av[e] = (xok && t >= tfirst && t <= tlast) ? x : 0.0f;
        }
    };
    // Digits of one entry: Xi = +-x 256^q with x = m 2^r < 2^31 (m the 24-bit
    // significand, sh = 8q + r its shift onto the row's grid).  The bytes of
    // 0x80..80 +- x 256^q are 0x80 below q, the four bytes of w = 0x80808080
    // +- x at q..q+3 (no borrow: x < 0x80808080), 0x80 plus the carry of
    // that add at q+4 and 0x80 above, so the balanced digits (bytes ^ 0x80)
    // are the bytes of the 33-bit value carry:(w ^ 0x80808080) shifted up by
    // q bytes, and 0 elsewhere.  With each entry's digit string as an 80-bit
    // value (planes 0..9), the thread's word of plane a is byte a of its four
    // entries: a byte transpose by permutes (v_perm_b32: selector byte k in
    // 0..3 names a byte of the second source, 4..7 one of the first), stored
    // as whole words into the planes the row uses.
    const int wofs = (((xa >> 4) * 64) + (xa & 15) + 16 * (t0 >> 4)) * 4 + ((t0 & 15) >> 2);  // in uint32
    auto stash_a = [&](int buf, const float (&av)[4]) {
        uint32_t *wb = (uint32_t *)&sA[buf][0][0][0] + wofs;
        uint32_t lo[4], mid[4], hi[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t bits = __float_as_uint(av[e]);
            const uint32_t be = (bits >> 23) & 0xffu;
            const uint32_t m = (bits & 0x7fffffu) | (be ? 0x800000u : 0u);
            const int sh = (int)(be ? be : 1u) - 150 - gx;  // >= 0 for every nonzero entry of the row
            const uint32_t x = m << (sh & 7);
            const bool neg = (bits >> 31) != 0;
            const uint32_t w = neg ? 0x80808080u - x : 0x80808080u + x;
            const bool carry = !neg && w < x;  // the add wrapped past 2^32
            const bool nz = (bits & 0x7fffffffu) != 0u;
            const uint64_t dv = nz ? ((uint64_t)carry << 32) | (w ^ 0x80808080u) : 0ull;
            const unsigned __int128 v = (unsigned __int128)dv << ((8 * (sh >> 3)) & 127);  // (q < kXA)
            lo[e] = (uint32_t)v;
            mid[e] = (uint32_t)(v >> 32);
            hi[e] = (uint32_t)(v >> 64);
        }
        uint32_t word[12];
        auto transpose4 = [&](const uint32_t (&L)[4], int a0) {
            const uint32_t x01l = __builtin_amdgcn_perm(L[1], L[0], 0x05010400u);
            const uint32_t x01h = __builtin_amdgcn_perm(L[1], L[0], 0x07030602u);
            const uint32_t x23l = __builtin_amdgcn_perm(L[3], L[2], 0x05010400u);
            const uint32_t x23h = __builtin_amdgcn_perm(L[3], L[2], 0x07030602u);
            word[a0] = __builtin_amdgcn_perm(x23l, x01l, 0x05040100u);
            word[a0 + 1] = __builtin_amdgcn_perm(x23l, x01l, 0x07060302u);
            word[a0 + 2] = __builtin_amdgcn_perm(x23h, x01h, 0x05040100u);
            word[a0 + 3] = __builtin_amdgcn_perm(x23h, x01h, 0x07060302u);
        };
        transpose4(lo, 0);
        transpose4(mid, 4);
        transpose4(hi, 8);
#pragma unroll
        for (int a = 0; a < kXA; ++a)
            if (a < nat) wb[a * 512] = word[a];
    };
    // the wave's B digits of a block are loaded at the start of its step
    // (other waves on the SIMD cover the latency: two workgroups per CU)
    v4i Bc[kXB];
    auto fetch_b = [&](int64_t kb) {
        if (!run) return;
        const v4i *q = pb + kb * kXB * 64 + lane;
#pragma unroll
        for (int b = 0; b < kXB; ++b)
            if (b < nbt) Bc[b] = q[b * 64];
    };
    // step kb: block kb's digits in slot (kb - k0) & 1; block kb + 1's f32
    // values are fetched first and its digits made after the products of
    // block kb
    float F[4];
    auto step = [&](int64_t kb) {
        const int buf = (int)((kb - k0) & 1);
        const bool more = kb + 1 < nblk;
        fetch_a(kb + 1, F);  // in range past the last block too: a fixed count of loads after B's
        if (run) {
            const v4i *sa_ = &sA[buf][0][rh][lane];
            v4i Acur = sa_[0];
#pragma unroll
            for (int a = 0; a < kXA; ++a) {
                if (a < nat) {
                    const v4i Anext = sa_[((a + 1) % kXA) * 128];  // digit a+1 read while a's products run
#pragma unroll
                    for (int b = 0; b < kXB; ++b)
                        if (a + b < kXC && b < nbt)
                            C[a + b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(Acur, Bc[b], C[a + b], 0, 0, 0);
                    Acur = Anext;
                }
            }
            if (((kb - k0) % kXCarry16) == kXCarry16 - 1) {
#pragma unroll
                for (int s = 0; s < kXC - 1; ++s) {
                    const v4i c = C[s] >> 8;
                    C[s] -= c << 8;
                    C[s + 1] += c;
                }
            }
        }
        mask_a(kb + 1, F);  // every step waits for its loads: none is in flight at the next
        if (more) stash_a(buf ^ 1, F);  // its readers passed the previous barrier
        fetch_b(more ? kb + 1 : kb);  // the next block's B digits load across the barrier
        __syncthreads();
    };
    if (k0 < nblk) {
        fetch_a(k0, F);
        mask_a(k0, F);
        stash_a(0, F);
    }
    if (k0 < nblk) fetch_b(k0);
    __syncthreads();
    for (int64_t kb = k0; kb < nblk; ++kb) step(kb);
    if (!mine || bad) return;
    // classes to bytes: C_0 .. C_11 in [0, 256), C_12 signed
#pragma unroll
    for (int s = 0; s < kXC - 1; ++s) {
        const v4i c = C[s] >> 8;
        C[s] &= 255;
        C[s + 1] += c;
    }
    int gam[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) gam[r] = __shfl(ga, rh * 16 + 4 * (lane >> 4) + r, 64);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int m = rh * 16 + 4 * (lane >> 4) + r;  // row of the 32-row tile
        const uint32_t l0 = (uint32_t)C[0][r] | ((uint32_t)C[1][r] << 8) | ((uint32_t)C[2][r] << 16) |
                            ((uint32_t)C[3][r] << 24);
        const uint32_t l1 = (uint32_t)C[4][r] | ((uint32_t)C[5][r] << 8) | ((uint32_t)C[6][r] << 16) |
                            ((uint32_t)C[7][r] << 24);
        const uint32_t l2 = (uint32_t)C[8][r] | ((uint32_t)C[9][r] << 8) | ((uint32_t)C[10][r] << 16) |
                            ((uint32_t)C[11][r] << 24);
        const uint64_t lo = ((uint64_t)l1 << 32) | l0;
        const int64_t hi = (int64_t)C[12][r] * ((int64_t)1 << 32) + (int64_t)l2;
        const int e = gam[r] + gb;
        if (d >= A.D) continue;
        if (MODE == 0) {
            const int64_t ir = y * 32 + m;
            if (ir >= A.ni) continue;
            const int64_t b = bh / A.Hq, hq = bh % A.Hq;
            const double v = i128_to_f64(hi, lo, e);
            A.dq.data[b * A.dq.sB + hq * A.dq.sH + (A.i0 + ir) * A.dq.sS + d] = (float)(A.scale * v);
        } else {
            const int64_t j = y * 32 + m;
            if (j >= A.Skv) continue;
            const __int128 num = (__int128)(((unsigned __int128)(uint64_t)hi << 64) | lo);
            int64_t *dig = MODE == 1 ? A.dk_dig : A.dv_dig;
            const int64_t plane = A.nbh / A.group * A.Skv * A.D;
            add_i128_digits<kBwdDigits>(num, e - kBwdElo, dig + (bhk * A.Skv + j) * A.D + d, plane);
        }
    }
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

// Per-term exact sums for a 16 x 16 tile of outputs, one thread per output,
// for the tiles k_bwd_mma flagged (the others return at once).
//   MODE 0 (dQ): rows = chunk rows i of head bh, terms ds_ij K_jd over keys j;
//     the tile owns every key, so dQ is rounded and stored here
//   MODE 1 (dK): rows = keys j of key head bhk, terms ds_ij Q_id over (query head, row)
//   MODE 2 (dV): the same with p_ij dO_id; both added into the digit planes
// Grid (column tiles, row tiles, heads).  Per step 32 terms of the tile's
// rows and columns are staged in LDS.
template <int MODE, typename T>
__global__ __launch_bounds__(256) void k_bwd_sum(BwdArgs A) {
    __shared__ int64_t dig[kBwdDigits][256];
    __shared__ float sa[kBT][kBStep + 1], sb[kBStep][kBT + 1];
    const int tid = threadIdx.x, r = tid >> 4, c = tid & 15;
    const int64_t da = (int64_t)blockIdx.x * kBT, ra = (int64_t)blockIdx.y * kBT, hh = blockIdx.z;
    // only the tiles the matrix-core sums left (flag 1); ra is a chunk row (dQ) or a key
    const int tf = MODE == 0 ? A.xf[0][(hh * A.nIB + ra / 32) * A.nG + da / 32]
                             : A.xf[MODE][(hh * A.nJB + ra / 32) * A.nG + da / 32];
    if (!tf) return;
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
        // the tile owns every key of its rows: dQ = RN32(RN64(scale RN64(sum)))
        const int64_t i = ia + r, d = da + c;
        if (i < iend && d < A.D) {
            int64_t x[kBwdDigits];
#pragma unroll
            for (int k = 0; k < kBwdDigits; ++k) x[k] = dig[k][tid];
            canonicalize<kBwdDigits>(x);
            A.dq.data[b * A.dq.sB + (bh % A.Hq) * A.dq.sH + i * A.dq.sS + d] =
                (float)(A.scale * digits_to_f64<kBwdDigits>(x, kBwdElo));
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

// out = RN32(RN64(f * RN64(X))) of each digit sum X: dK (f = scale) from the
// planes at dig0, then dV (f = 1) from those at dig1, one launch; row R of the
// planes is (head, s) = (R / S, R % S) of the output view.
__global__ __launch_bounds__(256) void k_bwd_finalize(const int64_t *dig0, const int64_t *dig1, int64_t rows,
                                                      int64_t D, int64_t S, int64_t H, double f0, OutView o0,
                                                      OutView o1) {
    int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= 2 * rows * D) return;
    const bool second = t >= rows * D;
    if (second) t -= rows * D;
    const int64_t *dig = second ? dig1 : dig0;
    const double f = second ? 1.0 : f0;
    const OutView o = second ? o1 : o0;
    const int64_t R = t / D, d = t % D;
    int64_t x[kBwdDigits];
#pragma unroll
    for (int k = 0; k < kBwdDigits; ++k) x[k] = dig[k * rows * D + t];
    canonicalize<kBwdDigits>(x);
    const double v = digits_to_f64<kBwdDigits>(x, kBwdElo);
    const int64_t head = R / S, s = R % S;
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

// The chunk workspace of ni query rows, carved in one place: returns its size
// and, with A, points A's chunk arrays into base.
static size_t bwd_chunk_layout(const AttnGeom &g, int64_t ni, BwdArgs *A, char *base) {
    const int64_t bh = g.B * g.Hq, bhk = g.B * g.Hkv, grp = g.Hq / g.Hkv;
    const int64_t nIB = (ni + 31) / 32, nJB = (g.Skv + 31) / 32, nG = (g.D + 31) / 32;
    const int64_t nIB64 = (ni + kT16 - 1) / kT16, nJB64 = (g.Skv + kT16 - 1) / kT16, nG16 = (g.D + 15) / 16;
    size_t at = 0;
    auto take = [&](size_t bytes) {
        char *p = base ? base + at : nullptr;
        at += align256(bytes);
        return p;
    };
    char *P = take((size_t)bh * ni * g.Skv * 4);
    char *DS = take((size_t)bh * ni * g.Skv * 4);
    char *st = take((size_t)(bh * ni + 2 * bhk * g.Skv + 3 * bhk * g.D) * 8);
    char *xb0 = take((size_t)kXB * 1024 * bhk * nG16 * nJB64);
    char *xb1 = take((size_t)kXB * 1024 * bhk * nG16 * grp * nIB64);
    char *xb2 = take((size_t)kXB * 1024 * bhk * nG16 * grp * nIB64);
    char *fl = take((size_t)(bh * nIB * nG + 2 * bhk * nJB * nG) * 4);
    if (A) {
        A->P = (float *)P;
        A->DS = (float *)DS;
        int2 *s2 = (int2 *)st;
        A->st_rds = s2;
        A->st_cds = s2 + bh * ni;
        A->st_cp = A->st_cds + bhk * g.Skv;
        A->st_k = A->st_cp + bhk * g.Skv;
        A->st_q = A->st_k + bhk * g.D;
        A->st_o = A->st_q + bhk * g.D;
        A->xb[0] = (v4i *)xb0;
        A->xb[1] = (v4i *)xb1;
        A->xb[2] = (v4i *)xb2;
        A->xf[0] = (int *)fl;
        A->xf[1] = A->xf[0] + bh * nIB * nG;
        A->xf[2] = A->xf[1] + bhk * nJB * nG;
        A->nIB = nIB;
        A->nJB = nJB;
        A->nG = nG;
        A->nIB64 = nIB64;
        A->nJB64 = nJB64;
        A->nG16 = nG16;
    }
    return at;
}

size_t bwd_chunk_bytes(const AttnGeom &g, int64_t ni) { return bwd_chunk_layout(g, ni, nullptr, nullptr); }

hipError_t launch_zero_view(const OutView &o, int64_t B, int64_t H, int64_t S, int64_t D, hipStream_t s) {
    const int64_t n = B * H * S * D;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_bwd_zero, dim3(blocks_of(n)), dim3(256), 0, s, o, H, S, D, n);
    return hipGetLastError();
}

template <typename T>
static hipError_t launch_sums(BwdArgs &A, const AttnGeom &g, const Tensor &q, const Tensor &k, const Tensor &dout,
                              hipStream_t s) {
    const int64_t bh = g.B * g.Hq, bhk = g.B * g.Hkv, grp = A.group;
    const int64_t nIB = A.nIB, nJB = A.nJB, nG = A.nG;
    {
        ProfScope prof_("bwd_slice", s);
        const dim3 gk((unsigned)nG, (unsigned)((g.Skv + 255) / 256), (unsigned)bhk);
        const dim3 gq((unsigned)nG, (unsigned)((A.ni + 255) / 256), (unsigned)(bhk * grp));
        hipLaunchKernelGGL(k_bwd_colstats<T>, gk, dim3(256), 0, s, k.data, k.sB, k.sH, k.sS, (int64_t)1, g.Hkv,
                           (int64_t)0, g.Skv, g.D, A.st_k);
        hipLaunchKernelGGL(k_bwd_colstats<T>, gq, dim3(256), 0, s, q.data, q.sB, q.sH, q.sS, grp, g.Hkv, A.i0,
                           A.i0 + A.ni, g.D, A.st_q);
        hipLaunchKernelGGL(k_bwd_colstats<float>, gq, dim3(256), 0, s, dout.data, dout.sB, dout.sH, dout.sS, grp,
                           g.Hkv, A.i0, A.i0 + A.ni, g.D, A.st_o);
        const int64_t u3 = bhk * A.nG16 * A.nJB64, u4 = bhk * A.nG16 * grp * A.nIB64;
        hipLaunchKernelGGL((k_bwd_slice<3, T>), dim3(blocks_of(u3 * 64)), dim3(256), 0, s, A, u3);
        hipLaunchKernelGGL((k_bwd_slice<4, T>), dim3(blocks_of(u4 * 64)), dim3(256), 0, s, A, u4);
        hipLaunchKernelGGL((k_bwd_slice<5, T>), dim3(blocks_of(u4 * 64)), dim3(256), 0, s, A, u4);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    {
        ProfScope prof_("bwd_mma", s);
        const unsigned gx = (unsigned)((A.nG16 + 3) / 4);
        hipLaunchKernelGGL(k_bwd_mma<0>, dim3(gx, (unsigned)nIB, (unsigned)bh), dim3(512), 0, s, A);
        hipLaunchKernelGGL(k_bwd_mma<1>, dim3(gx, (unsigned)nJB, (unsigned)(bhk * grp)), dim3(512), 0, s, A);
        hipLaunchKernelGGL(k_bwd_mma<2>, dim3(gx, (unsigned)nJB, (unsigned)(bhk * grp)), dim3(512), 0, s, A);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    {
        ProfScope prof_("bwd_sum", s);
        const unsigned cols = (unsigned)((g.D + kBT - 1) / kBT);
        const dim3 gq(cols, (unsigned)((A.ni + kBT - 1) / kBT), (unsigned)bh);
        const dim3 gk(cols, (unsigned)((g.Skv + kBT - 1) / kBT), (unsigned)bhk);
        hipLaunchKernelGGL((k_bwd_sum<0, T>), gq, dim3(256), 0, s, A);
        hipLaunchKernelGGL((k_bwd_sum<1, T>), gk, dim3(256), 0, s, A);
        hipLaunchKernelGGL((k_bwd_sum<2, T>), gk, dim3(256), 0, s, A);
        return hipGetLastError();
    }
}

hipError_t launch_attn_backward(const Tensor &q, const Tensor &k, const Tensor &v, const Tensor &o,
                                const Tensor &dout, const float *rowmax, const double *den64, const AttnGeom &g,
                                void *fixed_ws, void *chunk_ws, int64_t chunk, const OutView &dq,
                                const OutView &dk, const OutView &dv, int force_fallback, const ScoreFn *scores,
                                hipStream_t s) {
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
    A.force_fallback = force_fallback;
    A.dq = dq;
    char *f = (char *)fixed_ws;
    A.delta = (double *)f;
    f += align256((size_t)rows * 8);
    const size_t kvdig = align256((size_t)kBwdDigits * bhk * g.Skv * g.D * 8);
    A.dk_dig = (int64_t *)f;
    A.dv_dig = (int64_t *)(f + kvdig);
    bwd_chunk_layout(g, chunk, &A, (char *)chunk_ws);
    hipError_t e;
    const int64_t kvn = kBwdDigits * bhk * g.Skv * g.D;
    // the dK and dV planes are adjacent (the second starts kvdig bytes after the first)
    if ((e = launch_fill_i64(A.dk_dig, (int64_t)(kvdig / 8) + kvn, 0, s)) != hipSuccess) return e;
    {
        ProfScope prof_("bwd_delta", s);
        hipLaunchKernelGGL(k_bwd_delta, dim3((unsigned)((rows + kDeltaRows - 1) / kDeltaRows)), dim3(64), 0, s, A, rows);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const bool bf = q.dtype == 1;
    for (int64_t i0 = 0; i0 < g.Sq; i0 += chunk) {
        A.i0 = i0;
        A.ni = std::min(chunk, g.Sq - i0);
        A.nIB = (A.ni + 31) / 32;  // the chunk's row blocks (the layout is carved for the largest chunk)
        A.nIB64 = (A.ni + kT16 - 1) / kT16;
        const int64_t rt = (A.ni + kBT - 1) / kBT;
        const int64_t nst = bh * chunk + 2 * bhk * g.Skv + 3 * bhk * g.D;  // the carved statistics
        if ((e = launch_fill_i64((int64_t *)A.st_rds, nst, kStatEmpty, s)) != hipSuccess) return e;
        if (scores && (e = (*scores)(i0, i0 + A.ni, A.P)) != hipSuccess) return e;
        {
            ProfScope prof_("bwd_pds", s);
            dim3 grid((unsigned)((g.Skv + kPdsT - 1) / kPdsT), (unsigned)((A.ni + kPdsT - 1) / kPdsT), (unsigned)bh);
            if (scores) {
                if (bf) hipLaunchKernelGGL((k_bwd_pds64<bf16_t, true>), grid, dim3(256), 0, s, A);
                else hipLaunchKernelGGL((k_bwd_pds64<float, true>), grid, dim3(256), 0, s, A);
            } else {
                if (bf) hipLaunchKernelGGL((k_bwd_pds64<bf16_t, false>), grid, dim3(256), 0, s, A);
                else hipLaunchKernelGGL((k_bwd_pds64<float, false>), grid, dim3(256), 0, s, A);
            }
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        e = bf ? launch_sums<bf16_t>(A, g, q, k, dout, s) : launch_sums<float>(A, g, q, k, dout, s);
        if (e != hipSuccess) return e;
    }
    ProfScope prof_("bwd_finalize", s);
    const int64_t nk = bhk * g.Skv;
    hipLaunchKernelGGL(k_bwd_finalize, dim3(blocks_of(2 * nk * g.D)), dim3(256), 0, s, (const int64_t *)A.dk_dig,
                       (const int64_t *)A.dv_dig, nk, g.D, g.Skv, g.Hkv, g.scale, dk, dv);
    return hipGetLastError();
}

}  // namespace det
