// vprep.hpp -- preparation of V for the matrix-core pass 2 (det-attn page,
// "Method": NUM_id = sum_j w_ij V_jd exactly).  V is put on a per-column grid
// Vi = V * 2^-g_d (g_d the smallest lsb exponent of the column's nonzero
// entries, so Vi is an integer) and split into balanced base-256 digits in the
// matrix cores' lane order.  Device code only; the launches that host these
// workgroups live in pv.hip (standalone) and qk.hip (beside the score
// preparation and the score fix).
#pragma once

#include "dev_math.hpp"
#include "kernels.hpp"

namespace det {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kBmax = 5;          // at most five digits of a V column (40-bit integers)
constexpr int kKB = 32;           // keys per block (the MFMA K)
constexpr int kVChunks = 16;      // key chunks of the V column statistics

// Column statistics of V over one key chunk, by one 256-thread workgroup: per
// column the largest exponent and the smallest lsb exponent of the nonzero
// entries; 8 key strides x 32 columns, reduced in LDS and written to
// stats[((bhk * nG + G) * kVChunks + chunk) * 32 + column] as int2 {emax, lmin}
// (no atomics, nothing to clear).
template <typename TV>
__device__ __forceinline__ void vstats_block(const VJob &J, int64_t chunk, int64_t G, int64_t bhk) {
    __shared__ int smax[8][32], smin[8][32];
    const int t = threadIdx.x, c = t & 31, st = t >> 5;
    // start the remainder list (the digit slices, a later launch, fill it)
    if (chunk == 0 && t == 0) {
        J.rare_grp[bhk * J.nG + G] = 0;
        if (G == 0 && bhk == 0) *J.rare_n = 0;
    }
    const int64_t b = bhk / J.Hkv, hk = bhk % J.Hkv;
    const int64_t len = J.kv_hi - J.kv_lo, per = (len + kVChunks - 1) / kVChunks;
    const int64_t j0 = J.kv_lo + chunk * per, j1 = min64(J.kv_hi, j0 + per);
    const int64_t d = G * 32 + c;
    int emax = INT_MIN, lmin = INT_MAX;
    if (d < J.D) {
        const TV *col = (const TV *)J.v + b * J.vsB + hk * J.vsH + d;
#pragma unroll 4
        for (int64_t j = j0 + st; j < j1; j += 8) {
            const float x = elem<TV>::to_f32(col[j * J.vsS]);
            if (x != 0.0f) {
                const int e = f32_exp(x);
                emax = max(emax, e);
                lmin = min(lmin, max(e, -126) - elem<TV>::mant_bits);
            }
        }
    }
    smax[st][c] = emax;
    smin[st][c] = lmin;
    __syncthreads();
    if (t >= 32) return;
#pragma unroll
    for (int k = 1; k < 8; ++k) {
        emax = max(emax, smax[k][c]);
        lmin = min(lmin, smin[k][c]);
    }
    ((int2 *)J.stats)[((bhk * J.nG + G) * kVChunks + chunk) * 32 + c] = int2{emax, lmin};
}

// Digits of key block kb of 32-column group G, by one wave: block (bhk, G, kb)
// holds 64 lanes x 16 bytes, lane l byte p = e_b(Vi[key kv_lo + 32kb + 16(l/32) + p][dim 32G + l%32]).
// The group's digit count is what the largest |Vi| of its 32 columns needs.  A
// column that would need more than kBmax digits on its own lsb grid gets the
// coarser grid g_d = emax_d - 37 instead (|Vi| < 2^38, five digits): Vi is then
// V rounded toward zero to that grid, and every entry with bits below it leaves
// an exact remainder V - Vi 2^g_d (|remainder| < 2^g_d) that is appended to the
// remainder list, with its group flagged; pass 2 adds those products exactly.
// The waves of block 0 also record g_d and the count for pass 2.
template <typename TV>
__device__ __forceinline__ void vslice_block(const VJob &J, int64_t kb, int64_t G, int64_t bhk, int lane) {
    const int64_t b = bhk / J.Hkv, hk = bhk % J.Hkv;
    const int64_t d = G * 32 + (lane & 31);
    const TV *col = (const TV *)J.v + b * J.vsB + hk * J.vsH + (d < J.D ? d : 0);
    const int64_t jb = J.kv_lo + kb * kKB + 16 * (lane >> 5);
    // the block's 16 entries of this lane go out as one batch of loads with
    // the column statistics, no branch between them: clamped key indices keep
    // every load inside the range (an empty range reads the first word of the
    // statistics instead), and entries past the range or the head dim are
    // zeroed below
    const bool any = J.kv_hi > J.kv_lo;
    const TV *src = any ? col : (const TV *)J.stats;
    const int64_t jlast = any ? J.kv_hi - 1 : 0, stride = any ? J.vsS : 0;
    float xv[16];
#pragma unroll
    for (int p = 0; p < 16; ++p) xv[p] = elem<TV>::to_f32(src[min64(jb + p, jlast) * stride]);
    int emax = INT_MIN, lmin = INT_MAX;
    const int2 *cs = (const int2 *)J.stats + (bhk * J.nG + G) * kVChunks * 32 + (lane & 31);
#pragma unroll
    for (int k = 0; k < kVChunks; ++k) {
        const int2 e = cs[k * 32];
        emax = max(emax, e.x);
        lmin = min(lmin, e.y);
    }
    const bool nonzero = emax != INT_MIN;
    // digits needed: |Vi| < 2^(emax + 1 - g); balanced digits hold |x| <= 2^(8B-2)
    int g = nonzero ? lmin : 0;
    int bg = nonzero ? (emax + 1 - g + 2 + 7) / 8 : 0;
    const bool split = bg > kBmax;
    if (split) {
        g = emax - 37;  // > lmin: the column keeps its top 38 bits on the grid
        bg = kBmax;
    }
#pragma unroll
    for (int off = 16; off > 0; off >>= 1) bg = max(bg, __shfl_xor(bg, off, 64));
    bg = max(bg, 1);
    if (kb == 0 && lane < 32) J.colgrid[bhk * J.Dp32 + d] = g;
    if (kb == 0 && lane == 0) J.grpB[bhk * J.nG + G] = bg;
    // the kBmax balanced digits of Vi (|Vi| < 2^38) are the bytes of
    // Vi + 0x8080808080 with their top bit flipped
    uint64_t U[16];
#pragma unroll
    for (int p = 0; p < 16; ++p) {
        const double x = d < J.D && jb + p < J.kv_hi ? (double)xv[p] : 0.0;
        U[p] = (uint64_t)((int64_t)ldexp(x, -g) + 0x8080808080ll);  // toward zero onto the grid
    }
    if (__ballot(split)) {
        // the exact remainders of a split column's entries (reread: a rare path)
        for (int p = 0; p < 16; ++p) {
            const int64_t j = jb + p;
            if (!split || d >= J.D || j >= J.kv_hi) continue;
            const double x = (double)elem<TV>::to_f32(col[j * J.vsS]);
            const double rem = x - ldexp((double)(int64_t)ldexp(x, -g), g);  // exact: the low bits of x
            if (rem != 0.0) {
                const int at = atomicAdd(J.rare_n, 1);
                if (at < kRareCap) J.rare[at] = int4{(int)bhk, (int)j, (int)d, __float_as_int((float)rem)};
                J.rare_grp[bhk * J.nG + G] = 1;
            }
        }
    }
    v4i *out = (v4i *)J.vsl + ((bhk * J.nG + G) * J.nKB + kb) * kBmax * 64;
#pragma unroll
    for (int s = 0; s < kBmax; ++s) {
        uint32_t wv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint32_t pack = 0;
#pragma unroll
            for (int u = 0; u < 4; ++u) pack |= ((uint32_t)(U[4 * q + u] >> (8 * s)) & 255u) << (8 * u);
            wv[q] = pack ^ 0x80808080u;
        }
        out[s * 64 + lane] = v4i{(int)wv[0], (int)wv[1], (int)wv[2], (int)wv[3]};
    }
}

}  // namespace det
