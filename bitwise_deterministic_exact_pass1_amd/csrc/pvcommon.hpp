// pvcommon.hpp -- the parts of pass 2 (the exact deposit of NUM and DEN on
// the matrix cores, det-attn page, "Method") that its kernels share: the
// argument block, the weight rule with the W digit split, the tile
// description, and the scores by the rule itself for the pairs the matrix
// cores leave.  Device code only.
#pragma once

#include "dev_math.hpp"
#include "kernels.hpp"
#include "qkrow.hpp"
#include "vprep.hpp"

namespace det {

typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kAw = 6;                  // digits of W
constexpr int kSw = 8 * kAw - 2;        // W = w * 2^46, |W| <= 2^46 fits six balanced digits
constexpr int kNC = kAw + kBmax - 1;    // shift classes s = a + b
constexpr int kCarryEvery = 256;        // blocks (8192 keys) between carry passes
constexpr int kPW = 4;                  // weight-making ("producer") waves of the pass-2 kernel
constexpr int kDeferCap = 1024;         // deferred pairs a tile can hold (more: the tile takes the generic path)

// Tile flags written by the pass-2 kernel and read by k_pv_fix.
constexpr int kTileDone = 0, kTileGeneric = 1;

// ---------------------------------------------------------------- arguments

struct PvArgs {
    PvSrc src;
    const float *rowmax;          // rowmax[bh*rm_rows + i - rm_row0], or null and then
    const uint32_t *rowmax_keys;  // its order keys at the same place
    int64_t rm_rows, rm_row0;
    int64_t ni, i0, kv_lo, kv_hi;
    int64_t Hq, Hkv, group, D, Dp32, nKB;
    int causal;
    const v4i *vsl;
    const int *colgrid, *grpB;
    int *flags;  // [bh][ntiles]: kTileGeneric = the tile is left to the generic path
    int64_t ntiles;
    int force_fallback;
    // fused output
    float *o;
    int64_t osB, osH, osS;
    // digit output (accumulate): num [14][plane_rows][D], den [9][plane_rows]
    int64_t *num, *den;
    int64_t plane_rows, rows_per_bh, row0;
    // the generic path: V itself and (fused) 32-row digit scratch per tile
    const void *v;
    int vdtype;
    int64_t vsB, vsH, vsS;
    int64_t *fb_num, *fb_den;
    // remainders of V entries below their column grids (vprep.hpp)
    const int *rare_n, *rare_grp;
    const int4 *rare;
    // fused, optional: each row's max and RN64(DEN) at [bh * stat_rows + i]
    float *stat_m;
    double *stat_den;
    int64_t stat_rows;
};

// The row max of row i of head bh (from floats or from order keys).
__device__ __forceinline__ float pv_rowmax(const PvArgs &A, int64_t bh, int64_t i) {
    const int64_t at = bh * A.rm_rows + (i - A.rm_row0);
    return A.rowmax_keys ? key_value(A.rowmax_keys[at]) : A.rowmax[at];
}

// The score of query row i and key j of head bh by the rule itself: the
// stored pass-1 score (f32 inputs), or the fp64 fma chain over d ascending
// from +0 of the bf16 rows, then RN32(RN64(scale * dot)).  The rows are read
// 32 dimensions at a time with all of a chunk's loads issued before its
// chain steps (16-byte loads where both rows allow them).
__device__ __forceinline__ float pv_score(const PvArgs &A, int64_t bh, int64_t i, int64_t j) {
    const PvSrc &S = A.src;
    if (S.scores) return S.scores[(bh * A.ni + (i - A.i0)) * S.W + (j - A.kv_lo)];
    const int64_t b = bh / A.Hq, hq = bh % A.Hq, hk = hq / A.group;
    const bf16_t *qr = (const bf16_t *)S.q + b * S.qsB + hq * S.qsH + i * S.qsS;
    const bf16_t *kr = (const bf16_t *)S.k + b * S.ksB + hk * S.ksH + j * S.ksS;
    const int D = (int)A.D;
    double acc = 0.0;
    if (D % 32 == 0 && (((uintptr_t)qr | (uintptr_t)kr) & 15) == 0) {
        for (int d0 = 0; d0 < D; d0 += 32) {
            uint4 qv[4], kv[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                qv[t] = ((const uint4 *)(qr + d0))[t];
                kv[t] = ((const uint4 *)(kr + d0))[t];
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const uint32_t qw[4] = {qv[t].x, qv[t].y, qv[t].z, qv[t].w};
                const uint32_t kw[4] = {kv[t].x, kv[t].y, kv[t].z, kv[t].w};
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    acc = fma((double)__uint_as_float(qw[u] << 16), (double)__uint_as_float(kw[u] << 16), acc);
                    acc = fma((double)__uint_as_float(qw[u] & 0xffff0000u), (double)__uint_as_float(kw[u] & 0xffff0000u),
                              acc);
                }
            }
        }
    } else {
        for (int d = 0; d < D; ++d)
            acc = fma((double)elem<bf16_t>::to_f32(qr[d]), (double)elem<bf16_t>::to_f32(kr[d]), acc);
    }
    return (float)(S.scale * acc);
}

// Weights of KPT consecutive keys of one row for the calling lane, with
// scores sc[]; the first nv of them are visible.  w = RN32(exp_det(s - m)) and
// W = w 2^46 = M << (E + 23) for the f32 w = M 2^(E-23), an integer for
// 2^-23 <= w <= 1 (other nonzero weights set bad).  The six balanced
// base-256 digits of W are the bytes of W + 0x808080808080 with their top bit
// flipped (digit set [-128, 127], the unique such representation).  Digit a of
// the KPT keys goes to dst + a*1024 (MFMA lane order, set up by the caller).
// Returns the mask of digits nonzero for this lane and adds W to wsum.
//
// Every key runs the same instructions: exp_det's cutoff (t < -104 gives 0)
// and the visibility are selects after the arithmetic, on an argument clamped
// to [-105, 1] (equal to t wherever the result is kept; t > 0 only when the
// row max is below a score, and then w > 1 sets bad either way), so the KPT
// exp chains interleave instead of running one after another.
// (GRP: keys whose exponentials run interleaved; fewer hold fewer registers)
// W + 0x808080808080 (U) of KPT keys, key k visible when vis(k); the exp
// chains of GRP keys at a time run interleaved.
template <int KPT, int GRP, class VIS>
__device__ __forceinline__ void block_w(const float (&sc)[KPT], float m, VIS vis, uint64_t (&U)[KPT], int64_t &wsum,
                                        bool &bad) {
    static_assert(KPT % GRP == 0, "whole groups");
#pragma unroll
    for (int g0 = 0; g0 < KPT; g0 += GRP) {
        double t[GRP], n[GRP], r[GRP], p[GRP];
#pragma unroll
        for (int u = 0; u < GRP; ++u) {
            t[u] = (double)sc[g0 + u] - (double)m;
            r[u] = exp_det_reduce(fmin(fmax(t[u], -105.0), 1.0), n[u]);
        }
        exp_det_poly<GRP>(r, p, FmaVreg{});
#pragma unroll
        for (int u = 0; u < GRP; ++u) {
            const float w = (vis(g0 + u) && t[u] >= -104.0) ? (float)ldexp(p[u], (int)n[u]) : 0.0f;
            const uint32_t bits = __float_as_uint(w);
            // 0x34000000 = 2^-23, 0x3f800000 = 1
            if (bits != 0 && (bits < 0x34000000u || bits > 0x3f800000u)) bad = true;
            const uint64_t Wi =
                bits ? ((uint64_t)((bits & 0x7fffffu) | 0x800000u)) << (((bits >> 23) - 104u) & 63u) : 0ull;
            wsum += (int64_t)Wi;
            U[g0 + u] = Wi + 0x808080808080ull;
        }
    }
}

// Plane a's word tw at dst holds byte a of four keys' U: a 4 x 6 byte
// transpose by byte permutes (v_perm_b32 picks any four bytes of its two
// sources: selector byte k in 0..3 names a byte of the second source, 4..7
// one of the first); the flipped words are ORed into any[].
__device__ __forceinline__ void pack_w4(uint64_t u0, uint64_t u1, uint64_t u2, uint64_t u3, int tw, uint8_t *dst,
                                        uint32_t (&any)[kAw]) {
    static_assert(kAw == 6, "six W digit planes");
    const uint32_t L0 = (uint32_t)u0, L1 = (uint32_t)u1, L2 = (uint32_t)u2, L3 = (uint32_t)u3;
    const uint32_t H0 = (uint32_t)(u0 >> 32), H1 = (uint32_t)(u1 >> 32), H2 = (uint32_t)(u2 >> 32),
                   H3 = (uint32_t)(u3 >> 32);
    // bytes 0, 1 (resp. 2, 3) of keys 0 and 1 interleaved, likewise keys 2 and 3
    const uint32_t x01l = __builtin_amdgcn_perm(L1, L0, 0x05010400u), x01h = __builtin_amdgcn_perm(L1, L0, 0x07030602u);
    const uint32_t x23l = __builtin_amdgcn_perm(L3, L2, 0x05010400u), x23h = __builtin_amdgcn_perm(L3, L2, 0x07030602u);
    const uint32_t y01 = __builtin_amdgcn_perm(H1, H0, 0x05010400u), y23 = __builtin_amdgcn_perm(H3, H2, 0x05010400u);
    const uint32_t word[kAw] = {
        __builtin_amdgcn_perm(x23l, x01l, 0x05040100u), __builtin_amdgcn_perm(x23l, x01l, 0x07060302u),
        __builtin_amdgcn_perm(x23h, x01h, 0x05040100u), __builtin_amdgcn_perm(x23h, x01h, 0x07060302u),
        __builtin_amdgcn_perm(y23, y01, 0x05040100u),   __builtin_amdgcn_perm(y23, y01, 0x07060302u)};
#pragma unroll
    for (int a = 0; a < kAw; ++a) {
        const uint32_t wd = word[a] ^ 0x80808080u;
        any[a] |= wd;
        ((uint32_t *)(dst + a * 64 * 16))[tw] = wd;
    }
}

__device__ __forceinline__ uint32_t nonzero_planes(const uint32_t (&any)[kAw]) {
    uint32_t nzm = 0;
#pragma unroll
    for (int a = 0; a < kAw; ++a)
        if (any[a]) nzm |= 1u << a;
    return nzm;
}

template <int KPT, int GRP = KPT>
__device__ __forceinline__ uint32_t block_weights(const float (&sc)[KPT], float m, int nv, uint8_t *dst,
                                                  int64_t &wsum, bool &bad) {
    uint64_t U[KPT];
    block_w<KPT, GRP>(sc, m, [&](int k) { return k < nv; }, U, wsum, bad);
    uint32_t any[kAw] = {};
#pragma unroll
    for (int t = 0; t < KPT / 4; ++t) pack_w4(U[4 * t], U[4 * t + 1], U[4 * t + 2], U[4 * t + 3], t, dst, any);
    return nonzero_planes(any);
}

// The same for the four keys of each of two blocks at once (sc[0..3] with nv0
// visible into dst0, sc[4..7] with nv1 visible into dst1): their eight exp
// chains interleave, which keeps a single wave per SIMD issuing its fp64
// Horner steps closer to their rate.  The two blocks' masks go to nz0, nz1.
__device__ __forceinline__ void block_weights2(const float (&sc)[8], float m, int nv0, int nv1, uint8_t *dst0,
                                               uint8_t *dst1, int64_t &wsum, bool &bad, uint32_t &nz0,
                                               uint32_t &nz1) {
    uint64_t U[8];
    block_w<8, 8>(sc, m, [&](int k) { return k < 4 ? k < nv0 : k - 4 < nv1; }, U, wsum, bad);
    uint32_t a0[kAw] = {}, a1[kAw] = {};
    pack_w4(U[0], U[1], U[2], U[3], 0, dst0, a0);
    pack_w4(U[4], U[5], U[6], U[7], 0, dst1, a1);
    nz0 = nonzero_planes(a0);
    nz1 = nonzero_planes(a1);
}

// OR of a kAw-bit mask over the wave, by one ballot per bit (no LDS traffic).
__device__ __forceinline__ uint32_t wave_or_mask(uint32_t nz) {
    uint32_t r = 0;
#pragma unroll
    for (int a = 0; a < kAw; ++a)
        if (__ballot((nz >> a) & 1u)) r |= 1u << a;
    return r;
}

// K digit rows of one 32-key block in LDS (recomputed scores, ND 64-dim
// chunks per row): each row padded by 16 bytes, so the 16 lanes of a read
// pass fetch 16 different keys from disjoint sets of banks.
template <int ND> struct PvKRow {
    static constexpr int RB = kQKmax * 64 * ND;  // digit bytes of one K (or Q) row
    static constexpr int KROW = RB + 16;
};

// LDS of the pass-2 kernel: W digits of the key blocks in flight (a ring of
// kNDig), K digit rows and key statistics of two blocks (recomputed scores:
// per key its statistics and grid, per 16-key half the largest digit count
// and bound), digit masks, row sums, the bad-tile flag, and the consumers'
// int64 parts of the top class (tiles of 8192 keys or more).  With kept
// scores the weights of two blocks are made together, two blocks ahead of
// the products, and the roles meet every second block (four digit buffers);
// recomputing, one block ahead and every block (two).
template <int ND> struct PvShared {
    static constexpr int kNDig = ND == 0 ? 4 : 2;
    uint8_t dig[kNDig][kAw * 1024];
    uint8_t kd[2][ND > 0 ? 32 * PvKRow<ND>::KROW : 16];
    int4 ki[2][32];
    int kg[2][32];
    int2 kh[2][2];
    // pairs left out of the matrix-core scores (rule outside its bound), per
    // tile parity: count and {row in tile, key - kv_lo}; their chain scores
    // for the extra block being made
    int dn[2];
    int2 dl[2][kDeferCap];
    float dsc[32];
    uint32_t mask[kNDig][kPW];
    // per tile parity, so that a tile's finalize overlaps the next tile's start
    unsigned long long den_hi[2][32], den_lo[2][32];  // exact sum of W per row: hi 2^32 + lo
    double d64[2][32];                                // RN64(DEN) of the row
    int bad[2];
    int64_t top[4][16][64];  // [consumer wave][accumulator register][lane]
};

// Whether the roles of the pass-2 kernel meet (a workgroup barrier) after
// block step kb of nblk: after every step, or with kept scores after the odd
// steps and the last one.  Both roles take this same test.
template <int ND> __device__ __forceinline__ bool pv_meets(int kb, int nblk) {
    return ND > 0 || (kb & 1) != 0 || kb + 1 == nblk;
}

struct PvTile {
    int64_t b, hq, bhk, it0, i_end, nG, jhi;
    int nblk;
    bool badv;     // a V group the grid cannot hold: the whole tile takes the generic path
    uint32_t rem;  // groups with remainders below their grid: finalized through digits
};

__device__ __forceinline__ PvTile pv_tile_of(const PvArgs &A, int64_t bh, int64_t tile) {
    PvTile T;
    T.b = bh / A.Hq;
    T.hq = bh % A.Hq;
    T.bhk = T.b * A.Hkv + T.hq / A.group;
    T.it0 = A.i0 + tile * 32;
    T.i_end = A.i0 + A.ni;
    T.nG = A.Dp32 / 32;
    T.jhi = A.causal ? min64(A.kv_hi, T.it0 + 32) : A.kv_hi;
    T.nblk = T.jhi > A.kv_lo ? (int)((T.jhi - A.kv_lo + kKB - 1) / kKB) : 0;
    int bad = A.force_fallback;
    uint32_t rem = 0;
    for (int64_t g = 0; g < T.nG; ++g) {
        bad |= A.grpB[T.bhk * T.nG + g] > kBmax;
        if (A.rare_grp[T.bhk * T.nG + g]) rem |= 1u << g;
    }
    if (rem && *A.rare_n > kRareCap) bad = 1;  // the list lost entries
    T.badv = bad;
    T.rem = rem;
    return T;
}

}  // namespace det
