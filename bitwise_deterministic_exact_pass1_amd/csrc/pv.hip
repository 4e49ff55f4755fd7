// pv.hip -- pass 2 of the exact softmax on the matrix cores.
//
// The det-attn page ("Method") needs NUM_id = sum_j w_ij V_jd and
// DEN_i = sum_j w_ij exactly.  Both factors are turned into integers on fixed
// grids, split into balanced base-256 digits, and multiplied on the int8
// matrix cores, which add exactly in int32:
//
//   W_ij = w_ij * 2^46                 (an integer when w >= 2^-23: 24-bit mantissa)
//   Vi_jd = V_jd * 2^-g_d              (g_d = the smallest lsb exponent in column d)
//   W = sum_a c_a 256^a,  Vi = sum_b e_b 256^b,  c, e in [-128, 127]
//   NUM_id = 2^(g_d - 46) * sum_s 256^s * C_s[i][d],  C_s = sum_{a+b=s} sum_j c_a(W_ij) e_b(Vi_jd)
//
// v_mfma_i32_32x32x32_i8 computes one C_s update for a 32-row x 32-dim tile
// over 32 keys.  Every int32 partial sum is exact (|c e| <= 2^14 per key and
// pair; every 8192 keys the classes are carried into each other and the top
// class, which nothing above it absorbs, is moved into an int64 in LDS), so
// the result is the exact NUM whatever the order of keys, blocks or
// instructions, for any key range the launcher admits.  DEN is the exact sum
// of the W_ij, kept per thread in int64 halves that are folded every 8192
// keys and added up per row in 128 bits.  A tile whose weights do not fit the
// grid (w < 2^-23, or w > 1 from a rowmax below the scores) or whose V columns
// need more than five digits is redone by the generic exact path (windowed
// binary64 sums into digit planes) by the same workgroup: results never depend
// on which path ran.
#include "dev_math.hpp"
#include "kernels.hpp"
#include "vprep.hpp"

#include <algorithm>

namespace det {

typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kAw = 6;                  // digits of W
constexpr int kSw = 8 * kAw - 2;        // W = w * 2^46, |W| <= 2^46 fits six balanced digits
constexpr int kNC = kAw + kBmax - 1;    // shift classes s = a + b
constexpr int kCarryEvery = 256;        // blocks (8192 keys) between carry passes

// ---------------------------------------------------------------- V preparation

// Standalone launches of the V preparation (vprep.hpp): grid (chunk, group,
// head) for the statistics, (block, group, head) for the digit slices.
template <typename TV>
__global__ __launch_bounds__(256) void k_vstats(VJob J) {
    vstats_block<TV>(J, blockIdx.x, blockIdx.y, blockIdx.z);
}
template <typename TV>
__global__ __launch_bounds__(64) void k_vslice(VJob J) {
    vslice_block<TV>(J, blockIdx.x, blockIdx.y, blockIdx.z, threadIdx.x);
}

// ---------------------------------------------------------------- the MFMA kernels

struct PvArgs {
    const float *scores;  // [bh][ni][W] chunk scores
    const float *rowmax;          // rowmax[bh*rm_rows + i - rm_row0], or null and then
    const uint32_t *rowmax_keys;  // its order keys at the same place
    int64_t rm_rows, rm_row0;
    int64_t ni, W, i0, kv_lo, kv_hi;
    int64_t Hq, Hkv, group, D, Dp32, nKB;
    int causal;
    const v4i *vsl;
    const int *colgrid, *grpB;
    int *flags;  // [bh][ntiles]: 1 = the tile is left to the generic path
    int64_t ntiles;
    int force_fallback;
    // fused output
    float *o;
    int64_t osB, osH, osS;
    // digit output (accumulate): num [14][plane_rows][D], den [9][plane_rows]
    int64_t *num, *den;
    int64_t plane_rows, rows_per_bh, row0;
    // the generic path of flagged tiles: V itself and (fused) 32-row digit scratch per tile
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


// Weights of one 32-key block for the calling thread: KPT consecutive keys of
// one row with scores sc[]; the first nv of them are visible.  w =
// RN32(exp_det(s - m)) and W = w 2^46 = M << (E + 23) for the f32 w =
// M 2^(E-23), an integer for 2^-23 <= w <= 1 (other nonzero weights set bad).
// The six balanced base-256 digits of W are the bytes of W + 0x808080808080
// with their top bit flipped (digit set [-128, 127], the unique such
// representation).  Digit a of the KPT keys goes to dst + a*1024 (MFMA lane
// order, set up by the caller).  Returns the mask of digits nonzero for this
// thread and adds W to wsum.
//
// Every key runs the same instructions: exp_det's cutoff (t < -104 gives 0)
// and the visibility are selects after the arithmetic, on an argument clamped
// to [-105, 1] (equal to t wherever the result is kept; t > 0 only when the
// row max is below a score, and then w > 1 sets bad either way), so the KPT
// exp chains interleave instead of running one after another.
template <int KPT>
__device__ __forceinline__ uint32_t block_weights(const float (&sc)[KPT], float m, int nv, uint8_t *dst,
                                                  int64_t &wsum, bool &bad) {
    double t[KPT], n[KPT], r[KPT], p[KPT];
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
        t[u] = (double)sc[u] - (double)m;
        r[u] = exp_det_reduce(fmin(fmax(t[u], -105.0), 1.0), n[u]);
    }
    exp_det_poly<KPT>(r, p, FmaVreg{});
    uint64_t U[KPT];
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
        const float w = (u < nv && t[u] >= -104.0) ? (float)ldexp(p[u], (int)n[u]) : 0.0f;
        const uint32_t bits = __float_as_uint(w);
        // 0x34000000 = 2^-23, 0x3f800000 = 1
        if (bits != 0 && (bits < 0x34000000u || bits > 0x3f800000u)) bad = true;
        const uint64_t Wi =
            bits ? ((uint64_t)((bits & 0x7fffffu) | 0x800000u)) << (((bits >> 23) - 104u) & 63u) : 0ull;
        wsum += (int64_t)Wi;
        U[u] = Wi + 0x808080808080ull;
    }
    uint32_t nzm = 0;
#pragma unroll
    for (int a = 0; a < kAw; ++a) {
        uint32_t word[KPT / 4] = {};
#pragma unroll
        for (int u = 0; u < KPT; ++u) word[u / 4] |= ((uint32_t)(U[u] >> (8 * a)) & 255u) << (8 * (u % 4));
        uint32_t any = 0;
#pragma unroll
        for (int t = 0; t < KPT / 4; ++t) {
            word[t] ^= 0x80808080u;
            any |= word[t];
            ((uint32_t *)(dst + a * 64 * 16))[t] = word[t];
        }
        if (any) nzm |= 1u << a;
    }
    return nzm;
}

constexpr int kPW = 4;  // producer waves of the pass-2 kernel

// OR of a kAw-bit mask over the wave, by one ballot per bit (no LDS traffic).
__device__ __forceinline__ uint32_t wave_or_mask(uint32_t nz) {
    uint32_t r = 0;
#pragma unroll
    for (int a = 0; a < kAw; ++a)
        if (__ballot((nz >> a) & 1u)) r |= 1u << a;
    return r;
}

// LDS of the pass-2 kernel: W digits of two key blocks, the producers'
// staged scores of two blocks, digit masks, row sums, the bad-tile flag, and
// the consumers' int64 parts of the top class (tiles of 8192 keys or more).
struct PvShared {
    uint8_t dig[2][kAw * 1024];
    float sc[2][32][32];
    uint32_t mask[2][kPW];
    // per tile parity, so that a tile's finalize overlaps the next tile's start
    int64_t den_hi[2][32], den_lo[2][32];  // exact sum of W per row: hi 2^32 + lo, lo in [0, 2^32)
    double d64[2][32];   // RN64(DEN) of the row
    int bad[2];
    int64_t top[4][16][64];  // [consumer wave][accumulator register][lane]
};

// Pass 2 of a 32-row tile for the 32-dim groups G0 .. G0+NG-1.
//
// NG consumer waves, one per group, run C_s += W_a x V_b (s = a + b) on the
// matrix cores, with their V digits fetched from global memory one block
// ahead; kPW producer waves turn the next 32-key block's scores into W
// digits in LDS meanwhile (double buffered, one barrier per block).  The two
// roles run separate code with the same barriers, so the weight arithmetic on
// the vector ALUs overlaps the matrix-core work and neither role's registers
// are held in the other.  Producers stage the scores of the block after next
// in LDS, so every global load has a whole block of arithmetic to arrive in.
// DEN (the exact sum of W per row) stays in the producers' registers.  At the
// end the consumers finalize the exact NUM and DEN to o or add them into
// digit planes.  A tile whose weights or V columns do not fit the grids is
// flagged for the generic path and produces no output here.

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

// Producer side of one tile: thread ptid of the kPW producer waves.
// Returns whether the tile needs the generic path (known to both roles after
// the tile's last barrier).
template <int NG>
__device__ __forceinline__ bool pv_produce(const PvArgs &A, int64_t bh, int64_t tile, int ptid, int par,
                                           PvShared &S, uint32_t &rem) {
    constexpr int NPT = 64 * kPW;  // producer threads
    constexpr int TPR = NPT / 32;  // producer threads per row
    constexpr int KPT = 32 / TPR;  // keys per producer thread and block
    const PvTile T = pv_tile_of(A, bh, tile);
    rem = T.rem;
    if (T.badv) return true;
    const int lane = ptid & 63, pw = ptid >> 6;
    const int r = ptid / TPR, k0 = (ptid % TPR) * KPT;
    const int dofs = ((r + 32 * (k0 >> 4)) * 16) + (k0 & 15);
    const int64_t i = T.it0 + r;
    const bool rowok = i < T.i_end;
    const float m = rowok ? pv_rowmax(A, bh, i) : 0.0f;
    // keys this row sees: [kv_lo, jend), counted from this thread's first key
    // kv_lo + k0 (32-bit: the launcher bounds the key range)
    const int64_t jend = rowok ? (A.causal ? min64(T.jhi, i + 1) : T.jhi) : A.kv_lo;
    const int vis0 = (int)(jend - A.kv_lo - k0);
    auto nvis = [&](int kb) {  // visible keys among this thread's KPT keys of block kb
        return max(0, min(KPT, vis0 - kb * kKB));
    };
    // The tile's scores through a buffer resource based at its first row: key
    // kv_lo + j of row r at byte (r W + j) 4.  A lane's offset is fixed and the
    // block step is the scalar offset, so a load needs no address registers.
    // Keys past a row's end read the next row or, past the scores array, zero
    // (buffer bounds); those keys are invisible and their weights discarded.
    const int64_t row_first = bh * A.ni + (T.it0 - A.i0);
    const int64_t bytes_left = ((int64_t)gridDim.y * A.ni - row_first) * A.W * 4;
    const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(A.scores + row_first * A.W), (short)0, (int)min64(bytes_left, INT32_MAX), 0x00020000);
    const int voff = (r * (int)A.W + k0) * 4;
    auto load_scores = [&](int kb, float (&x)[KPT]) {
#pragma unroll
        for (int u = 0; u < KPT; ++u)
            x[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(srs, voff + 4 * u, kb * kKB * 4, 0));
    };
    float *my0 = &S.sc[0][r][k0], *my1 = &S.sc[1][r][k0];
    // this thread's sum of W: whi 2^32 + wsum; wsum grows by at most KPT 2^46
    // per block and is folded into whi every kCarryEvery blocks (< 2^57 between)
    int64_t wsum = 0, whi = 0;
    bool bad = false;
    // Scores travel three blocks ahead of their use: loaded into registers,
    // parked in this thread's LDS slots one block later, read the block after.
    float pend[KPT];
    if (T.nblk > 0) {
        float sc[KPT], s1[KPT];
        load_scores(0, sc);
        load_scores(1, s1);
        load_scores(2, pend);
        const uint32_t nz = wave_or_mask(block_weights<KPT>(sc, m, nvis(0), S.dig[0] + dofs, wsum, bad));
        if (lane == 0) S.mask[0][pw] = nz;
#pragma unroll
        for (int u = 0; u < KPT; ++u) my1[u] = s1[u];
    }
    __syncthreads();
    // One block step: weights of block kb+1 into the digit buffer the consumers
    // read next, scores of block kb+3 into `load`, block kb+2's scores (`park`,
    // loaded one step earlier) into this thread's LDS slots.  The loop is
    // unrolled by two so that the two register sets swap roles without copies
    // (a copy of a register still being loaded would wait for the load).
    auto step = [&](int kb, float (&park)[KPT], float (&load)[KPT]) {
        const int nb = (kb & 1) ^ 1;
        if (kb + 1 < T.nblk) {
            float sc[KPT];
            load_scores(kb + 3, load);
            const float *cur = nb ? my1 : my0;
#pragma unroll
            for (int u = 0; u < KPT; ++u) sc[u] = cur[u];
            const uint32_t nz = wave_or_mask(block_weights<KPT>(sc, m, nvis(kb + 1), S.dig[nb] + dofs, wsum, bad));
            if (lane == 0) S.mask[nb][pw] = nz;
            if (((kb + 1) % kCarryEvery) == 0) {
                whi += wsum >> 32;
                wsum &= 0xffffffffll;
            }
            float *nxt = nb ? my0 : my1;  // block kb+2 uses buffer (kb+2)&1
#pragma unroll
            for (int u = 0; u < KPT; ++u) nxt[u] = park[u];
        }
        __syncthreads();
    };
    float pend2[KPT];
    for (int kb = 0; kb < T.nblk; kb += 2) {
        step(kb, pend, pend2);
        if (kb + 1 < T.nblk) step(kb + 1, pend2, pend);
    }
    // exact row sums of W: the TPR threads of a row are consecutive lanes
    // (each wsum < 2^57, so their sum fits; whi counts units of 2^32)
#pragma unroll
    for (int off = 1; off < TPR; off <<= 1) {
        wsum += __shfl_xor(wsum, off, 64);
        whi += __shfl_xor(whi, off, 64);
    }
    if (ptid % TPR == 0) {
        const int64_t hi = whi + (wsum >> 32), lo = wsum & 0xffffffffll;  // DEN 2^46 = hi 2^32 + lo
        S.den_hi[par][r] = hi;
        S.den_lo[par][r] = lo;
        // correctly rounded RN64(DEN): the 128-bit value (hi >> 32) 2^64 + ((hi << 32) | lo)
        S.d64[par][r] = i128_to_f64(hi >> 32, ((uint64_t)hi << 32) | (uint64_t)lo, -kSw);
    }
    if (bad) S.bad[par] = 1;
    __syncthreads();
    const bool generic = S.bad[par] != 0;
    if (A.stat_den && !generic && rowok && ptid % TPR == 0) {  // (generic tiles write theirs there)
        A.stat_den[bh * A.stat_rows + i] = S.d64[par][r];
        A.stat_m[bh * A.stat_rows + i] = m;
    }
    return generic;
}

// The consumer's block loop for a wave whose group has BV V digits (0: no
// group, barriers only).  Per block: the six W digit fragments of the block
// are read from LDS up front, the next block's V digits are fetched into the
// other register set (the loop is unrolled by two so the sets swap roles
// without copies), and the class sums C_(a+b) += W_a x V_b run on the matrix
// cores for the W digit planes the producers marked nonzero.
template <int BV>
__device__ __forceinline__ void pv_consume_loop(const PvTile &T, const v4i *vb, int lane, int wave, v16i (&C)[kNC],
                                                PvShared &S) {
    v4i VA[BV > 0 ? BV : 1], VB[BV > 0 ? BV : 1];
    if (BV > 0 && T.nblk > 0) {
#pragma unroll
        for (int s = 0; s < BV; ++s) VA[s] = vb[s * 64];
    }
    __syncthreads();
    auto step = [&](int kb, const v4i (&cur)[BV > 0 ? BV : 1], v4i (&nxt)[BV > 0 ? BV : 1]) {
        if (BV > 0) {
            const int buf = kb & 1;
            if (kb + 1 < T.nblk) {
#pragma unroll
                for (int s = 0; s < BV; ++s) nxt[s] = vb[((int64_t)(kb + 1) * kBmax + s) * 64];
            }
            const uint8_t *dg = S.dig[buf] + lane * 16;
            uint32_t mask = 0;
#pragma unroll
            for (int w = 0; w < kPW; ++w) mask |= S.mask[buf][w];
            mask = __builtin_amdgcn_readfirstlane(mask);
            // W digit a+1 is read while digit a's products run
            v4i Acur = *(const v4i *)dg;
#pragma unroll
            for (int a = 0; a < kAw; ++a) {
                const v4i Anext = *(const v4i *)(dg + ((a + 1) % kAw) * 1024);
                if (mask & (1u << a)) {
#pragma unroll
                    for (int s = 0; s < BV; ++s)
                        C[a + s] = __builtin_amdgcn_mfma_i32_32x32x32_i8(Acur, cur[s], C[a + s], 0, 0, 0);
                }
                Acur = Anext;
            }
            if ((kb % kCarryEvery) == kCarryEvery - 1) {
                // carry each class into the next so every partial sum stays far below 2^31,
                // and move the top class into its int64 part in LDS (wave-private slots)
#pragma unroll
                for (int s = 0; s < kNC - 1; ++s) {
                    const v16i c = C[s] >> 8;
                    C[s] -= c << 8;
                    C[s + 1] += c;
                }
#pragma unroll
                for (int rr = 0; rr < 16; ++rr) S.top[wave][rr][lane] += C[kNC - 1][rr];
                C[kNC - 1] = v16i{0};
            }
        }
        __syncthreads();
    };
    for (int kb = 0; kb < T.nblk; kb += 2) {
        step(kb, VA, VB);
        if (kb + 1 < T.nblk) step(kb + 1, VB, VA);
    }
}

// Consumer side of one tile: wave `wave` (< NG) owns 32-dim group G0 + wave.
// Returns whether the tile needs the generic path.
template <bool FUSED, int NG>
__device__ __forceinline__ bool pv_consume(const PvArgs &A, int G0, int64_t bh, int64_t tile, int wave, int par,
                                           PvShared &S, uint32_t &rem) {
    const int tid = threadIdx.x, lane = tid & 63;
    const PvTile T = pv_tile_of(A, bh, tile);
    rem = T.rem;
    if (T.badv) {
        if (tid == 0) A.flags[bh * A.ntiles + tile] = 1;
        return true;
    }
    if (tid == 0) S.bad[par] = 0;
    const int64_t G = G0 + wave;
    const bool mine = G < T.nG;
    const int Bv = mine ? A.grpB[T.bhk * T.nG + G] : 0;
    const v4i *vb = A.vsl + ((T.bhk * T.nG + (mine ? G : 0)) * A.nKB) * kBmax * 64 + lane;
    v16i C[kNC];
#pragma unroll
    for (int s = 0; s < kNC; ++s) C[s] = v16i{0};
    // the top class's int64 part, used by tiles of kCarryEvery blocks or more
    const bool longt = T.nblk >= kCarryEvery;
    if (longt) {
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) S.top[wave][rr][lane] = 0;
    }
    // the block loop with the wave's V digit count as a constant (one copy per
    // count; a wave without a group only meets the barriers)
    switch (mine ? Bv : 0) {
        case 1: pv_consume_loop<1>(T, vb, lane, wave, C, S); break;
        case 2: pv_consume_loop<2>(T, vb, lane, wave, C, S); break;
        case 3: pv_consume_loop<3>(T, vb, lane, wave, C, S); break;
        case 4: pv_consume_loop<4>(T, vb, lane, wave, C, S); break;
        case 5: pv_consume_loop<5>(T, vb, lane, wave, C, S); break;
        default: pv_consume_loop<0>(T, vb, lane, wave, C, S); break;
    }
    __syncthreads();
    if (S.bad[par]) {
        if (tid == 0) A.flags[bh * A.ntiles + tile] = 1;
        return true;
    }
    if (tid == 0) A.flags[bh * A.ntiles + tile] = 0;
    if (!mine) return false;

    // carry the classes into bytes: C_0..C_8 in [0, 256), C_9 signed, so that
    // NUM = top 2^72 + sum_{s<9} C_s 2^(8s) = hi 2^64 + lo, with top = C_9
    // plus its int64 part from LDS
#pragma unroll
    for (int s = 0; s < kNC - 1; ++s) {
        const v16i c = C[s] >> 8;
        C[s] &= 255;
        C[s + 1] += c;
    }
    // the top class of accumulator register rr, with its int64 part
    auto top = [&](int rr) -> int64_t {
        return (int64_t)C[kNC - 1][rr] + (longt ? S.top[wave][rr][lane] : 0);
    };
    const int64_t d = G * 32 + (lane & 31);
    const int g = A.colgrid[T.bhk * A.Dp32 + d];
    if (FUSED && ((T.rem >> G) & 1)) {
        // this group's remainders are added later: its exact NUM goes to the
        // tile's 32-row digit scratch (cleared here), finalized after them
        const int64_t nplane = A.ntiles * 32 * (int64_t)gridDim.y * A.D;
        int64_t *nb = A.fb_num + (bh * A.ntiles + tile) * 32 * A.D;
        for (int t = lane; t < 32 * 32 * kNumDigits; t += 64) {
            const int k = t >> 10, r = (t >> 5) & 31, c = t & 31;
            if (G * 32 + c < A.D) nb[k * nplane + r * A.D + G * 32 + c] = 0;
        }
        __threadfence();
        if (d < A.D) {
#pragma unroll 1
            for (int rr = 0; rr < 16; ++rr) {
                const int row = 8 * (rr >> 2) + 4 * (lane >> 5) + (rr & 3);
                const uint32_t l0 = (uint32_t)C[0][rr] | ((uint32_t)C[1][rr] << 8) |
                                    ((uint32_t)C[2][rr] << 16) | ((uint32_t)C[3][rr] << 24);
                const uint32_t l1 = (uint32_t)C[4][rr] | ((uint32_t)C[5][rr] << 8) |
                                    ((uint32_t)C[6][rr] << 16) | ((uint32_t)C[7][rr] << 24);
                const uint64_t lo = ((uint64_t)l1 << 32) | l0;
                const int64_t hi = top(rr) * 256 + C[kNC - 2][rr];
                const __int128 num = (__int128)(((unsigned __int128)(uint64_t)hi << 64) | lo);
                add_i128_digits<kNumDigits>(num, g - kSw - kNumElo, nb + row * A.D + d, nplane);
            }
        }
        __threadfence();
        return false;
    }
    if (FUSED) {
        // all 16 outputs of the lane first (no branches: their conversions and
        // divisions interleave), then the stores of the rows that exist
        // NUM = P_hi 2^48 + P_lo with P_lo = bytes C_0..C_5 (48 bits) and
        // P_hi = C_9 2^24 + bytes C_8 C_7 C_6: both exact in binary64 while
        // |P_hi| < 2^53, and then fma(P_hi, 2^48, P_lo) is the correctly rounded
        // NUM (one rounding).  A lane holding a larger P_hi redoes its outputs
        // by the 128-bit conversion.
        float out[16];
        bool big = false;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            const int row = 8 * (rr >> 2) + 4 * (lane >> 5) + (rr & 3);
            const uint64_t plo = (uint64_t)((uint32_t)C[0][rr] | ((uint32_t)C[1][rr] << 8) |
                                            ((uint32_t)C[2][rr] << 16) | ((uint32_t)C[3][rr] << 24)) |
                                 ((uint64_t)((uint32_t)C[4][rr] | ((uint32_t)C[5][rr] << 8)) << 32);
            const int64_t phi = top(rr) * (1 << 24) +
                                (int64_t)((uint32_t)C[6][rr] | ((uint32_t)C[7][rr] << 8) | ((uint32_t)C[8][rr] << 16));
            big |= (uint64_t)(phi + ((int64_t)1 << 53)) >= ((uint64_t)1 << 54);
            const double n64 = ldexp(fma((double)phi, 0x1p48, (double)plo), g - kSw);
            out[rr] = (float)(n64 / S.d64[par][row]);
        }
        if (big) {
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                const int row = 8 * (rr >> 2) + 4 * (lane >> 5) + (rr & 3);
                const uint32_t l0 = (uint32_t)C[0][rr] | ((uint32_t)C[1][rr] << 8) | ((uint32_t)C[2][rr] << 16) |
                                    ((uint32_t)C[3][rr] << 24);
                const uint32_t l1 = (uint32_t)C[4][rr] | ((uint32_t)C[5][rr] << 8) | ((uint32_t)C[6][rr] << 16) |
                                    ((uint32_t)C[7][rr] << 24);
                const uint64_t lo = ((uint64_t)l1 << 32) | l0;
                const int64_t hi = top(rr) * 256 + C[kNC - 2][rr];
                out[rr] = (float)(i128_to_f64(hi, lo, g - kSw) / S.d64[par][row]);
            }
        }
        // keep the arithmetic here, ahead of the guarded stores (else it is
        // moved into each store's branch and the outputs run one after another)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) asm volatile("" ::"v"(out[rr]));
        // the tile's output rows from a wave-uniform base, 32-bit lane offsets
        // (the launcher bounds 32 rows of output stride)
        float *ob = A.o + T.b * A.osB + T.hq * A.osH + T.it0 * A.osS;
        const int nrows = (int)min64(32, T.i_end - T.it0), ostride = (int)A.osS;
        const bool dok = d < A.D;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            const int row = 8 * (rr >> 2) + 4 * (lane >> 5) + (rr & 3);
            if (row < nrows && dok) ob[row * ostride + (int)d] = out[rr];
        }
        return false;
    }
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
        const int row = 8 * (rr >> 2) + 4 * (lane >> 5) + (rr & 3);
        const int64_t io = T.it0 + row;
        if (io >= T.i_end || d >= A.D) continue;
        const uint32_t l0 = (uint32_t)C[0][rr] | ((uint32_t)C[1][rr] << 8) | ((uint32_t)C[2][rr] << 16) |
                            ((uint32_t)C[3][rr] << 24);
        const uint32_t l1 = (uint32_t)C[4][rr] | ((uint32_t)C[5][rr] << 8) | ((uint32_t)C[6][rr] << 16) |
                            ((uint32_t)C[7][rr] << 24);
        const uint64_t lo = ((uint64_t)l1 << 32) | l0;
        const int64_t hi = top(rr) * 256 + C[kNC - 2][rr];
        const __int128 num = (__int128)(((unsigned __int128)(uint64_t)hi << 64) | lo);
        const int64_t prow = bh * A.rows_per_bh + (io - A.row0);
        add_i128_digits<kNumDigits>(num, g - kSw - kNumElo, A.num + prow * A.D + d, A.plane_rows * A.D);
        if (G == 0 && (lane & 31) == 0)
            add_i128_digits<kDenDigits>(((__int128)S.den_hi[par][row] << 32) + S.den_lo[par][row], -kSw - kDenElo,
                                        A.den + prow, A.plane_rows);
    }
    return false;
}

// One workgroup per tile, or for causal attention per pair of tiles (x,
// ntiles-1-x), whose key counts add up to the same total for every pair: the
// whole grid then runs in one balanced round.  Both roles walk the same tiles
// and meet at the same barriers.
template <typename TV, bool FUSED>
__device__ __forceinline__ void fallback_tile(const PvArgs &A, const TV *__restrict__ vp, int64_t vsB, int64_t vsH, int64_t vsS,
                              int64_t *__restrict__ num_ws, int64_t *__restrict__ den_ws, int64_t bh, int64_t tile,
                              int64_t nbh);

// A flagged tile, by the whole workgroup right after both roles learn of it
// (the launch over the first four groups only: it covers every dimension).
template <bool FUSED>
__device__ __forceinline__ void pv_generic_tile(const PvArgs &A, int64_t bh, int64_t tile) {
    if (A.vdtype == 0)
        fallback_tile<float, FUSED>(A, (const float *)A.v, A.vsB, A.vsH, A.vsS, A.fb_num, A.fb_den, bh, tile,
                                    (int64_t)gridDim.y);
    else
        fallback_tile<bf16_t, FUSED>(A, (const bf16_t *)A.v, A.vsB, A.vsH, A.vsS, A.fb_num, A.fb_den, bh, tile,
                                     (int64_t)gridDim.y);
}

// The remainders of a tile's groups G0 .. G0+NG-1 (V entries with bits below
// their column grid, vprep.hpp), by the whole workgroup after both roles are
// done: each visible (row, remainder) product w V_rem is exact in binary64 and
// is added into the row's digits (the caller's planes, or the tile's scratch,
// where the consumers left the matrix-core part of those groups), then (fused)
// those groups' outputs are finalized from the digits.  grp: the groups of
// this launch that have remainders (nonzero, the same for every thread).
template <bool FUSED, int NG>
__device__ __forceinline__ void pv_remainder_tile(const PvArgs &A, int G0, int64_t bh, int64_t tile, int par,
                                                  uint32_t grp, PvShared &S) {
    const PvTile T = pv_tile_of(A, bh, tile);
    __syncthreads();  // the consumers' scratch deposits of this tile are done (and fenced)
    int64_t *num = FUSED ? A.fb_num : A.num;
    const int64_t nplane_rows = FUSED ? A.ntiles * 32 * (int64_t)gridDim.y : A.plane_rows;
    auto prow_of = [&](int64_t i) -> int64_t {
        return FUSED ? (bh * A.ntiles + tile) * 32 + (i - T.it0) : bh * A.rows_per_bh + (i - A.row0);
    };
    const int n = min(*A.rare_n, kRareCap);
    for (int t = threadIdx.x; t < n * 32; t += blockDim.x) {
        const int4 E = A.rare[t >> 5];
        const int64_t i = T.it0 + (t & 31), j = E.y, d = E.z;
        const int gd = E.z / 32 - G0;  // the entry's group within this launch
        if (E.x != T.bhk || gd < 0 || gd >= NG || !((grp >> gd) & 1) || i >= T.i_end) continue;
        const int64_t jend = A.causal ? min64(A.kv_hi, i + 1) : A.kv_hi;
        if (j < A.kv_lo || j >= jend) continue;
        const float w = weight(A.scores[(bh * A.ni + (i - A.i0)) * A.W + (j - A.kv_lo)], pv_rowmax(A, bh, i));
        if (w == 0.0f) continue;
        const float rv = __int_as_float(E.w);
        const int ew = f32_exp(w), ev = f32_exp(rv);
        int64_t *dst = num + prow_of(i) * A.D + d;
        Window win;
        win.init();
        win.add<kNumDigits>((double)w * (double)rv, max(ew, -126) - 23 + max(ev, -126) - 23, ew + ev + 2, kNumGcap,
                            kNumElo, dst, nplane_rows * A.D);
        win.flush<kNumDigits>(kNumElo, dst, nplane_rows * A.D);
    }
    __threadfence();
    __syncthreads();
    if (!FUSED) return;
    for (int t = threadIdx.x; t < 32 * NG * 32; t += blockDim.x) {
        const int r = t / (NG * 32), c = t % (NG * 32);
        const int64_t d = G0 * 32 + c, i = T.it0 + r;
        if (!((grp >> (c >> 5)) & 1) || d >= A.D || i >= T.i_end) continue;
        const int64_t at = prow_of(i) * A.D + d;
        int64_t nd[kNumDigits];
        unsigned long long *np = (unsigned long long *)num;
#pragma unroll
        for (int k = 0; k < kNumDigits; ++k) nd[k] = (int64_t)atomicAdd(np + k * nplane_rows * A.D + at, 0ull);
        canonicalize<kNumDigits>(nd);
        const double n64 = digits_to_f64<kNumDigits>(nd, kNumElo);
        A.o[T.b * A.osB + T.hq * A.osH + i * A.osS + d] = (float)(n64 / S.d64[par][r]);
    }
}

template <bool FUSED, int NG>
__global__ __launch_bounds__(64 * (NG + kPW), 2) void k_pv(PvArgs A, int G0) {
    __shared__ __align__(16) PvShared S;
    const int64_t bh = blockIdx.y, x = blockIdx.x;
    const int npass = (A.causal && x != A.ntiles - 1 - x) ? 2 : 1;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // No barrier between the tiles: the producers start the second tile while
    // the consumers finalize the first (row sums and flags are kept per tile).
    // Both roles learn whether a tile needs the generic path; such tiles are
    // redone at the end by the whole workgroup (from one call site).
    bool generic[2] = {false, false};
    uint32_t rem[2] = {0u, 0u};
    if (wave >= NG) {
        for (int pass = 0; pass < npass; ++pass)
            generic[pass] = pv_produce<NG>(A, bh, (A.causal && pass == 0) ? A.ntiles - 1 - x : x,
                                           threadIdx.x - 64 * NG, pass, S, rem[pass]);
    } else {
        for (int pass = 0; pass < npass; ++pass)
            generic[pass] = pv_consume<FUSED, NG>(A, G0, bh, (A.causal && pass == 0) ? A.ntiles - 1 - x : x, wave,
                                                  pass, S, rem[pass]);
    }
    for (int pass = 0; pass < npass; ++pass) {
        const int64_t tile = (A.causal && pass == 0) ? A.ntiles - 1 - x : x;
        const uint32_t grp = (rem[pass] >> G0) & ((1u << NG) - 1);
        if (generic[pass]) {
            if (G0 == 0) pv_generic_tile<FUSED>(A, bh, tile);
        } else if (grp) {
            pv_remainder_tile<FUSED, NG>(A, G0, bh, tile, pass, grp, S);
        }
    }
}

// ---------------------------------------------------------------- generic exact fallback

// One flagged tile, by the whole workgroup: the windowed exact deposit of the
// general path over all keys of the tile's rows, then (fused) an in-kernel
// finalize.  nbh = number of heads in the launch.
template <typename TV, bool FUSED>
__device__ __forceinline__ void fallback_tile(const PvArgs &A, const TV *__restrict__ vp, int64_t vsB, int64_t vsH, int64_t vsS,
                              int64_t *__restrict__ num_ws, int64_t *__restrict__ den_ws, int64_t bh, int64_t tile,
                              int64_t nbh) {
    const int64_t b = bh / A.Hq, hq = bh % A.Hq, hk = hq / A.group;
    const int64_t it0 = A.i0 + tile * 32, i_end = A.i0 + A.ni;
    const int64_t D = A.D;
    constexpr int VMB = elem<TV>::mant_bits;
    // digit target: fused -> 32-row scratch of this tile (zeroed here); digits -> caller planes
    int64_t *num = FUSED ? num_ws : A.num;
    int64_t *den = FUSED ? den_ws : A.den;
    const int64_t nplane_rows = FUSED ? A.ntiles * 32 * nbh : A.plane_rows;
    auto prow_of = [&](int64_t i) -> int64_t {
        return FUSED ? (bh * A.ntiles + tile) * 32 + (i - it0) : bh * A.rows_per_bh + (i - A.row0);
    };
    if (FUSED) {
        for (int64_t t = threadIdx.x; t < 32 * D * kNumDigits; t += blockDim.x) {
            const int64_t k = t / (32 * D), rem = t % (32 * D);
            num[k * nplane_rows * D + prow_of(it0) * D + rem] = 0;
        }
        for (int64_t t = threadIdx.x; t < 32 * kDenDigits; t += blockDim.x)
            den[(t / 32) * nplane_rows + prow_of(it0) + (t % 32)] = 0;
        __threadfence();
        __syncthreads();
    }
    for (int64_t t = threadIdx.x; t < 32 * (D + 1); t += blockDim.x) {
        const int64_t r = t / (D + 1), d = t % (D + 1);  // d == D: the DEN window of row r
        const int64_t i = it0 + r;
        if (i >= i_end) continue;
        const int64_t row = bh * A.ni + (i - A.i0);
        const float m = pv_rowmax(A, bh, i);
        const int64_t jend = A.causal ? min64(A.kv_hi, i + 1) : A.kv_hi;
        const TV *vcol = vp + b * vsB + hk * vsH + (d < D ? d : 0);
        const int64_t prow = prow_of(i);
        Window win;
        win.init();
        for (int64_t j = A.kv_lo; j < jend; ++j) {
            const float w = weight(A.scores[row * A.W + (j - A.kv_lo)], m);
            if (w == 0.0f) continue;
            const int ew = f32_exp(w);
            const int lw = max(ew, -126) - 23;
            if (d == D) {
                win.add<kDenDigits>((double)w, lw, ew + 1, kDenGcap, kDenElo, den + prow, nplane_rows);
            } else {
                const float vf = elem<TV>::to_f32(vcol[j * vsS]);
                if (vf == 0.0f) continue;
                const int ev = f32_exp(vf);
                win.add<kNumDigits>((double)w * (double)vf, lw + max(ev, -126) - VMB, ew + ev + 2, kNumGcap,
                                    kNumElo, num + prow * D + d, nplane_rows * D);
            }
        }
        if (d == D) win.flush<kDenDigits>(kDenElo, den + prow, nplane_rows);
        else win.flush<kNumDigits>(kNumElo, num + prow * D + d, nplane_rows * D);
    }
    if (!FUSED) return;
    __threadfence();
    __syncthreads();
    for (int64_t t = threadIdx.x; t < 32 * D; t += blockDim.x) {
        const int64_t r = t / D, d = t % D, i = it0 + r;
        if (i >= i_end) continue;
        const int64_t prow = prow_of(i);
        int64_t nd[kNumDigits], dd[kDenDigits];
        unsigned long long *np = (unsigned long long *)num, *dp = (unsigned long long *)den;
#pragma unroll
        for (int k = 0; k < kNumDigits; ++k) nd[k] = (int64_t)atomicAdd(np + k * nplane_rows * D + prow * D + d, 0ull);
#pragma unroll
        for (int k = 0; k < kDenDigits; ++k) dd[k] = (int64_t)atomicAdd(dp + k * nplane_rows + prow, 0ull);
        canonicalize<kNumDigits>(nd);
        canonicalize<kDenDigits>(dd);
        const double n64 = digits_to_f64<kNumDigits>(nd, kNumElo);
        const double d64 = digits_to_f64<kDenDigits>(dd, kDenElo);
        A.o[b * A.osB + hq * A.osH + i * A.osS + d] = (float)(n64 / d64);
        if (A.stat_den && d == 0) {
            A.stat_den[bh * A.stat_rows + i] = d64;
            A.stat_m[bh * A.stat_rows + i] = pv_rowmax(A, bh, i);
        }
    }
}

// ---------------------------------------------------------------- launchers

size_t vslice_bytes(const AttnGeom &g, int64_t kv_len) {
    const int64_t bhk = g.B * g.Hkv, nG = (g.D + 31) / 32;
    const int64_t nKB = std::max<int64_t>((kv_len + kKB - 1) / kKB, 1);
    return align256((size_t)bhk * nG * nKB * kBmax * 1024);
}

size_t vstats_bytes(const AttnGeom &g) {
    const int64_t bhk = g.B * g.Hkv, nG = (g.D + 31) / 32;
    return align256((size_t)bhk * nG * kVChunks * 32 * 8);
}

size_t vrare_bytes(const AttnGeom &g) {
    const int64_t bhk = g.B * g.Hkv, nG = (g.D + 31) / 32;
    return align256(4) + align256((size_t)bhk * nG * 4) + align256((size_t)kRareCap * 16);
}

size_t vprep_bytes(const AttnGeom &g, int64_t kv_len) {
    const int64_t bhk = g.B * g.Hkv, Dp32 = (g.D + 31) / 32 * 32, nG = Dp32 / 32;
    return vstats_bytes(g) + align256((size_t)bhk * Dp32 * 4) + align256((size_t)bhk * nG * 4) +
           vslice_bytes(g, kv_len) + vrare_bytes(g);
}

size_t pv_fallback_bytes(const AttnGeom &g, int64_t rows_i) {
    const int64_t tiles = (rows_i + 31) / 32, bh = g.B * g.Hq;
    return align256((size_t)bh * tiles * 4) +                                   // flags
           align256((size_t)kNumDigits * bh * tiles * 32 * g.D * 8) +           // fused scratch NUM
           align256((size_t)kDenDigits * bh * tiles * 32 * 8);                  // fused scratch DEN
}

VJob make_vjob(const Tensor &v, const AttnGeom &g, int64_t kv_lo, int64_t kv_hi, VPrep &vp) {
    const int64_t Dp32 = (g.D + 31) / 32 * 32, len = kv_hi - kv_lo;
    vp.Dp32 = Dp32;
    vp.nKB = std::max<int64_t>((len + kKB - 1) / kKB, 1);
    VJob J{};
    J.v = v.data;
    J.dtype = v.dtype;
    J.vsB = v.sB;
    J.vsH = v.sH;
    J.vsS = v.sS;
    J.Hkv = g.Hkv;
    J.D = g.D;
    J.Dp32 = Dp32;
    J.nG = Dp32 / 32;
    J.kv_lo = kv_lo;
    J.kv_hi = kv_hi;
    J.nKB = vp.nKB;
    J.nbhk = g.B * g.Hkv;
    J.stats = vp.stats;
    J.colgrid = vp.colgrid;
    J.grpB = vp.grpB;
    J.vsl = vp.slices;
    J.rare_n = vp.rare_n;
    J.rare_grp = vp.rare_grp;
    J.rare = vp.rare;
    return J;
}

hipError_t launch_vprep(const Tensor &v, const AttnGeom &g, int64_t kv_lo, int64_t kv_hi, VPrep &vp,
                        hipStream_t s) {
    ProfScope prof_("vprep", s);
    const VJob J = make_vjob(v, g, kv_lo, kv_hi, vp);
    hipError_t e;
    dim3 gs((unsigned)kVChunks, (unsigned)J.nG, (unsigned)J.nbhk);  // (an empty range leaves every chunk empty)
    if (v.dtype == 0) hipLaunchKernelGGL(k_vstats<float>, gs, dim3(256), 0, s, J);
    else hipLaunchKernelGGL(k_vstats<bf16_t>, gs, dim3(256), 0, s, J);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    dim3 gsl((unsigned)J.nKB, (unsigned)J.nG, (unsigned)J.nbhk);
    if (v.dtype == 0) hipLaunchKernelGGL(k_vslice<float>, gsl, dim3(64), 0, s, J);
    else hipLaunchKernelGGL(k_vslice<bf16_t>, gsl, dim3(64), 0, s, J);
    return hipGetLastError();
}

template <bool FUSED>
static hipError_t launch_pv_t(const Tensor &v, const AttnGeom &g, const VPrep &vp, PvArgs &a, int64_t bh,
                              int64_t *num_ws, int64_t *den_ws, hipStream_t s) {
    hipError_t e;
    {
        ProfScope prof_("pv_mfma", s);
        const int64_t nG = vp.Dp32 / 32;
        dim3 grid((unsigned)(a.causal ? (a.ntiles + 1) / 2 : a.ntiles), (unsigned)bh);
        // at most four groups per launch; wider heads take several launches over
        // the same tiles (the weights are recomputed, the digits are not shared)
        for (int G0 = 0; G0 < nG; G0 += 4) {
            if (nG == 1) hipLaunchKernelGGL((k_pv<FUSED, 1>), grid, dim3(64 * (1 + kPW)), 0, s, a, G0);
            else if (nG == 2) hipLaunchKernelGGL((k_pv<FUSED, 2>), grid, dim3(64 * (2 + kPW)), 0, s, a, G0);
            else hipLaunchKernelGGL((k_pv<FUSED, 4>), grid, dim3(64 * (4 + kPW)), 0, s, a, G0);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_pv(const Tensor &v, const AttnGeom &g, const VPrep &vp, const float *scores, const float *rowmax,
                     const uint32_t *rowmax_keys, int64_t rm_rows, int64_t rm_row0, int64_t i0, int64_t i1, int64_t kv_lo, int64_t kv_hi,
                     int *flags, int64_t *fb_num, int64_t *fb_den, const OutView *o, int64_t *num, int64_t *den,
                     int64_t plane_rows, int64_t rows_per_bh, int64_t row0, int force_fallback, hipStream_t s,
                     float *stat_m, double *stat_den, int64_t stat_rows) {
    const int64_t ni = i1 - i0;
    if (ni <= 0) return hipSuccess;
    if (vp.Dp32 > 256) return hipErrorInvalidValue;
    // key offsets, and byte offsets within a 32-row tile of scores, are 32-bit in the kernel
    if ((kv_hi - kv_lo + 64) * 32 * 4 > INT32_MAX) return hipErrorInvalidValue;
    const int64_t ntiles = (ni + 31) / 32, bh = g.B * g.Hq;
    PvArgs a{};
    a.scores = scores;
    a.rowmax = rowmax;
    a.rowmax_keys = rowmax_keys;
    a.rm_rows = rm_rows;
    a.rm_row0 = rm_row0;
    a.ni = ni;
    a.W = kv_hi - kv_lo;
    a.i0 = i0;
    a.kv_lo = kv_lo;
    a.kv_hi = kv_hi;
    a.Hq = g.Hq;
    a.Hkv = g.Hkv;
    a.group = g.Hq / g.Hkv;
    a.D = g.D;
    a.Dp32 = vp.Dp32;
    a.nKB = vp.nKB;
    a.causal = g.causal;
    a.vsl = (const v4i *)vp.slices;
    a.colgrid = vp.colgrid;
    a.grpB = vp.grpB;
    a.flags = flags;
    a.ntiles = ntiles;
    a.force_fallback = force_fallback;
    if (o) {
        if (o->sS < 0 || o->sS * 32 + g.D > INT32_MAX) return hipErrorInvalidValue;  // 32-bit offsets in a tile
        a.o = o->data;
        a.osB = o->sB;
        a.osH = o->sH;
        a.osS = o->sS;
    }
    a.num = num;
    a.den = den;
    a.plane_rows = plane_rows;
    a.rows_per_bh = rows_per_bh;
    a.row0 = row0;
    a.v = v.data;
    a.vdtype = v.dtype;
    a.vsB = v.sB;
    a.vsH = v.sH;
    a.vsS = v.sS;
    a.fb_num = fb_num;
    a.fb_den = fb_den;
    a.rare_n = vp.rare_n;
    a.rare_grp = vp.rare_grp;
    a.rare = vp.rare;
    if (o && stat_m && stat_den) {
        a.stat_m = stat_m;
        a.stat_den = stat_den;
        a.stat_rows = stat_rows;
    }
    return o ? launch_pv_t<true>(v, g, vp, a, bh, fb_num, fb_den, s)
             : launch_pv_t<false>(v, g, vp, a, bh, fb_num, fb_den, s);
}

}  // namespace det
