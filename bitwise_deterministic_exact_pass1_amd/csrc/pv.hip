// pv.hip -- pass 2 of the exact softmax on the matrix cores.
//
// The det-attn page ("Method") needs NUM_id = sum_j w_ij V_jd and
// DEN_i = sum_j w_ij exactly, with w_ij = RN32(exp_det(RN64(s_ij - m_i))).
// Both factors are turned into integers on fixed grids, split into balanced
// base-256 digits, and multiplied on the int8 matrix cores, which add exactly
// in int32:
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
// of the W_ij, kept per lane in int64 halves that are folded every 8192 keys
// and added up per row in 128 bits.
//
// The scores s_ij of bf16 inputs are not stored between the passes: the
// weight-making waves recompute them on the matrix cores from the digit rows
// of Q and K that pass 1 prepared (the exactness argument of qk.hip: within
// the per-pair bound the integer dot product IS the fp64 chain's result), and
// run the fp64 chain itself for the rare pairs outside that bound.  f32 inputs
// keep their pass-1 scores in the workspace.
//
// A tile whose weights do not fit the grid (w < 2^-23, or w > 1 from a rowmax
// below the scores) or whose V columns need more than five digits is flagged
// and redone by the generic exact path (windowed binary64 sums into digit
// planes) in k_pv_fix, which also adds the exact remainders of V entries below
// their column grid: results never depend on which path ran.
#include "pvcommon.hpp"

#include <algorithm>

namespace det {

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

// ---------------------------------------------------------------- producers
//
// Producer wave pw owns, in every 32-key block, the 16 x 16 sub-block of
// query rows qr0 = 16 (pw & 1) .. +15 and keys kc0 = 16 (pw >> 1) .. +15; lane
// l has row qr0 + l % 16 and the four keys kc0 + 4 (l / 16) + 0..3.  With
// recomputed scores the wave forms S^T = K Q^T on v_mfma_i32_16x16x64_i8
// (A = the block's K digit rows from LDS, B = the tile's Q digit rows held in
// registers; lane l supplies row / column l % 16 with the 16 dims
// 16 (l / 16) .. of each 64), whose result register r of lane l is exactly
// key kc0 + 4 (l / 16) + r of row qr0 + l % 16.

// The lane's Q digit row (B operand of every block), its grid exponent, digit
// count and log2 bound of max|Qi| (qk.hip).
template <int ND> struct PvQRow {
    v4i Bq[kQKmax][ND > 0 ? ND : 1];
    int4 qi;        // {grid, digit count, log2 bound, packed second grid and position} (qkrow.hpp)
    int qcnt, qbnd;  // the largest digit count and bound of the wave's rows without a slot (wave-uniform)
    int slot;        // the row's score slot (pass 1's chain scores), or -1
    bool slots;      // a row of the wave has one (wave-uniform)
};

// The digit products of the lane's 16 x 16 item over NQ digits per side
// (NQ = 3 when every row and key of the item has at most three digits: the
// fourth digit planes are zero and are skipped) into 2 NQ - 1 shift classes.
template <int ND, int NQ>
__device__ __forceinline__ void pv_score_products(const PvQRow<ND> &P, const uint8_t *krow, v4i (&C)[2 * NQ - 1]) {
#pragma unroll
    for (int c = 0; c < 2 * NQ - 1; ++c) C[c] = v4i{0, 0, 0, 0};
#pragma unroll
    for (int n = 0; n < ND; ++n) {
        v4i Ak[NQ];
#pragma unroll
        for (int c = 0; c < NQ; ++c) Ak[c] = *(const v4i *)(krow + c * 64 * ND + 64 * n);
#pragma unroll
        for (int c = 0; c < NQ; ++c)
#pragma unroll
            for (int a = 0; a < NQ; ++a)
                C[a + c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(Ak[c], P.Bq[a][n], C[a + c], 0, 0, 0);
    }
}

// Scores of the lane's four keys of a block whose K digit rows and key
// statistics are in LDS buffer kbuf, recomputed on the matrix cores.  When the
// item's bound holds for all its pairs (largest row bound plus largest key
// bound: the common case) that is all.  Otherwise each pair takes the finer
// test, and the visible pairs outside it are deferred: their score here is
// -inf (weight 0), and {row in tile, key - kv_lo} goes to the tile's list, from
// which they are added after the tile's last block with their scores by the
// rule itself.  r: the lane's row in the tile; jrel: its first key - kv_lo;
// nv: visible keys among the four.  Returns false when the list is full.
template <int ND, int NQ>
__device__ __forceinline__ bool pv_scores_nq(const PvArgs &A, const PvQRow<ND> &P, PvShared<ND> &S, int kbuf, int par,
                                             int r, int jrel, int nv, int lane, int kc0, bool crude, float (&sc)[4]) {
    constexpr int KROW = PvKRow<ND>::KROW;
    const int kk = kc0 + 4 * (lane >> 4);
    const int4 kg4 = *(const int4 *)&S.kg[kbuf][kk];  // the four keys' grids
    const int kg[4] = {kg4.x, kg4.y, kg4.z, kg4.w};
    v4i C[2 * NQ - 1];
    pv_score_products<ND, NQ>(P, S.kd[kbuf] + (kc0 + (lane & 15)) * KROW + 16 * (lane >> 4), C);
#pragma unroll
    for (int u = 0; u < 4; ++u) sc[u] = (float)(A.src.scale * qk_dot_value<2 * NQ - 1>(C, u, P.qi.x + kg[u]));
    if (crude) return true;
    // the four keys' statistics in registers before any test (read together:
    // one LDS round trip), then the tests as plain arithmetic
    const int4 t0 = S.ki[kbuf][kk], t1 = S.ki[kbuf][kk + 1], t2 = S.ki[kbuf][kk + 2], t3 = S.ki[kbuf][kk + 3];
    int x0 = t0.x, y0 = t0.y, z0 = t0.z, w0 = t0.w, x1 = t1.x, y1 = t1.y, z1 = t1.z, w1 = t1.w;
    int x2 = t2.x, y2 = t2.y, z2 = t2.z, w2 = t2.w, x3 = t3.x, y3 = t3.y, z3 = t3.z, w3 = t3.w;
    asm volatile("" : "+v"(x0), "+v"(y0), "+v"(z0), "+v"(w0), "+v"(x1), "+v"(y1), "+v"(z1), "+v"(w1), "+v"(x2),
                 "+v"(y2), "+v"(z2), "+v"(w2), "+v"(x3), "+v"(y3), "+v"(z3), "+v"(w3));
    const int4 kis[4] = {int4{x0, y0, z0, w0}, int4{x1, y1, z1, w1}, int4{x2, y2, z2, w2}, int4{x3, y3, z3, w3}};
    int chain = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u)
        chain |= (u < nv && P.slot < 0 && qk_pair_class(P.qi, kis[u], kQKmax) == kPairChain) ? 1 << u : 0;
    bool fits = true;
    if (chain) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if ((chain >> u) & 1) {
                sc[u] = -__builtin_inff();
                const int at = atomicAdd(&S.dn[par], 1);
                if (at < kDeferCap) S.dl[par][at] = int2{r, jrel + u};
                else fits = false;
            }
        }
    }
    return fits;
}

template <int ND>
__device__ __forceinline__ bool pv_block_scores(const PvArgs &A, const PvQRow<ND> &P, PvShared<ND> &S, int kbuf,
                                                int par, int r, int jrel, int nv, int lane, int kc0, float (&sc)[4]) {
    const int2 kh = S.kh[kbuf][kc0 >> 4];
    const int kcnt = __builtin_amdgcn_readfirstlane(kh.x), kbnd = __builtin_amdgcn_readfirstlane(kh.y);
    const bool crude = P.qcnt <= kQKmax && kcnt <= kQKmax && P.qbnd + kbnd <= 53;
    if (P.qcnt <= 3 && kcnt <= 3) return pv_scores_nq<ND, 3>(A, P, S, kbuf, par, r, jrel, nv, lane, kc0, crude, sc);
    return pv_scores_nq<ND, kQKmax>(A, P, S, kbuf, par, r, jrel, nv, lane, kc0, crude, sc);
}

// Producer side of one tile: thread ptid of the kPW producer waves.  Returns
// whether the tile needs the generic path (known to both roles after the
// tile's last barrier).  Barriers per tile: [A] (the first K blocks staged),
// [B] (block 0's weights ready), one per key block, [C] (row sums and the bad
// flag complete), [D] (RN64(DEN) of every row in LDS); the consumers meet the
// same ones.
template <int NG, int ND>
__device__ __forceinline__ bool pv_produce(const PvArgs &A, int64_t bh, int64_t tile, int ptid, int par,
                                           PvShared<ND> &S) {
    constexpr int RB = PvKRow<ND>::RB, KROW = PvKRow<ND>::KROW;
    constexpr int CPT = ND > 0 ? RB / 128 : 1;  // 16-byte K chunks per producer lane and block
    const PvTile T = pv_tile_of(A, bh, tile);
    const int lane = ptid & 63, pw = ptid >> 6;
    const int qr0 = 16 * (pw & 1), kc0 = 16 * (pw >> 1);
    const int r = qr0 + (lane & 15), k0 = kc0 + 4 * (lane >> 4);
    const int64_t i = T.it0 + r;
    const bool rowok = i < T.i_end;
    if (ptid < 32) {
        S.den_hi[par][ptid] = 0;
        S.den_lo[par][ptid] = 0;
    }
    if (T.badv) {
        __syncthreads();  // [A]
        __syncthreads();  // [B]
        __syncthreads();  // [C]
        __syncthreads();  // [D]
        return true;
    }
    const float m = rowok ? pv_rowmax(A, bh, i) : 0.0f;
    // keys this row sees: [kv_lo, jend), counted from this lane's first key
    // kv_lo + k0 (32-bit: the launcher bounds the key range)
    const int64_t jend = rowok ? (A.causal ? min64(T.jhi, i + 1) : T.jhi) : A.kv_lo;
    const int vis0 = (int)(jend - A.kv_lo - k0);
    auto nvis = [&](int kb) { return max(0, min(4, vis0 - kb * kKB)); };
    const int dofs = ((r + 32 * (k0 >> 4)) * 16) + (k0 & 15);  // this lane's bytes in a W digit plane
    // this lane's sum of W: whi 2^32 + wsum; wsum grows by at most 4 2^46 per
    // block and is folded into whi every kCarryEvery blocks (< 2^57 between)
    int64_t wsum = 0, whi = 0;
    bool bad = false;

    // ---- score sources
    PvQRow<ND> P;
    P.slot = -1;
    P.slots = false;
    const uint8_t *kbase = nullptr;
    v4i kst[CPT];
    int4 kist = int4{0, 0, 0, 0};
    if constexpr (ND > 0) {
        const int64_t qrow = bh * A.src.ni_pad + (T.it0 - A.i0) + r;
        P.qi = A.src.qinfo[qrow];
        P.slot = A.src.qslot ? A.src.qslot[qrow] : -1;
        P.slots = __ballot(P.slot >= 0) != 0;
        // (rows past the end are padding rows: one digit, bound 0; rows with a
        // slot take their scores from it)
        int qc = P.slot < 0 ? P.qi.y : 0, qb = P.slot < 0 ? P.qi.z : 0;
#pragma unroll
        for (int off = 8; off > 0; off >>= 1) {
            qc = max(qc, __shfl_xor(qc, off, 64));
            qb = max(qb, __shfl_xor(qb, off, 64));
        }
        P.qcnt = __builtin_amdgcn_readfirstlane(qc);
        P.qbnd = __builtin_amdgcn_readfirstlane(qb);
        const int8_t *qd = A.src.qdig + qrow * RB + 16 * (lane >> 4);
#pragma unroll
        for (int a = 0; a < kQKmax; ++a)
#pragma unroll
            for (int n = 0; n < ND; ++n) P.Bq[a][n] = *(const v4i *)(qd + a * 64 * ND + 64 * n);
        kbase = (const uint8_t *)A.src.kdig + T.bhk * A.src.kv_pad * (int64_t)RB;
    }
    // K digit rows of block kb: chunk c = ptid + 256 t is bytes 16 (c % (RB/16)) of key c / (RB/16)
    auto k_load = [&](int kb) {
        if constexpr (ND > 0) {
            const uint8_t *src = kbase + (int64_t)kb * 32 * RB;
#pragma unroll
            for (int t = 0; t < CPT; ++t) kst[t] = *(const v4i *)(src + (int64_t)(ptid + 256 * t) * 16);
            if (ptid < 32) kist = A.src.kinfo[T.bhk * A.src.kv_pad + kb * 32 + ptid];
        }
    };
    auto k_store = [&](int buf) {
        if constexpr (ND > 0) {
#pragma unroll
            for (int t = 0; t < CPT; ++t) {
                const int c = ptid + 256 * t;
                *(v4i *)(S.kd[buf] + (c / (RB / 16)) * KROW + (c % (RB / 16)) * 16) = kst[t];
            }
            // the block's 32 key statistics are in lanes 0..31 of producer wave 0:
            // their grids, and per 16-key half the largest digit count and bound
            if (pw == 0) {
                int kc = kist.y, kb = kist.z;
#pragma unroll
                for (int off = 8; off > 0; off >>= 1) {
                    kc = max(kc, __shfl_xor(kc, off, 64));
                    kb = max(kb, __shfl_xor(kb, off, 64));
                }
                if (lane < 32) {
                    S.ki[buf][lane] = kist;
                    S.kg[buf][lane] = kist.x;
                    if ((lane & 15) == 0) S.kh[buf][lane >> 4] = int2{kc, kb};
                }
            }
        }
    };
    // stored scores (f32 inputs): the lane's four scores of block kb through a
    // buffer resource based at the tile's first row (key kv_lo + j of row r at
    // byte (r W + j) 4): a lane's offset is fixed and the block step is the
    // scalar offset; keys past a row's end read the next row or, past the
    // scores array, zero (buffer bounds): those keys are invisible
    // Recomputed scores: the same for the score slots of rows that have one
    // (slot s at byte (s kv_pad + j) 4, key kv_lo + j); the block step is again
    // the scalar offset.
    const int64_t row_first = bh * A.ni + (T.it0 - A.i0);
    const int64_t bytes_left = ND == 0 ? ((int64_t)gridDim.y * A.ni - row_first) * A.src.W * 4 : A.src.slot_bytes;
    const bool sload = ND == 0 || P.slots;
    const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(ND == 0 ? A.src.scores + row_first * A.src.W : A.src.slots), (short)0,
        (int)min64(bytes_left, INT32_MAX), 0x00020000);
    const int voff = ND == 0 ? (r * (int)A.src.W + k0) * 4 : (P.slot >= 0 ? (P.slot * (int)A.src.kv_pad + k0) * 4 : 0);
    auto s_load = [&](int kb, float (&x)[4]) {
        if (sload) {
#pragma unroll
            for (int u = 0; u < 4; ++u)
                x[u] = __builtin_bit_cast(float,
                                          __builtin_amdgcn_raw_buffer_load_b32(srs, voff + 4 * u, kb * kKB * 4, 0));
        }
    };
    // kept scores: the lane's four scores of blocks kb and kb + 1
    auto s_load2 = [&](int kb, float (&x)[8]) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            x[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(srs, voff + 4 * u, kb * kKB * 4, 0));
            x[4 + u] = __builtin_bit_cast(
                float, __builtin_amdgcn_raw_buffer_load_b32(srs, voff + 4 * u, (kb + 1) * kKB * 4, 0));
        }
    };
    constexpr int kRing = PvShared<ND>::kNDig - 1;
    // the weights of block kb into digit buffer kb % kNDig (its K rows are in
    // the K buffer of parity kb & 1)
    auto produce = [&](int kb, const float (&stored)[4]) {
        float sc[4];
        const int nv = nvis(kb), db = kb & 1, dg = kb & kRing;
        if constexpr (ND > 0) {
            if (!pv_block_scores<ND>(A, P, S, db, par, r, kb * kKB + k0, nv, lane, kc0, sc)) bad = true;
            if (P.slots && P.slot >= 0) {
#pragma unroll
                for (int u = 0; u < 4; ++u) sc[u] = stored[u];
            }
        } else {
#pragma unroll
            for (int u = 0; u < 4; ++u) sc[u] = stored[u];
        }
        const uint32_t nz = wave_or_mask(block_weights<4>(sc, m, nv, S.dig[dg] + dofs, wsum, bad));
        if (lane == 0) S.mask[dg][pw] = nz;
    };
    // kept scores: the weights of blocks kb and kb + 1 together (eight exp
    // chains per lane) into digit buffers kb % kNDig and (kb + 1) % kNDig
    auto produce2 = [&](int kb, const float (&stored)[8]) {
        const int d0 = kb & kRing, d1 = (kb + 1) & kRing;
        uint32_t nz0, nz1;
        block_weights2(stored, m, nvis(kb), nvis(kb + 1), S.dig[d0] + dofs, S.dig[d1] + dofs, wsum, bad, nz0, nz1);
        nz0 = wave_or_mask(nz0);
        nz1 = wave_or_mask(nz1);
        if (lane == 0) {
            S.mask[d0][pw] = nz0;
            S.mask[d1][pw] = nz1;
        }
    };

    // prologue: K blocks 0 and 1 in LDS ([A] makes them visible), block 2 in
    // registers; block 0's weights ([B] hands them to the consumers).  Stored
    // scores: blocks 0 and 1 in the two register sets.
    float s0[4] = {}, s1[4] = {};
    float p0[8] = {}, p1[8] = {};  // kept scores: blocks 4q, 4q+1 and 4q+2, 4q+3
    if constexpr (ND == 0) {
        if (T.nblk > 0) s_load2(0, p0);
        if (T.nblk > 2) s_load2(2, p1);
    } else if (T.nblk > 0) {
        k_load(0);
        k_store(0);
        s_load(0, s0);
        if (T.nblk > 1) {
            k_load(1);
            k_store(1);
            s_load(1, s1);
        }
    }
    if constexpr (ND > 0) {
        // the Q row is needed from here on: waiting for it now (it was loaded
        // before K's blocks 0 and 1, which the stores have waited for) keeps
        // the block loop free of waits for it, which would also wait for the
        // prefetched K rows
#pragma unroll
        for (int a = 0; a < kQKmax; ++a)
#pragma unroll
            for (int n = 0; n < ND; ++n) asm volatile("" ::"v"(P.Bq[a][n]));
    }
    __syncthreads();  // [A]
    if constexpr (ND == 0) {  // blocks 0 and 1
        if (T.nblk > 0) {
            produce2(0, p0);
            if (T.nblk > 4) s_load2(4, p0);
        }
    } else {
        if (T.nblk > 2) k_load(2);
        if (T.nblk > 0) {
            produce(0, s0);
            if (T.nblk > 2) s_load(2, s0);
        }
    }
    __syncthreads();  // [B]
    // One block step, while the consumers multiply block kb: block kb+2's K
    // rows (in registers) into K buffer kb & 1 (block kb's, done with) and
    // block kb+3's into registers; the weights of block kb+1.  Stored scores of
    // block kb+1 sit in register set (kb+1) & 1, which then takes block kb+3's
    // (the loop is unrolled by two so the sets keep their roles without copies).
    auto step = [&](int kb, float (&set)[4]) {
        if (kb + 1 < T.nblk) {
            if constexpr (ND > 0) {
                if (kb + 2 < T.nblk) {
                    k_store(kb & 1);
                    if (kb + 3 < T.nblk) k_load(kb + 3);
                }
            }
            produce(kb + 1, set);
            if (kb + 3 < T.nblk) s_load(kb + 3, set);
            if (((kb + 2) % kCarryEvery) == 0) {
                whi += wsum >> 32;
                wsum &= 0xffffffffll;
            }
        }
        __syncthreads();
    };
    // Kept scores, per even step kb while the consumers multiply blocks kb and
    // kb + 1: the weights of blocks kb + 2 and kb + 3 (their scores in one of
    // the two pair sets, which then takes blocks kb + 6 and kb + 7); the roles
    // meet after odd steps and the last one.
    auto step2 = [&](int kb, float (&set)[8]) {
        if (kb + 2 < T.nblk) {
            produce2(kb + 2, set);
            if (kb + 6 < T.nblk) s_load2(kb + 6, set);
            if (((kb + 4) % kCarryEvery) == 0) {
                whi += wsum >> 32;
                wsum &= 0xffffffffll;
            }
        }
        if (pv_meets<ND>(kb, T.nblk)) __syncthreads();
        if (kb + 1 < T.nblk && pv_meets<ND>(kb + 1, T.nblk)) __syncthreads();
    };
    if constexpr (ND == 0) {
        for (int kb = 0; kb < T.nblk; kb += 4) {
            step2(kb, p1);
            if (kb + 2 < T.nblk) step2(kb + 2, p0);
        }
    } else {
        for (int kb = 0; kb < T.nblk; kb += 2) {
            step(kb, s1);
            if (kb + 1 < T.nblk) step(kb + 1, s0);
        }
    }
    // The deferred pairs (final after the last block's barrier), 32 at a time
    // as the virtual keys of extra blocks.  Per extra block: their q and k
    // rows into the K digit buffers (free after the last block; [E0]), their
    // scores by the rule itself, one lane per pair ([E1] hands them to every
    // producer lane), the weights of those whose row is the lane's ([E2] hands
    // them to the consumers, who form the V digits of the pairs' keys).  The
    // block count and the carry schedule continue those of the tile's keys.
    if constexpr (ND > 0) {
        const int ndef = min(S.dn[par], kDeferCap);
        const int D = (int)A.D;
        const bf16_t *qb = (const bf16_t *)A.src.q + T.b * A.src.qsB + T.hq * A.src.qsH;
        const bf16_t *kb0 = (const bf16_t *)A.src.k + T.b * A.src.ksB + (T.hq / A.group) * A.src.ksH;
        uint16_t *qs = (uint16_t *)S.kd[0], *ks = (uint16_t *)S.kd[1];
        for (int x = 0; x < (ndef + 31) / 32; ++x) {
            for (int t = ptid; t < 32 * D; t += 64 * kPW) {
                const int ee = t / D, d = t - ee * D, e = 32 * x + ee;
                const int2 E = e < ndef ? S.dl[par][e] : int2{0, 0};  // (padding: the tile's first row and key)
                qs[t] = qb[(T.it0 + E.x) * A.src.qsS + d].bits;
                ks[t] = kb0[(A.kv_lo + E.y) * A.src.ksS + d].bits;
            }
            __syncthreads();  // [E0]
            if (ptid < 32) {
                const int e = 32 * x + ptid;
                double acc = 0.0;
#pragma unroll 8
                for (int d = 0; d < D; ++d)
                    acc = fma((double)__uint_as_float((uint32_t)qs[ptid * D + d] << 16),
                              (double)__uint_as_float((uint32_t)ks[ptid * D + d] << 16), acc);
                S.dsc[ptid] = e < ndef ? (float)(A.src.scale * acc) : -__builtin_inff();
            }
            __syncthreads();  // [E1]
            const int kbv = T.nblk + x, db = kbv & 1;
            float sc[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int e = 32 * x + k0 + u;
                sc[u] = (e < ndef && S.dl[par][e].x == r) ? S.dsc[k0 + u] : -__builtin_inff();
            }
            const uint32_t nz = wave_or_mask(block_weights<4>(sc, m, 4, S.dig[db] + dofs, wsum, bad));
            if (lane == 0) S.mask[db][pw] = nz;
            if (((kbv + 1) % kCarryEvery) == 0) {
                whi += wsum >> 32;
                wsum &= 0xffffffffll;
            }
            __syncthreads();  // [E2]
        }
    }
    // exact row sums of W: the four lanes of a row (l, l^16, l^32, l^48), then
    // the two waves of a row half add theirs in LDS (each wsum < 2^57, so four
    // fit; whi counts units of 2^32)
#pragma unroll
    for (int off = 16; off < 64; off <<= 1) {
        wsum += __shfl_xor(wsum, off, 64);
        whi += __shfl_xor(whi, off, 64);
    }
    if (lane < 16) {
        const int64_t hi = whi + (wsum >> 32), lo = wsum & 0xffffffffll;
        atomicAdd(&S.den_hi[par][r], (unsigned long long)hi);
        atomicAdd(&S.den_lo[par][r], (unsigned long long)lo);
    }
    if (bad) S.bad[par] = 1;
    __syncthreads();  // [C]
    const bool generic = S.bad[par] != 0;
    if (pw < 2 && lane < 16) {
        // DEN 2^46 = hi 2^32 + lo; RN64(DEN) correctly rounded from its 128 bits
        const int64_t hi = (int64_t)S.den_hi[par][r] + (int64_t)(S.den_lo[par][r] >> 32);
        const uint64_t lo = S.den_lo[par][r] & 0xffffffffull;
        const double d64 = i128_to_f64(hi >> 32, ((uint64_t)hi << 32) | lo, -kSw);
        S.d64[par][r] = d64;
        if (A.stat_den && !generic && rowok) {  // (generic tiles write theirs in k_pv_fix)
            A.stat_den[bh * A.stat_rows + i] = d64;
            A.stat_m[bh * A.stat_rows + i] = m;
        }
    }
    __syncthreads();  // [D]
    return generic;
}

// ---------------------------------------------------------------- consumers

// The consumer's block loop for a wave whose group has BV V digits (0: no
// group, barriers only).  Per block: the six W digit fragments of the block
// are read from LDS, the next block's V digits are fetched into the other
// register set (the loop is unrolled by two so the sets swap roles without
// copies), and the class sums C_(a+b) += W_a x V_b run on the matrix cores for
// the W digit planes the producers marked nonzero.
template <int BV, int ND>
__device__ __forceinline__ void pv_consume_loop(const PvArgs &A, const PvTile &T, int G, const v4i *vb, int lane, int wave,
                                                v16i (&C)[kNC], PvShared<ND> &S, int par) {
    v4i VA[BV > 0 ? BV : 1], VB[BV > 0 ? BV : 1];
    __syncthreads();  // [A]
    if (BV > 0 && T.nblk > 0) {
#pragma unroll
        for (int s = 0; s < BV; ++s) VA[s] = vb[s * 64];
    }
    __syncthreads();  // [B]
    auto step = [&](int kb, const v4i (&cur)[BV > 0 ? BV : 1], v4i (&nxt)[BV > 0 ? BV : 1]) {
        if (BV > 0) {
            const int buf = kb & (PvShared<ND>::kNDig - 1);
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
        if (pv_meets<ND>(kb, T.nblk)) __syncthreads();
    };
    for (int kb = 0; kb < T.nblk; kb += 2) {
        step(kb, VA, VB);
        if (kb + 1 < T.nblk) step(kb + 1, VB, VA);
    }
    // extra blocks of deferred pairs (the producers' side says how they are
    // made): lane l supplies virtual keys 16 (l / 32) + p, p = 0..15, of its
    // column, whose V digits it forms from V itself as the slices do (the
    // value toward zero onto the column's grid; entries with bits below it
    // are the remainders added elsewhere)
    if constexpr (ND > 0) {
        const int ndef = min(S.dn[par], kDeferCap);
        for (int x = 0; x < (ndef + 31) / 32; ++x) {
            if (BV > 0) {
                const int64_t d = (int64_t)G * 32 + (lane & 31);
                const bool dok = d < A.D;
                const int g = dok ? A.colgrid[T.bhk * A.Dp32 + d] : 0;
                const int64_t vbase = T.b * A.vsB + (T.bhk % A.Hkv) * A.vsH + (dok ? d : 0);
                uint64_t U[16];
#pragma unroll
                for (int p = 0; p < 16; ++p) {
                    const int e = 32 * x + 16 * (lane >> 5) + p;
                    const int64_t j = A.kv_lo + (e < ndef ? S.dl[par][e].y : 0);
                    const double v = A.vdtype == 0 ? (double)((const float *)A.v)[vbase + j * A.vsS]
                                                   : (double)elem<bf16_t>::to_f32(((const bf16_t *)A.v)[vbase + j * A.vsS]);
                    U[p] = (uint64_t)((int64_t)ldexp(dok ? v : 0.0, -g) + 0x8080808080ll);
                }
#pragma unroll
                for (int bb = 0; bb < BV; ++bb) {
                    uint32_t w4[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        uint32_t pack = 0;
#pragma unroll
                        for (int u = 0; u < 4; ++u) pack |= ((uint32_t)(U[4 * q + u] >> (8 * bb)) & 255u) << (8 * u);
                        w4[q] = pack ^ 0x80808080u;
                    }
                    VA[bb] = v4i{(int)w4[0], (int)w4[1], (int)w4[2], (int)w4[3]};
                }
            }
            __syncthreads();  // [E0]
            __syncthreads();  // [E1]
            __syncthreads();  // [E2]
            if (BV > 0) {
                const int kbv = T.nblk + x, buf = kbv & 1;
                const uint8_t *dg = S.dig[buf] + lane * 16;
                uint32_t mask = 0;
#pragma unroll
                for (int w = 0; w < kPW; ++w) mask |= S.mask[buf][w];
                mask = __builtin_amdgcn_readfirstlane(mask);
#pragma unroll
                for (int a2 = 0; a2 < kAw; ++a2) {
                    const v4i Aw = *(const v4i *)(dg + a2 * 1024);
                    if (mask & (1u << a2)) {
#pragma unroll
                        for (int bb = 0; bb < BV; ++bb)
                            C[a2 + bb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(Aw, VA[bb], C[a2 + bb], 0, 0, 0);
                    }
                }
                if ((kbv % kCarryEvery) == kCarryEvery - 1) {
#pragma unroll
                    for (int c = 0; c < kNC - 1; ++c) {
                        const v16i cc = C[c] >> 8;
                        C[c] -= cc << 8;
                        C[c + 1] += cc;
                    }
#pragma unroll
                    for (int rr = 0; rr < 16; ++rr) S.top[wave][rr][lane] += C[kNC - 1][rr];
                    C[kNC - 1] = v16i{0};
                }
            }
        }
    }
}

// Consumer side of one tile: wave `wave` (< NG) owns 32-dim group G0 + wave.
// Returns whether the tile needs the generic path.
template <bool FUSED, int NG, int ND>
__device__ __forceinline__ bool pv_consume(const PvArgs &A, int G0, int64_t bh, int64_t tile, int wave, int par,
                                           PvShared<ND> &S) {
    const int tid = threadIdx.x, lane = tid & 63;
    const PvTile T = pv_tile_of(A, bh, tile);
    if (T.badv) {
        __syncthreads();  // [A]
        __syncthreads();  // [B]
        __syncthreads();  // [C]
        __syncthreads();  // [D]
        if (tid == 0) A.flags[bh * A.ntiles + tile] = kTileGeneric;
        return true;
    }
    if (tid == 0) {  // (before [A]; the producers set them after [A])
        S.bad[par] = 0;
        S.dn[par] = 0;
    }
    const int64_t G = G0 + wave;
    const bool mine = G < T.nG;
    const int Bv = mine ? A.grpB[T.bhk * T.nG + G] : 0;
    const v4i *vb = A.vsl + ((T.bhk * T.nG + (mine ? G : 0)) * A.nKB) * kBmax * 64 + lane;
    v16i C[kNC];
#pragma unroll
    for (int s = 0; s < kNC; ++s) C[s] = v16i{0};
    // the top class's int64 part, used by tiles of kCarryEvery blocks or more
    const bool longt = T.nblk + kDeferCap / 32 >= kCarryEvery;  // (extra blocks continue the count)
    if (longt) {
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) S.top[wave][rr][lane] = 0;
    }
    // the block loop with the wave's V digit count as a constant (one copy per
    // count; a wave without a group only meets the barriers)
    switch (mine ? Bv : 0) {
        case 1: pv_consume_loop<1, ND>(A, T, (int)G, vb, lane, wave, C, S, par); break;
        case 2: pv_consume_loop<2, ND>(A, T, (int)G, vb, lane, wave, C, S, par); break;
        case 3: pv_consume_loop<3, ND>(A, T, (int)G, vb, lane, wave, C, S, par); break;
        case 4: pv_consume_loop<4, ND>(A, T, (int)G, vb, lane, wave, C, S, par); break;
        case 5: pv_consume_loop<5, ND>(A, T, (int)G, vb, lane, wave, C, S, par); break;
        default: pv_consume_loop<0, ND>(A, T, (int)G, vb, lane, wave, C, S, par); break;
    }
    __syncthreads();  // [C]
    const bool generic = S.bad[par] != 0;
    __syncthreads();  // [D]: RN64(DEN) of every row is in LDS
    if (generic) {
        if (tid == 0) A.flags[bh * A.ntiles + tile] = kTileGeneric;
        return true;
    }
    if (tid == 0) A.flags[bh * A.ntiles + tile] = kTileDone;
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
    auto top = [&](int rr) -> int64_t {
        return (int64_t)C[kNC - 1][rr] + (longt ? S.top[wave][rr][lane] : 0);
    };
    auto row_of = [&](int rr) { return 8 * (rr >> 2) + 4 * (lane >> 5) + (rr & 3); };
    const int64_t d = G * 32 + (lane & 31);
    const int g = A.colgrid[T.bhk * A.Dp32 + d];
    if (FUSED && ((T.rem >> G) & 1)) {
        // this group's remainders are added by k_pv_fix: its exact NUM goes to
        // the tile's 32-row digit scratch (cleared here), with each row's
        // RN64(DEN) beside it, and is finalized there after the remainders
        const int64_t nplane = A.ntiles * 32 * (int64_t)gridDim.y * A.D;
        int64_t *nb = A.fb_num + (bh * A.ntiles + tile) * 32 * A.D;
        for (int t = lane; t < 32 * 32 * kNumDigits; t += 64) {
            const int k = t >> 10, rr = (t >> 5) & 31, c = t & 31;
            if (G * 32 + c < A.D) nb[k * nplane + rr * A.D + G * 32 + c] = 0;
        }
        if (lane < 32) ((double *)A.fb_den)[(bh * A.ntiles + tile) * 32 + lane] = S.d64[par][lane];
        __threadfence();
        if (d < A.D) {
#pragma unroll 1
            for (int rr = 0; rr < 16; ++rr) {
                const uint32_t l0 = (uint32_t)C[0][rr] | ((uint32_t)C[1][rr] << 8) |
                                    ((uint32_t)C[2][rr] << 16) | ((uint32_t)C[3][rr] << 24);
                const uint32_t l1 = (uint32_t)C[4][rr] | ((uint32_t)C[5][rr] << 8) |
                                    ((uint32_t)C[6][rr] << 16) | ((uint32_t)C[7][rr] << 24);
                const uint64_t lo = ((uint64_t)l1 << 32) | l0;
                const int64_t hi = top(rr) * 256 + C[kNC - 2][rr];
                const __int128 num = (__int128)(((unsigned __int128)(uint64_t)hi << 64) | lo);
                add_i128_digits<kNumDigits>(num, g - kSw - kNumElo, nb + row_of(rr) * A.D + d, nplane);
            }
        }
        return false;
    }
    if (FUSED) {
        // the lane's 16 outputs in two halves of 8 (no branches within a half:
        // its conversions and divisions interleave), each followed by the
        // stores of the rows that exist.
        // NUM = P_hi 2^48 + P_lo with P_lo = bytes C_0..C_5 (48 bits) and
        // P_hi = top 2^24 + bytes C_8 C_7 C_6: both exact in binary64 while
        // |P_hi| < 2^53, and then fma(P_hi, 2^48, P_lo) is the correctly rounded
        // NUM (one rounding).  A half holding a larger P_hi redoes its outputs
        // by the 128-bit conversion.
        // The output rows from a wave-uniform base and 32-bit lane offsets (the
        // launcher bounds 32 rows of output stride); the stride passes through an
        // empty asm so that no address is formed (and kept live) before here.
        int ostride = (int)A.osS;
        asm volatile("" : "+s"(ostride));
        float *ob = A.o + T.b * A.osB + T.hq * A.osH + T.it0 * A.osS;
        const int nrows = (int)min64(32, T.i_end - T.it0);
        const bool dok = d < A.D;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            float out[8];
            bool big = false;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int rr = 8 * h + u;
                const uint64_t plo = (uint64_t)((uint32_t)C[0][rr] | ((uint32_t)C[1][rr] << 8) |
                                                ((uint32_t)C[2][rr] << 16) | ((uint32_t)C[3][rr] << 24)) |
                                     ((uint64_t)((uint32_t)C[4][rr] | ((uint32_t)C[5][rr] << 8)) << 32);
                const int64_t phi = top(rr) * (1 << 24) + (int64_t)((uint32_t)C[6][rr] | ((uint32_t)C[7][rr] << 8) |
                                                                    ((uint32_t)C[8][rr] << 16));
                big |= (uint64_t)(phi + ((int64_t)1 << 53)) >= ((uint64_t)1 << 54);
                const double n64 = ldexp(fma((double)phi, 0x1p48, (double)plo), g - kSw);
                out[u] = (float)(n64 / S.d64[par][row_of(rr)]);
            }
            if (big) {
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int rr = 8 * h + u;
                    const uint32_t l0 = (uint32_t)C[0][rr] | ((uint32_t)C[1][rr] << 8) |
                                        ((uint32_t)C[2][rr] << 16) | ((uint32_t)C[3][rr] << 24);
                    const uint32_t l1 = (uint32_t)C[4][rr] | ((uint32_t)C[5][rr] << 8) |
                                        ((uint32_t)C[6][rr] << 16) | ((uint32_t)C[7][rr] << 24);
                    const uint64_t lo = ((uint64_t)l1 << 32) | l0;
                    const int64_t hi = top(rr) * 256 + C[kNC - 2][rr];
                    out[u] = (float)(i128_to_f64(hi, lo, g - kSw) / S.d64[par][row_of(rr)]);
                }
            }
            // keep the arithmetic ahead of the guarded stores (else it is moved
            // into each store's branch and the outputs run one after another)
#pragma unroll
            for (int u = 0; u < 8; ++u) asm volatile("" ::"v"(out[u]));
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int row = row_of(8 * h + u);
                if (row < nrows && dok) ob[row * ostride + (int)d] = out[u];
            }
        }
        return false;
    }
    // (the row base passes through an empty asm so that no address is formed
    // and kept live before here)
    int64_t pbase = bh * A.rows_per_bh + (T.it0 - A.row0);
    asm volatile("" : "+s"(pbase));
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
        const int row = row_of(rr);
        const int64_t io = T.it0 + row;
        if (io >= T.i_end || d >= A.D) continue;
        const uint32_t l0 = (uint32_t)C[0][rr] | ((uint32_t)C[1][rr] << 8) | ((uint32_t)C[2][rr] << 16) |
                            ((uint32_t)C[3][rr] << 24);
        const uint32_t l1 = (uint32_t)C[4][rr] | ((uint32_t)C[5][rr] << 8) | ((uint32_t)C[6][rr] << 16) |
                            ((uint32_t)C[7][rr] << 24);
        const uint64_t lo = ((uint64_t)l1 << 32) | l0;
        const int64_t hi = top(rr) * 256 + C[kNC - 2][rr];
        const __int128 num = (__int128)(((unsigned __int128)(uint64_t)hi << 64) | lo);
        const int64_t prow = pbase + row;
        add_i128_digits<kNumDigits>(num, g - kSw - kNumElo, A.num + prow * A.D + d, A.plane_rows * A.D);
        if (G == 0 && (lane & 31) == 0) {
            const int64_t hi2 = (int64_t)S.den_hi[par][row] + (int64_t)(S.den_lo[par][row] >> 32);
            const int64_t lo2 = (int64_t)(S.den_lo[par][row] & 0xffffffffull);
            add_i128_digits<kDenDigits>(((__int128)hi2 << 32) + lo2, -kSw - kDenElo, A.den + prow, A.plane_rows);
        }
    }
    return false;
}

// One workgroup per tile, or for causal attention per pair of tiles (x,
// ntiles-1-x), whose key counts add up to the same total for every pair: the
// whole grid then runs in one balanced round.  Both roles walk the same tiles
// and meet at the same barriers.  No barrier separates the two tiles beyond
// those: the producers start the second tile while the consumers finalize the
// first (row sums and flags are kept per tile).
template <bool FUSED, int NG, int ND>
__global__ __launch_bounds__(64 * (NG + kPW), 2) void k_pv(PvArgs A, int G0) {
    __shared__ __align__(16) PvShared<ND> S;
    const GridPos gp = xcd_grouped_pos();
    const int64_t bh = gp.y, x = gp.x;
    const int npass = (A.causal && x != A.ntiles - 1 - x) ? 2 : 1;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (wave >= NG) {
        for (int pass = 0; pass < npass; ++pass)
            pv_produce<NG, ND>(A, bh, (A.causal && pass == 0) ? A.ntiles - 1 - x : x, threadIdx.x - 64 * NG, pass,
                               S);
    } else {
        for (int pass = 0; pass < npass; ++pass)
            pv_consume<FUSED, NG, ND>(A, G0, bh, (A.causal && pass == 0) ? A.ntiles - 1 - x : x, wave, pass, S);
    }
}

// ---------------------------------------------------------------- flagged tiles and remainders

constexpr int kFixThreads = 256;
constexpr int kFixKeys = 64;  // keys whose weights one pass of the generic path holds in LDS

// The weights of rows [it0, it0+32) against keys [j0, j0 + kFixKeys) into wl
// (0 for invisible pairs), by the whole workgroup.
__device__ void fix_weights(const PvArgs &A, int64_t bh, int64_t it0, int64_t i_end, int64_t j0, int64_t jhi,
                            const float *m, float (*wl)[kFixKeys]) {
    for (int t = threadIdx.x; t < 32 * kFixKeys; t += blockDim.x) {
        const int r = t / kFixKeys, c = t % kFixKeys;
        const int64_t i = it0 + r, j = j0 + c;
        float w = 0.0f;
        if (i < i_end && j < jhi && (!A.causal || j <= i)) w = weight(pv_score(A, bh, i, j), m[r]);
        wl[r][c] = w;
    }
}

// A flagged tile by the generic exact path: per pass over kFixKeys keys, the
// tile's weights into LDS, then one binary64 window per (row, column) and per
// row for DEN, whose terms all lie on a grid 2^g with |window| < 2^(g+53), so
// every addition is exact; windows are flushed into digit planes by integer
// atomics at the end of each pass.  Fused: the tile's 32-row digit scratch,
// then the finalize; otherwise the caller's planes.
template <typename TV, bool FUSED>
__device__ void fix_generic_tile(const PvArgs &A, int64_t bh, int64_t tile, float *m, float (*wl)[kFixKeys]) {
    const int64_t b = bh / A.Hq, hq = bh % A.Hq, hk = hq / A.group;
    const int64_t it0 = A.i0 + tile * 32, i_end = A.i0 + A.ni;
    const int64_t D = A.D, nbh = gridDim.y;
    const int64_t jhi = A.causal ? min64(A.kv_hi, it0 + 32) : A.kv_hi;
    constexpr int VMB = elem<TV>::mant_bits;
    const TV *vp = (const TV *)A.v;
    int64_t *num = FUSED ? A.fb_num : A.num;
    int64_t *den = FUSED ? A.fb_den : A.den;
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
    }
    if (threadIdx.x < 32) m[threadIdx.x] = it0 + threadIdx.x < i_end ? pv_rowmax(A, bh, it0 + threadIdx.x) : 0.0f;
    __threadfence();
    __syncthreads();
    for (int64_t j0 = A.kv_lo; j0 < jhi; j0 += kFixKeys) {
        fix_weights(A, bh, it0, i_end, j0, jhi, m, wl);
        __syncthreads();
        const int nk = (int)min64(kFixKeys, jhi - j0);
        for (int64_t t = threadIdx.x; t < 32 * (D + 1); t += blockDim.x) {
            const int64_t r = t / (D + 1), d = t % (D + 1);  // d == D: the DEN window of row r
            const int64_t i = it0 + r;
            if (i >= i_end) continue;
            const TV *vcol = vp + b * A.vsB + hk * A.vsH + (d < D ? d : 0);
            const int64_t prow = prow_of(i);
            Window win;
            win.init();
            for (int c = 0; c < nk; ++c) {
                const float w = wl[r][c];
                if (w == 0.0f) continue;
                const int ew = f32_exp(w);
                const int lw = max(ew, -126) - 23;
                if (d == D) {
                    win.add<kDenDigits>((double)w, lw, ew + 1, kDenGcap, kDenElo, den + prow, nplane_rows);
                } else {
                    const float vf = elem<TV>::to_f32(vcol[(j0 + c) * A.vsS]);
                    if (vf == 0.0f) continue;
                    const int ev = f32_exp(vf);
                    win.add<kNumDigits>((double)w * (double)vf, lw + max(ev, -126) - VMB, ew + ev + 2, kNumGcap,
                                        kNumElo, num + prow * D + d, nplane_rows * D);
                }
            }
            if (d == D) win.flush<kDenDigits>(kDenElo, den + prow, nplane_rows);
            else win.flush<kNumDigits>(kNumElo, num + prow * D + d, nplane_rows * D);
        }
        __syncthreads();
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
            A.stat_m[bh * A.stat_rows + i] = m[r];
        }
    }
}

// The remainders of a tile's groups `grp` (V entries with bits below their
// column grid, vprep.hpp): each visible (row, remainder) product w V_rem is
// exact in binary64 and is added into the row's digits (the caller's planes,
// or the tile's scratch, where the consumers left the matrix-core part of
// those groups with each row's RN64(DEN)), then (fused) those groups' outputs
// are finalized from the digits.
template <bool FUSED>
__device__ void fix_remainder_tile(const PvArgs &A, int64_t bh, int64_t tile, uint32_t grp, float *m) {
    const PvTile T = pv_tile_of(A, bh, tile);
    int64_t *num = FUSED ? A.fb_num : A.num;
    const int64_t nplane_rows = FUSED ? A.ntiles * 32 * (int64_t)gridDim.y : A.plane_rows;
    auto prow_of = [&](int64_t i) -> int64_t {
        return FUSED ? (bh * A.ntiles + tile) * 32 + (i - T.it0) : bh * A.rows_per_bh + (i - A.row0);
    };
    if (threadIdx.x < 32)
        m[threadIdx.x] = T.it0 + threadIdx.x < T.i_end ? pv_rowmax(A, bh, T.it0 + threadIdx.x) : 0.0f;
    __syncthreads();
    const int n = min(*A.rare_n, kRareCap);
    for (int t = threadIdx.x; t < n * 32; t += blockDim.x) {
        const int4 E = A.rare[t >> 5];
        const int64_t i = T.it0 + (t & 31), j = E.y, d = E.z;
        if (E.x != T.bhk || !((grp >> (E.z / 32)) & 1) || i >= T.i_end) continue;
        const int64_t jend = A.causal ? min64(A.kv_hi, i + 1) : A.kv_hi;
        if (j < A.kv_lo || j >= jend) continue;
        const float w = weight(pv_score(A, bh, i, j), m[t & 31]);
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
    const double *d64s = (const double *)A.fb_den + (bh * A.ntiles + tile) * 32;
    for (int t = threadIdx.x; t < 32 * (int)T.nG * 32; t += blockDim.x) {
        const int r = t / ((int)T.nG * 32), c = t % ((int)T.nG * 32);
        const int64_t i = T.it0 + r;
        if (!((grp >> (c >> 5)) & 1) || c >= A.D || i >= T.i_end) continue;
        const int64_t at = prow_of(i) * A.D + c;
        int64_t nd[kNumDigits];
        unsigned long long *np = (unsigned long long *)num;
#pragma unroll
        for (int k = 0; k < kNumDigits; ++k) nd[k] = (int64_t)atomicAdd(np + k * nplane_rows * A.D + at, 0ull);
        canonicalize<kNumDigits>(nd);
        const double n64 = digits_to_f64<kNumDigits>(nd, kNumElo);
        A.o[T.b * A.osB + T.hq * A.osH + i * A.osS + c] = (float)(n64 / d64s[r]);
    }
}

// One workgroup per tile: the generic path for flagged tiles, the remainders
// for the others that have any.  Most workgroups find nothing to do.
template <bool FUSED>
__global__ __launch_bounds__(kFixThreads) void k_pv_fix(PvArgs A) {
    __shared__ float m[32];
    __shared__ float wl[32][kFixKeys];
    const int64_t tile = blockIdx.x, bh = blockIdx.y;
    if (A.flags[bh * A.ntiles + tile] == kTileGeneric) {
        if (A.vdtype == 0) fix_generic_tile<float, FUSED>(A, bh, tile, m, wl);
        else fix_generic_tile<bf16_t, FUSED>(A, bh, tile, m, wl);
        return;
    }
    const PvTile T = pv_tile_of(A, bh, tile);
    if (T.rem && T.nblk > 0) fix_remainder_tile<FUSED>(A, bh, tile, T.rem, m);
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

hipError_t launch_vslice(const VJob &J, hipStream_t s) {
    dim3 gsl((unsigned)J.nKB, (unsigned)J.nG, (unsigned)J.nbhk);
    if (J.dtype == 0) hipLaunchKernelGGL(k_vslice<float>, gsl, dim3(64), 0, s, J);
    else hipLaunchKernelGGL(k_vslice<bf16_t>, gsl, dim3(64), 0, s, J);
    return hipGetLastError();
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
    return launch_vslice(J, s);
}

template <bool FUSED> hipError_t launch_pv2_t(const PvArgs &a, int64_t bh, int nd, hipStream_t s);

template <bool FUSED>
static hipError_t launch_pv_t(const PvArgs &a, int64_t nG, int64_t bh, int nd, hipStream_t s) {
    hipError_t e;
    // Recomputed scores with head dims up to 128 over long key ranges: every
    // wave makes weights and multiplies (pv2.hip); its larger per-tile set-up
    // pays off past a few thousand keys.
    const int layout = pass2_layout();
    const bool eight = nd == 0 ? (nG <= 4 && layout == 1)
                               : ((nd == 1 || nd == 2) && (layout == 1 || (layout == 0 && a.kv_hi - a.kv_lo >= 4096)));
    if (eight) {
        {
            ProfScope prof_("pv_mfma", s);
            if ((e = launch_pv2_t<FUSED>(a, bh, nd, s)) != hipSuccess) return e;
        }
        ProfScope prof_("pv_fix", s);
        hipLaunchKernelGGL(k_pv_fix<FUSED>, dim3((unsigned)a.ntiles, (unsigned)bh), dim3(kFixThreads), 0, s, a);
        return hipGetLastError();
    }
    {
        ProfScope prof_("pv_mfma", s);
        dim3 grid((unsigned)(a.causal ? (a.ntiles + 1) / 2 : a.ntiles), (unsigned)bh);
        // at most four groups per launch; wider heads take several launches over
        // the same tiles (the weights are recomputed, the digits are not shared)
        for (int G0 = 0; G0 < nG; G0 += 4) {
            // the score source: stored (nd = 0) or recomputed from digit rows of nd 64-dim chunks
            if (nd == 0) {
                if (nG == 1) hipLaunchKernelGGL((k_pv<FUSED, 1, 0>), grid, dim3(64 * (1 + kPW)), 0, s, a, G0);
                else if (nG == 2) hipLaunchKernelGGL((k_pv<FUSED, 2, 0>), grid, dim3(64 * (2 + kPW)), 0, s, a, G0);
                else hipLaunchKernelGGL((k_pv<FUSED, 4, 0>), grid, dim3(64 * (4 + kPW)), 0, s, a, G0);
            } else if (nd == 1) {
                if (nG == 1) hipLaunchKernelGGL((k_pv<FUSED, 1, 1>), grid, dim3(64 * (1 + kPW)), 0, s, a, G0);
                else hipLaunchKernelGGL((k_pv<FUSED, 2, 1>), grid, dim3(64 * (2 + kPW)), 0, s, a, G0);
            } else if (nd == 2) {
                hipLaunchKernelGGL((k_pv<FUSED, 4, 2>), grid, dim3(64 * (4 + kPW)), 0, s, a, G0);
            } else if (nd == 3) {
                hipLaunchKernelGGL((k_pv<FUSED, 4, 3>), grid, dim3(64 * (4 + kPW)), 0, s, a, G0);
            } else {
                hipLaunchKernelGGL((k_pv<FUSED, 4, 4>), grid, dim3(64 * (4 + kPW)), 0, s, a, G0);
            }
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
    }
    ProfScope prof_("pv_fix", s);
    hipLaunchKernelGGL(k_pv_fix<FUSED>, dim3((unsigned)a.ntiles, (unsigned)bh), dim3(kFixThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_pv(const Tensor &v, const AttnGeom &g, const VPrep &vp, const PvSrc &src, const float *rowmax,
                     const uint32_t *rowmax_keys, int64_t rm_rows, int64_t rm_row0, int64_t i0, int64_t i1,
                     int64_t kv_lo, int64_t kv_hi, int *flags, int64_t *fb_num, int64_t *fb_den, const OutView *o,
                     int64_t *num, int64_t *den, int64_t plane_rows, int64_t rows_per_bh, int64_t row0,
                     int force_fallback, hipStream_t s, float *stat_m, double *stat_den, int64_t stat_rows) {
    const int64_t ni = i1 - i0;
    if (ni <= 0) return hipSuccess;
    if (vp.Dp32 > 256) return hipErrorInvalidValue;
    // key offsets, and byte offsets within a 32-row tile of scores, are 32-bit in the kernel
    if ((kv_hi - kv_lo + 64) * 32 * 4 > INT32_MAX) return hipErrorInvalidValue;
    const int64_t nG = vp.Dp32 / 32;
    const int nd = src.scores ? 0 : (int)(src.Dp64 / 64);
    if (!src.scores) {
        // recomputed scores: digit rows of (D rounded up to 64) bytes per digit, whole
        // 32-key blocks of K rows and 32-row tiles of Q rows; the kernels come in
        // (groups, chunks) = (1, 1), (2, 1), (4, 2..4)
        if (src.Dp64 != (g.D + 63) / 64 * 64 || src.kv_pad % 32 || src.ni_pad % 32 || src.ni_pad < ni ||
            src.kv_pad < kv_hi - kv_lo || (nd == 1) != (nG <= 2))
            return hipErrorInvalidValue;
    }
    const int64_t ntiles = (ni + 31) / 32, bh = g.B * g.Hq;
    PvArgs a{};
    a.src = src;
    a.rowmax = rowmax;
    a.rowmax_keys = rowmax_keys;
    a.rm_rows = rm_rows;
    a.rm_row0 = rm_row0;
    a.ni = ni;
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
    return o ? launch_pv_t<true>(a, nG, bh, nd, s) : launch_pv_t<false>(a, nG, bh, nd, s);
}

}  // namespace det
