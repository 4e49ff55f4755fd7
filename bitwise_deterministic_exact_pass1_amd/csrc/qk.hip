// qk.hip -- pass-1 scores of bf16 inputs on the int8 matrix cores.
//
// The score rule is the fp64 fma chain over d = 0..D-1 (then RN64(scale*dot),
// RN32).  For bf16 operands every product q_d k_d has at most 16 significant
// bits, and with q = Qi * 2^gq, k = Ki * 2^gk (gq, gk = the smallest lsb
// exponent of the row; Qi, Ki integers) every partial sum of the chain is an
// integer times 2^(gq+gk).  When sum_d |Qi_d| |Ki_d| < 2^53 every partial sum
// is exactly representable in binary64, so the chain's result IS the exact
// integer dot product, whatever order it is summed in.  That integer is
// computed here from balanced int8 digits of Qi and Ki with
// v_mfma_i32_16x16x64_i8 (exact int32 sums).  The bound is checked per
// 16-row x 16-key item from per-row max|Qi| and per-key sum|Ki|; where it
// fails, each pair takes the finer test of qkrow.hpp (whose dot products may
// need 128 bits), and the pairs that fail that too (or whose rows need more
// than kQKmax digits) are recomputed by the plain fp64 chain in k_qk_fix, so
// the scores are the chain's bits either way.
#include "dev_math.hpp"
#include "kernels.hpp"
#include "qkrow.hpp"
#include "vprep.hpp"

#include <algorithm>
#include <type_traits>

namespace det {


constexpr int kQKbad = 99;             // row needs more digits than kQKmax

// Per-row statistics and digits: grid exponent g (smallest lsb), digit count,
// log2 bound of max|Xi| (Q) or of sum|Xi| (K); digits in [row][kQKmax][Dp64]
// bytes, zero padded to a multiple of 64 dims.  16 lanes per row, DPL = Dp64/16
// consecutive dims per lane, so each digit plane is one DPL-byte store per
// lane.  The Q pass also starts the rowmax keys of its rows at "empty" and the
// fix count at 0 (the score pass that follows max-reduces and counts into them).
struct QPrep {
    const bf16_t *x;
    int64_t sB, sH, sS, H, D, Dp64, s0, ns, ns_pad, nrows;
    int4 *info;
    int8_t *dig;
    uint32_t *keys;  // Q only (may be null)
    int64_t key_rows, key_row0;
    int *nfix;  // Q only
    int *slot;  // Q only: every prepared row's score slot, set to none (-1) here
    int vec;    // rows are whole 64-dim groups on 16-byte boundaries
};

template <bool IS_K, int DPL>
__device__ __forceinline__ void qkprep_rows(const QPrep &P, int64_t blk) {
    const bf16_t *__restrict__ x = P.x;
    const int64_t sB = P.sB, sH = P.sH, sS = P.sS, H = P.H, D = P.D, Dp64 = P.Dp64, s0 = P.s0, ns = P.ns;
    const int64_t ns_pad = P.ns_pad, nrows = P.nrows, key_rows = P.key_rows, key_row0 = P.key_row0;
    int4 *__restrict__ info = P.info;
    int8_t *__restrict__ dig = P.dig;
    uint32_t *__restrict__ keys = P.keys;
    int *__restrict__ nfix = P.nfix;
    const int vec = P.vec;
    const int sub = threadIdx.x & 15;
    const int64_t row = blk * 16 + (threadIdx.x >> 4);
    if (row >= nrows) return;  // whole 16-lane groups leave together
    const int64_t bh = row / ns_pad, ii = row % ns_pad;
    const int64_t b = bh / H, h = bh % H;
    const bool live = ii < ns;
    const bf16_t *xr = x + b * sB + h * sH + (s0 + (live ? ii : 0)) * sS;
    float v[DPL];
    int emax = INT_MIN, lmin = INT_MAX, lmin2 = INT_MAX, pmin = 0;
    bool loaded = false;
    if constexpr (DPL % 8 == 0) {
        if (vec) {  // whole rows of D = Dp64 dims, 16-byte aligned: DPL/8 vector loads per lane
            const uint4 *xv = (const uint4 *)(xr + sub * DPL);
#pragma unroll
            for (int q = 0; q < DPL / 8; ++q) {
                const uint4 u = xv[q];
                const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    v[8 * q + 2 * k] = live ? __uint_as_float(w[k] << 16) : 0.0f;
                    v[8 * q + 2 * k + 1] = live ? __uint_as_float(w[k] & 0xffff0000u) : 0.0f;
                }
            }
            loaded = true;
        }
    }
    if (!loaded) {
#pragma unroll
        for (int t = 0; t < DPL; ++t) {
            const int64_t d = sub * DPL + t;
            const float xv = elem<bf16_t>::to_f32(xr[min64(d, D - 1)]);  // in range; used only if d < D
            v[t] = (live && d < D) ? xv : 0.0f;
        }
    }
#pragma unroll
    for (int t = 0; t < DPL; ++t) {
        if (v[t] != 0.0f) {
            const int e = f32_exp(v[t]);
            const int l = max(e, -126) - 7;
            emax = max(emax, e);
            // the smallest lsb exponent, a position holding it, the second smallest
            lmin2 = min(lmin2, max(lmin, l));
            if (l < lmin) pmin = sub * DPL + t;
            lmin = min(lmin, l);
        }
    }
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) {
        emax = max(emax, __shfl_xor(emax, off, 64));
        const int om = __shfl_xor(lmin, off, 64), om2 = __shfl_xor(lmin2, off, 64), op = __shfl_xor(pmin, off, 64);
        lmin2 = min(min(lmin2, om2), max(lmin, om));
        if (om < lmin || (om == lmin && op < pmin)) pmin = op;
        lmin = min(lmin, om);
    }
    const bool zero = emax == INT_MIN;
    const int g = zero ? 0 : lmin;
    const int mbits = zero ? 0 : emax + 1 - g;  // |Xi| < 2^mbits
    int nd = zero ? 1 : (mbits + 2 + 7) / 8;
    if (nd > kQKmax) nd = kQKbad;
    // balanced base-256 digits of |Xi| < 2^30: the bytes of Xi + 0x80808080
    // with their top bit flipped (digit set [-128, 127])
    uint32_t U[DPL];
    int64_t l1 = 0;
#pragma unroll
    for (int t = 0; t < DPL; ++t) {
        // (an integer; |Xi| < 2^30 wherever it is used, so a 32-bit conversion of
        // the value clamped to that range gives the same integer)
        const double xd = fmin(fmax(ldexp((double)v[t], -g), -1073741824.0), 1073741824.0);
        const int64_t xi = nd == kQKbad ? 0 : (int64_t)(int32_t)xd;
        l1 += xi < 0 ? -xi : xi;
        U[t] = (uint32_t)(xi + 0x80808080ll);
    }
    int bound = mbits;
    if (IS_K) {
#pragma unroll
        for (int off = 8; off > 0; off >>= 1) l1 += __shfl_xor(l1, off, 64);
        bound = l1 ? 64 - __clzll((long long)l1) : 0;  // sum|Ki| < 2^bound
    }
    if (sub == 0) {
        const int g2 = (zero || lmin2 == INT_MAX) ? kQKnoG2 : lmin2;
        info[row] = int4{g, nd, bound, qk_row_pack(zero ? 0 : pmin, g2)};
        if (!IS_K) {
            if (keys && live) keys[bh * key_rows + (s0 + ii - key_row0)] = kKeyNegInf;
            if (P.slot) P.slot[row] = -1;
            if (row == 0) {
                nfix[0] = 0;
                nfix[1] = 0;  // the slot count
            }
        }
    }
    int8_t *out = dig + row * kQKmax * Dp64 + sub * DPL;
#pragma unroll
    for (int a = 0; a < kQKmax; ++a) {
        uint32_t w[DPL / 4];
#pragma unroll
        for (int q = 0; q < DPL / 4; ++q) {
            uint32_t pack = 0;
#pragma unroll
            for (int u = 0; u < 4; ++u) pack |= ((U[4 * q + u] >> (8 * a)) & 255u) << (8 * u);
            w[q] = pack ^ 0x80808080u;
        }
        uint32_t *o = (uint32_t *)(out + a * Dp64);
        if constexpr (DPL == 8) {
            *(uint2 *)o = uint2{w[0], w[1]};
        } else if constexpr (DPL == 16) {
            *(uint4 *)o = uint4{w[0], w[1], w[2], w[3]};
        } else {
#pragma unroll
            for (int q = 0; q < DPL / 4; ++q) o[q] = w[q];
        }
    }
}

template <bool IS_K, int DPL>
__global__ __launch_bounds__(256) void k_qkprep(QPrep P) {
    qkprep_rows<IS_K, DPL>(P, blockIdx.x);
}

// One launch for the independent preparations before the scores: K's digit
// rows (nk workgroups, when K is prepared here), Q's digit rows (nq), and the
// column statistics of V (the rest, when V is prepared here).
template <int DPL>
__global__ __launch_bounds__(256) void k_prep(QPrep K, QPrep Q, VJob J, int64_t nk, int64_t nq) {
    int64_t blk = blockIdx.x;
    // Q's rows reset the fix and slot counts; without them the first workgroup does
    if (nq == 0 && blk == 0 && threadIdx.x == 0) {
        Q.nfix[0] = 0;
        Q.nfix[1] = 0;
    }
    if (blk < nk) {
        qkprep_rows<true, DPL>(K, blk);
        return;
    }
    blk -= nk;
    if (blk < nq) {
        qkprep_rows<false, DPL>(Q, blk);
        return;
    }
    blk -= nq;
    const int64_t chunk = blk % kVChunks, rest = blk / kVChunks;
    vstats_block<bf16_t>(J, chunk, rest % J.nG, rest / J.nG);
}

static QPrep make_qprep(const bf16_t *x, int64_t sB, int64_t sH, int64_t sS, int64_t H, int64_t D, int64_t Dp64,
                        int64_t s0, int64_t ns, int64_t ns_pad, int64_t nrows, int4 *info, int8_t *dig,
                        uint32_t *keys, int64_t key_rows, int64_t key_row0, int *nfix, int *slot) {
    QPrep P{};
    P.x = x;
    P.sB = sB;
    P.sH = sH;
    P.sS = sS;
    P.H = H;
    P.D = D;
    P.Dp64 = Dp64;
    P.s0 = s0;
    P.ns = ns;
    P.ns_pad = ns_pad;
    P.nrows = nrows;
    P.info = info;
    P.dig = dig;
    P.keys = keys;
    P.key_rows = key_rows;
    P.key_row0 = key_row0;
    P.nfix = nfix;
    P.slot = slot;
    // vector loads when every row is whole 64-dim groups starting on 16 bytes
    P.vec = D == Dp64 && ((uintptr_t)x & 15) == 0 && sS % 8 == 0 && sH % 8 == 0 && sB % 8 == 0;
    return P;
}

template <bool IS_K>
static void launch_qkprep(const QPrep &P, hipStream_t s) {
    const dim3 grid((unsigned)((P.nrows + 15) / 16));
#define DET_QKPREP(DPL) hipLaunchKernelGGL((k_qkprep<IS_K, DPL>), grid, dim3(256), 0, s, P)
    switch (P.Dp64 / 16) {
        case 4: DET_QKPREP(4); break;
        case 8: DET_QKPREP(8); break;
        case 12: DET_QKPREP(12); break;
        default: DET_QKPREP(16); break;
    }
#undef DET_QKPREP
}

// K (when set), Q (when with_q) and V statistics (when J is set) in one launch.
static void launch_prep(const QPrep *K, const QPrep &Q, bool with_q, const VJob *J, hipStream_t s) {
    const int64_t nk = K ? (K->nrows + 15) / 16 : 0, nq = with_q ? (Q.nrows + 15) / 16 : 0;
    if (nk + nq == 0 && !J) return;
    const int64_t nv = J ? kVChunks * J->nG * J->nbhk : 0;
    const QPrep k0 = K ? *K : QPrep{};
    const VJob j0 = J ? *J : VJob{};
    const dim3 grid((unsigned)(nk + nq + nv));
#define DET_PREP(DPL) hipLaunchKernelGGL((k_prep<DPL>), grid, dim3(256), 0, s, k0, Q, j0, nk, nq)
    switch (Q.Dp64 / 16) {
        case 4: DET_PREP(4); break;
        case 8: DET_PREP(8); break;
        case 12: DET_PREP(12); break;
        default: DET_PREP(16); break;
    }
#undef DET_PREP
}

constexpr int kQkT = 16;     // rows and keys per matrix-core item
constexpr int kFixWhole = 1;  // fix-list entry: every pair of the item takes the chain
constexpr int kFixPairs = 0;  // fix-list entry: the pairs outside their own bound
constexpr int kQkWaves = 4;  // waves per workgroup, one 16-row tile each: 64-row groups

// Extents are 32-bit (the launcher rejects larger ones); offsets are formed
// in 64 bits.  Fewer 64-bit scalars keep the kernel's scalar registers in
// bounds.
struct QkArgs {
    const int8_t *qdig, *kdig;  // [row][kQKmax][Dp64]
    const int4 *qinfo, *kinfo;
    float *scores;  // [bh][ni][W] or null
    uint32_t *keys;  // rowmax keys, [bh*key_rows + i - key_row0], or null
    int *nfix;       // number of items left (in whole or in part) to the fp64 chain; nfix[1]: slots taken
    int4 *fixlist;   // their (kb, tile, bh, kFixWhole or kFixPairs)
    int fixcap;      // capacity of the list: one entry per item of the launch
    // score slots of rows with more than kQKmax digits (every pair of such a row
    // takes the chain): qslot[bh * ni_pad + row] (-1: none), slots[slot * kv_pad + key]
    int *qslot;
    float *slots;
    int slotcap;
    double scale;
    int Dp64, ni, ni_pad, i0, kv_lo, kv_hi, kv_pad;
    int Hq, Hkv, group;
    int causal;
    int W, key_rows, key_row0;
    int nKB, ntiles, ngroups;
};

// LDS of the score kernel: the digits and statistics of two 16-key blocks.
// Each key's row is padded by 16 bytes: the 16 lanes of a read pass then
// fetch 16 different keys from 16 disjoint sets of four banks.
template <int ND>
struct QkShared {
    static constexpr int kRow = kQKmax * 64 * ND + 16;
    uint8_t k[2][kQkT * kRow];
    int4 info[2][kQkT];
};

// One 64-row group of one head: wave w owns 16-row tile 4*group + w and keeps
// its digits in registers; the workgroup walks key blocks part, part + P, ...
// (P = gridDim.x) up to the last block the group can see.  The digits of the
// next block are loaded from global memory while the current one is
// multiplied and are stored to LDS only afterwards, so the loads overlap the
// matrix-core work and the epilogue.  Per block and wave: the item bound, the
// digit products, the exact integer dot per pair turned into the score, and a
// running per-lane max of each row.  Items that fail the bound go to a list
// for the fp64 chain.  All kQKmax digit products are issued: digits above a
// row's count are zero, and branching per product costs more registers than
// the products do.  Operand layout of v_mfma_i32_16x16x64_i8: lane l supplies
// row (A) or column (B) l%16 with k = 16*(l/16) + 0..15; result register r of
// lane l holds row 4*(l/16) + r, column l%16.
template <int ND>
__device__ __forceinline__ void qk_group(const QkArgs &A, int64_t bh, int64_t group, int part, QkShared<ND> &S) {
    constexpr int RB = kQKmax * 64 * ND;  // digit bytes of one key (or row) in global memory
    constexpr int KROW = QkShared<ND>::kRow;
    constexpr int NCH = kQkT * RB / 16;   // 16-byte chunks of one block
    constexpr int CPT = (NCH + 255) / 256;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lq = lane >> 4;
    const int P = gridDim.x;  // (part: this workgroup's key-block phase, 0 <= part < P)
    const int64_t b = bh / A.Hq, hq = bh % A.Hq, hk = hq / A.group, bhk = b * A.Hkv + hk;
    const int tile = (int)group * kQkWaves + wave;
    const bool live = tile < A.ntiles;
    const int it0 = A.i0 + tile * kQkT, i_end = A.i0 + A.ni;

    // key blocks of this workgroup: part, part + P, ... below kb_end
    int kb_end = A.nKB;
    if (A.causal) {
        const int last = A.i0 + min(((int)group + 1) * kQkWaves * kQkT, A.ni) - 1;
        kb_end = last >= A.kv_lo ? min(kb_end, (last - A.kv_lo) / kQkT + 1) : 0;
    }
    const int nb = kb_end > part ? (kb_end - (int)part + (int)P - 1) / (int)P : 0;

    // this wave's rows: digits, digit count and bound (max over the 16 rows), grids
    int aq = 0, qbt = 0;
    int4 qi = int4{0, 0, 0, 0};
    v4i Aq[kQKmax][ND];
    if (live) {
        qi = A.qinfo[bh * A.ni_pad + tile * kQkT + lr];
        const int8_t *qrow = A.qdig + (bh * A.ni_pad + (int64_t)(tile * kQkT + lr)) * RB + 16 * lq;
#pragma unroll
        for (int a = 0; a < kQKmax; ++a)
#pragma unroll
            for (int n = 0; n < ND; ++n) Aq[a][n] = *(const v4i *)(qrow + a * 64 * ND + 64 * n);
    }
    aq = qi.y;
    qbt = qi.z;
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) {
        aq = max(aq, __shfl_xor(aq, off, 64));
        qbt = max(qbt, __shfl_xor(qbt, off, 64));
    }
    aq = __builtin_amdgcn_readfirstlane(aq);  // wave-uniform after the reduction
    qbt = __builtin_amdgcn_readfirstlane(qbt);
    // the grids of the four rows of the lane's result registers (their other
    // statistics are fetched the same way where the per-pair test needs them)
    int gq[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) gq[r] = __shfl(qi.x, 4 * lq + r, 64);
    // rows with more digits than the digit rows hold: every pair takes the
    // chain (in k_qk_fix); each gets a score slot for pass 2 while slots last
    // (assigned by the first part of the group only: one writer per row)
    if (aq > kQKmax && A.qslot && part == 0 && lq == 0 && live && qi.y > kQKmax && it0 + lr < i_end) {
        int at = tile * kQkT + lr;
        asm volatile("" : "+v"(at));  // (the address is formed here, not kept from the start)
        int *sp = A.qslot + bh * A.ni_pad + at;
        if (*sp < 0) {
            const int n = atomicAdd(A.nfix + 1, 1);
            if (n < A.slotcap) *sp = n;
        }
    }
    uint32_t mkey[4] = {kKeyNegInf, kKeyNegInf, kKeyNegInf, kKeyNegInf};
    float *srow = (A.scores && live) ? A.scores + (bh * A.ni + (it0 + 4 * lq - A.i0)) * (int64_t)A.W : nullptr;

    // staging of a block's digits: chunk c = tid + 256 t is bytes 16*(c % (RB/16)) of key c / (RB/16)
    const int8_t *kbase = A.kdig + bhk * A.kv_pad * (int64_t)RB;
    const int4 *ibase = A.kinfo + bhk * A.kv_pad;
    auto block_src = [&](int n) { return kbase + (int64_t)((part + n * P) * kQkT) * RB; };
    v4i stage[CPT];
    int4 sinfo = int4{0, 0, 0, 0};
    auto load_block = [&](int n) {
        const int8_t *src = block_src(n);
        // (no branches: a load under a lane condition was issued behind a wait
        // for every load before it; lanes past the block read its last chunk)
#pragma unroll
        for (int t = 0; t < CPT; ++t) stage[t] = *(const v4i *)(src + (int64_t)min(tid + 256 * t, NCH - 1) * 16);
        sinfo = ibase[(part + n * P) * kQkT + min(tid, kQkT - 1)];
    };
    auto store_block = [&](int buf) {
#pragma unroll
        for (int t = 0; t < CPT; ++t) {
            const int c = tid + 256 * t;
            if (c < NCH) *(v4i *)(S.k[buf] + (c / (RB / 16)) * KROW + (c % (RB / 16)) * 16) = stage[t];
        }
        if (tid < kQkT) S.info[buf][tid] = sinfo;
    };
    if (nb > 0) {
        load_block(0);
        store_block(0);
    }
    // the Q rows are needed from here on: waiting for them now (they were
    // loaded before block 0, which store_block has waited for) keeps the
    // block loop free of waits for them, which would also wait for the
    // prefetched next block
#pragma unroll
    for (int a = 0; a < kQKmax; ++a)
#pragma unroll
        for (int n = 0; n < ND; ++n) asm volatile("" ::"v"(Aq[a][n]));
    __syncthreads();
    for (int n = 0; n < nb; ++n) {
        const int buf = n & 1;
        const int kb = part + n * P;
        if (n + 1 < nb) load_block(n + 1);
        const int j0 = A.kv_lo + kb * kQkT;
        if (live && !(A.causal && j0 > it0 + kQkT - 1)) {
            const int4 ki = S.info[buf][lr];
            int bk = ki.y, kbnd = ki.z;
#pragma unroll
            for (int off = 8; off > 0; off >>= 1) {
                bk = max(bk, __shfl_xor(bk, off, 64));
                kbnd = max(kbnd, __shfl_xor(kbnd, off, 64));
            }
            bk = __builtin_amdgcn_readfirstlane(bk);
            kbnd = __builtin_amdgcn_readfirstlane(kbnd);
            if (aq > kQKmax || bk > kQKmax) {  // rows with more digits: the whole item takes the chain
                if (lane == 0) {
                    const int at = atomicAdd(A.nfix, 1);
                    if (at < A.fixcap) A.fixlist[at] = int4{kb, tile, (int)bh, kFixWhole};
                }
            } else {
                // pairs within the bound are exact here; when the item's bound does not
                // hold, each pair takes the finer test (qkrow.hpp) and the pairs that fail
                // it are left to the chain.  NQ digits per side: three when every row and
                // key of the item has at most three (the fourth digit planes are zero)
                const bool perpair = qbt + kbnd > 53;
                const uint8_t *krow = S.k[buf] + lr * KROW + 16 * lq;
                auto item = [&](auto nq) {
                    constexpr int NQ = decltype(nq)::value, NC = 2 * NQ - 1;
                    v4i C[NC];
#pragma unroll
                    for (int c = 0; c < NC; ++c) C[c] = v4i{0, 0, 0, 0};
#pragma unroll
                    for (int nn = 0; nn < ND; ++nn) {
                        v4i Bk[NQ];
#pragma unroll
                        for (int c = 0; c < NQ; ++c) Bk[c] = *(const v4i *)(krow + c * 64 * ND + 64 * nn);
#pragma unroll
                        for (int a = 0; a < NQ; ++a)
#pragma unroll
                            for (int c = 0; c < NQ; ++c)
                                C[a + c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(Aq[a][nn], Bk[c], C[a + c], 0, 0, 0);
                    }
                    const int j = j0 + lr;
                    const bool jv = j < A.kv_hi;
                    const int gk = ki.x;
                    bool ok[4] = {true, true, true, true};
                    if (perpair) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int qbr = __shfl(qi.z, 4 * lq + r, 64), qw = __shfl(qi.w, 4 * lq + r, 64);
                            ok[r] = qk_pair_class(int4{gq[r], 0, qbr, qw}, ki, kQKmax) != kPairChain;
                        }
                    }
                    bool left = false;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int i = it0 + 4 * lq + r;
                        const float sc = (float)(A.scale * qk_dot_value<NC>(C, r, gq[r] + gk));
                        left |= !ok[r];
                        if (jv && i < i_end && ok[r]) {
                            if (srow) srow[(int64_t)r * A.W + (j - A.kv_lo)] = sc;
                            if (!A.causal || j <= i) mkey[r] = max(mkey[r], order_key(sc));
                        }
                    }
                    if (__ballot(left) && lane == 0) {
                        const int at = atomicAdd(A.nfix, 1);
                        if (at < A.fixcap) A.fixlist[at] = int4{kb, tile, (int)bh, kFixPairs};
                    }
                };
                if (aq <= 3 && bk <= 3) item(std::integral_constant<int, 3>{});
                else item(std::integral_constant<int, kQKmax>{});
            }
        }
        if (n + 1 < nb) store_block(buf ^ 1);
        // every path waits for the staged loads here, so none is in flight when
        // the next block's loads reuse their registers (else each waits for all)
#pragma unroll
        for (int t = 0; t < CPT; ++t) asm volatile("" ::"v"(stage[t]));
        asm volatile("" ::"v"(sinfo.x), "v"(sinfo.y), "v"(sinfo.z), "v"(sinfo.w));
        __syncthreads();
    }
    if (!A.keys || !live) return;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        uint32_t m = mkey[r];
#pragma unroll
        for (int off = 8; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
        const int i = it0 + 4 * lq + r;
        if (lr == 0 && i < i_end && m != kKeyNegInf) atomicMax(&A.keys[bh * A.key_rows + (i - A.key_row0)], m);
    }
}

// Grid (P parts, groups or causal pairs of groups, heads).  A causal
// workgroup takes group ngroups-1-y and then group y, whose visible key
// counts add up alike for every y.
template <int ND>
__global__ __launch_bounds__(64 * kQkWaves, ND <= 2 ? 3 : 2) void k_qk_mfma(QkArgs A) {
    __shared__ __align__(16) QkShared<ND> S;
    const GridPos gp = xcd_grouped_pos();
    const int64_t bh = gp.z, y = gp.y;
    const int npass = (A.causal && y != A.ngroups - 1 - y) ? 2 : 1;
    for (int pass = 0; pass < npass; ++pass) {
        if (pass) __syncthreads();  // the LDS of the first group is free again
        qk_group<ND>(A, bh, (A.causal && pass == 0) ? A.ngroups - 1 - y : y, (int)gp.x, S);
    }
}

// The fp64 chain for the pairs k_qk_mfma left: every pair of a kFixWhole
// item, the pairs of a kFixPairs item whose row bound plus key bound exceeds
// 53.  Per listed item the workgroup stages its 16 q rows and 16 k rows in LDS
// as f32 (exact for bf16) with every load issued before the first is used,
// then one thread per pair that needs it runs the chain in ascending d.
constexpr int kFixD = 256;
//
// Workgroups from nfw on instead prepare V's digit slices (when V is prepared
// in this launch), one 32-key block per wave: both kinds of work are short and
// bound by memory latency, so they share one launch.
__global__ __launch_bounds__(256) void k_qk_fix(QkArgs A, const bf16_t *__restrict__ q, int64_t qsB, int64_t qsH,
                                                int64_t qsS, const bf16_t *__restrict__ k, int64_t ksB, int64_t ksH,
                                                int64_t ksS, int64_t D, int nfw, VJob J) {
    __shared__ float sq[kQkT][kFixD + 1], sk[kQkT][kFixD + 1];
    const int tid = threadIdx.x;
    if ((int)blockIdx.x >= nfw) {
        const int64_t blk = blockIdx.x - nfw, nkb4 = (J.nKB + 3) / 4;
        const int64_t kb = (blk % nkb4) * 4 + (tid >> 6), rest = blk / nkb4;
        if (kb < J.nKB) vslice_block<bf16_t>(J, kb, rest % J.nG, rest / J.nG, tid & 63);
        return;
    }
    const int r = tid >> 4, c = tid & 15;
    // the count and this workgroup's first entry are read together (the list
    // holds fixcap entries; an entry at or past the count is never used), and
    // each item's successor is fetched while the item is worked on
    const int n = min(*A.nfix, A.fixcap);
    int4 next = (int)blockIdx.x < A.fixcap ? A.fixlist[blockIdx.x] : int4{0, 0, 0, 0};
    const int i_end = A.i0 + A.ni;
    for (int it = blockIdx.x; it < n; it += nfw) {
        const int4 item = next;
        if (it + nfw < n) next = A.fixlist[it + nfw];
        const int kb = item.x, tile = item.y, bh = item.z;
        const int b = bh / A.Hq, hq = bh - b * A.Hq, hk = hq / A.group, bhk = b * A.Hkv + hk;
        const int it0 = A.i0 + tile * kQkT, j0 = A.kv_lo + kb * kQkT;
        const bf16_t *qb = q + b * qsB + hq * qsH, *kbp = k + b * ksB + hk * ksH;
        __syncthreads();  // the previous item's rows are no longer read
        const int i = it0 + r, j = j0 + c;
        // pair statistics, the row's score slot and its current key go out with
        // the row loads below, so their latency overlaps the staging (all the
        // indices are in range: rows and keys of a tile are padded, and the key
        // row is clamped to the last row)
        const int64_t qrow = (int64_t)bh * A.ni_pad + tile * kQkT + r;
        const int4 qi = A.qinfo[qrow], ki = A.kinfo[(int64_t)bhk * A.kv_pad + kb * kQkT + c];
        const int sl = A.qslot ? A.qslot[qrow] : -1;
        uint32_t *kp = A.keys ? &A.keys[(int64_t)bh * A.key_rows + (min(i, i_end - 1) - A.key_row0)] : nullptr;
        const uint32_t kcur = kp && c == 0 ? __hip_atomic_load(kp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
        // thread tid loads dim tid (D <= 256) of the 16 rows of each side; clamped
        // indices keep every load in range, and clamped values are never used
        {
            const int64_t dd = tid < D ? tid : D - 1;
            float xq[kQkT], xk[kQkT];
#pragma unroll
            for (int rr = 0; rr < kQkT; ++rr) {
                xq[rr] = elem<bf16_t>::to_f32(qb[min(it0 + rr, i_end - 1) * qsS + dd]);
                xk[rr] = elem<bf16_t>::to_f32(kbp[min(j0 + rr, A.kv_hi - 1) * ksS + dd]);
            }
            if (tid < D) {
#pragma unroll
                for (int rr = 0; rr < kQkT; ++rr) {
                    sq[rr][tid] = xq[rr];
                    sk[rr][tid] = xk[rr];
                }
            }
        }
        bool need = i < i_end && j < A.kv_hi;
        if (item.w == kFixPairs) need = need && qk_pair_class(qi, ki, kQKmax) == kPairChain;
        __syncthreads();
        uint32_t key = 0;  // below order_key of every number
        if (need) {
            // (unrolled: the LDS reads of 16 steps go out together, only the fma chain is serial)
            double acc = 0.0;
            const int Di = (int)D;
#pragma unroll 16
            for (int d = 0; d < Di; ++d) acc = fma((double)sq[r][d], (double)sk[c][d], acc);
            const float sc = (float)(A.scale * acc);
            if (A.scores) A.scores[((int64_t)bh * A.ni + (i - A.i0)) * A.W + (j - A.kv_lo)] = sc;
            if (sl >= 0 && sl < A.slotcap) A.slots[(int64_t)sl * A.kv_pad + (j - A.kv_lo)] = sc;  // the row's score slot
            if (!A.causal || j <= i) key = order_key(sc);
        }
        // the row's max over the item's 16 keys (16 consecutive lanes), then one
        // atomic per row, skipped when the row's key read above is already at
        // least as large (keys only grow within the launch, so a stale read only
        // costs an atomic): a row listed for every key block would otherwise send
        // all its pairs to one address
#pragma unroll
        for (int off = 8; off > 0; off >>= 1) key = max(key, (uint32_t)__shfl_xor((int)key, off, 64));
        if (kp && c == 0 && key > kcur) atomicMax(kp, key);
    }
}

// ---------------------------------------------------------------- launchers

static int64_t qk_dp64(const AttnGeom &g) { return (g.D + 63) / 64 * 64; }
// K digit rows of a key range: whole 64-key blocks (pass 2 stages 32 or 64 keys at a time), zero past the range
static int64_t qk_pad(int64_t len) { return std::max<int64_t>((len + 63) / 64, 1) * 64; }

size_t qk_kprep_bytes(const AttnGeom &g, int64_t kv_len) {
    const int64_t rows = g.B * g.Hkv * qk_pad(kv_len);
    return align256((size_t)rows * 16) + align256((size_t)rows * kQKmax * qk_dp64(g));
}

// Score slots of a chunk: one per 1024 query rows, at least 32 and at most 1024
// (rows with more digits than the digit rows hold are rare; rows beyond the
// capacity are left to pass 2's other paths).
static int64_t qk_slot_cap(int64_t rows) { return std::min<int64_t>(1024, std::max<int64_t>(32, rows / 1024)); }

// The chunk's part of the workspace: Q's statistics and digit rows, the fix
// and slot counts, the rows' slots (all four at places that do not depend on
// the key range: Q's part is kept across the key ranges of one chunk), the
// fix list and the slot scores.
struct QkChunk {
    int4 *qinfo;
    int8_t *qdig;
    int *nfix;
    int4 *fixlist;
    int *qslot;
    float *slots;
    int64_t slotcap, bytes;
};

static QkChunk qk_chunk(const AttnGeom &g, int64_t ni, int64_t kv_len, void *ws) {
    const int64_t ni_pad = padded_rows(ni), bh = g.B * g.Hq, rows = bh * ni_pad;
    const int64_t kv_pad = qk_pad(kv_len), nKB = kv_pad / kQkT;
    QkChunk C{};
    char *c = (char *)ws;
    size_t at = 0;
    auto take = [&](size_t n) { char *p = c ? c + at : nullptr; at += align256(n); return p; };
    C.qinfo = (int4 *)take((size_t)rows * 16);
    C.qdig = (int8_t *)take((size_t)rows * kQKmax * qk_dp64(g));
    C.nfix = (int *)take(8);
    C.qslot = (int *)take((size_t)rows * 4);
    C.fixlist = (int4 *)take((size_t)bh * (ni_pad / kQkT) * nKB * 16);
    C.slotcap = qk_slot_cap(rows);
    C.slots = (float *)take((size_t)C.slotcap * kv_pad * 4);
    C.bytes = (int64_t)at;
    return C;
}

size_t qk_chunk_bytes(const AttnGeom &g, int64_t ni, int64_t kv_len) {
    return (size_t)qk_chunk(g, ni, kv_len, nullptr).bytes;
}

bool qk_uses_mfma(const Tensor &q) { return q.dtype == 1; }

static QPrep k_rows(const Tensor &k, const AttnGeom &g, int64_t kv_lo, int64_t kv_hi, void *ws) {
    const int64_t Dp64 = qk_dp64(g), len = kv_hi - kv_lo;
    const int64_t kv_pad = qk_pad(len), rows = g.B * g.Hkv * kv_pad;
    int4 *info = (int4 *)ws;
    int8_t *dig = (int8_t *)ws + align256((size_t)rows * 16);
    return make_qprep((const bf16_t *)k.data, k.sB, k.sH, k.sS, g.Hkv, g.D, Dp64, kv_lo, len, kv_pad, rows, info, dig,
                      nullptr, 0, 0, nullptr, nullptr);
}

PvSrc qk_pv_src(const Tensor &q, const Tensor &k, const AttnGeom &g, void *kprep, void *chunk_ws, int64_t ni,
                int64_t kv_len, bool slots) {
    const int64_t Dp64 = qk_dp64(g), ni_pad = padded_rows(ni);
    const int64_t kv_pad = qk_pad(kv_len), krows = g.B * g.Hkv * kv_pad;
    const QkChunk C = qk_chunk(g, ni, kv_len, chunk_ws);
    PvSrc P{};
    P.qinfo = C.qinfo;
    P.qdig = C.qdig;
    if (slots) {
        P.qslot = C.qslot;
        P.slots = C.slots;
        P.slot_bytes = C.slotcap * kv_pad * 4;
    }
    P.kinfo = (const int4 *)kprep;
    P.kdig = (const int8_t *)kprep + align256((size_t)krows * 16);
    P.ni_pad = ni_pad;
    P.kv_pad = kv_pad;
    P.Dp64 = Dp64;
    P.scale = g.scale;
    P.q = q.data;
    P.k = k.data;
    P.qsB = q.sB;
    P.qsH = q.sH;
    P.qsS = q.sS;
    P.ksB = k.sB;
    P.ksH = k.sH;
    P.ksS = k.sS;
    return P;
}

hipError_t launch_qkv_prep(const Tensor &q, const Tensor &k, const Tensor &v, const AttnGeom &g, void *kprep,
                           bool prep_k, bool prep_q, VPrep *vp, void *chunk_ws, int64_t i0, int64_t i1, int64_t kv_lo,
                           int64_t kv_hi, hipStream_t s) {
    ProfScope prof_("qk_prep", s);
    const int64_t ni = i1 - i0;
    if (ni <= 0 || kv_hi <= kv_lo) return hipSuccess;
    if (g.D > 256) return hipErrorInvalidValue;
    const int64_t Dp64 = qk_dp64(g), ni_pad = padded_rows(ni), bh = g.B * g.Hq;
    const QkChunk C = qk_chunk(g, ni, kv_hi - kv_lo, chunk_ws);
    const QPrep Q = make_qprep((const bf16_t *)q.data, q.sB, q.sH, q.sS, g.Hq, g.D, Dp64, i0, ni, ni_pad, bh * ni_pad,
                               C.qinfo, C.qdig, nullptr, 0, 0, C.nfix, C.qslot);
    const QPrep K = prep_k ? k_rows(k, g, kv_lo, kv_hi, kprep) : QPrep{};
    VJob vj{};
    if (vp) vj = make_vjob(v, g, kv_lo, kv_hi, *vp);
    launch_prep(prep_k ? &K : nullptr, Q, prep_q, vp ? &vj : nullptr, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !vp) return e;
    return launch_vslice(vj, s);
}

hipError_t launch_qk_kprep(const Tensor &k, const AttnGeom &g, int64_t kv_lo, int64_t kv_hi, void *ws,
                           hipStream_t s) {
    ProfScope prof_("qk_prep", s);
    launch_qkprep<true>(k_rows(k, g, kv_lo, kv_hi, ws), s);
    return hipGetLastError();
}

hipError_t launch_scores_qk(const Tensor &q, const Tensor &k, const AttnGeom &g, void *kprep, bool prep_k,
                            bool prep_q, const VJob *vj, void *chunk_ws, int64_t i0, int64_t i1, int64_t kv_lo, int64_t kv_hi,
                            float *scores, uint32_t *rowmax_keys, int64_t key_rows, int64_t key_row0,
                            hipStream_t s) {
    const int64_t ni = i1 - i0;
    if (ni <= 0 || kv_hi <= kv_lo) return (prep_k || vj) ? hipErrorInvalidValue : hipSuccess;
    if (g.D > 256) return hipErrorInvalidValue;
    const int64_t Dp64 = qk_dp64(g), ni_pad = padded_rows(ni), bh = g.B * g.Hq;
    const int64_t len = kv_hi - kv_lo, kv_pad = qk_pad(len);
    const int64_t ntiles = ni_pad / kQkT, nKB = kv_pad / kQkT;
    const QkChunk C = qk_chunk(g, ni, len, chunk_ws);
    int4 *qinfo = C.qinfo;
    int8_t *qdig = C.qdig;
    int *nfix = C.nfix;
    int4 *fixlist = C.fixlist;
    const int64_t krows = g.B * g.Hkv * kv_pad;
    // every extent the kernels see must fit 32 bits (offsets are formed in 64)
    const int64_t lim = INT32_MAX;
    if (ni_pad > lim || kv_pad > lim || i0 + ni_pad > lim || kv_hi > lim || key_rows > lim || g.Hq > lim ||
        bh * ntiles * nKB > lim || C.slotcap * kv_pad * 4 > lim)
        return hipErrorInvalidValue;
    hipError_t e;
    {
        ProfScope prof_("qk_prep", s);
        // also sets the rowmax keys of the chunk to "empty" and the fix count to
        // 0; with K's digit rows and V's column statistics when they are asked for
        const QPrep Q = make_qprep((const bf16_t *)q.data, q.sB, q.sH, q.sS, g.Hq, g.D, Dp64, i0, ni, ni_pad,
                                   bh * ni_pad, qinfo, qdig, rowmax_keys, key_rows, key_row0, nfix, C.qslot);
        if (!prep_q && !prep_k && !vj) {
            // the fix count; the rows keep no slots (their digits are kept, the key range changed)
            if ((e = launch_fill_u32((uint32_t *)nfix, 2, 0u, s)) != hipSuccess) return e;
            if ((e = launch_fill_u32((uint32_t *)C.qslot, bh * ni_pad, 0xffffffffu, s)) != hipSuccess) return e;
        } else if (prep_k || vj || !prep_q) {
            const QPrep K = prep_k ? k_rows(k, g, kv_lo, kv_hi, kprep) : QPrep{};
            launch_prep(prep_k ? &K : nullptr, Q, prep_q, vj, s);
            if (!prep_q && (e = launch_fill_u32((uint32_t *)C.qslot, bh * ni_pad, 0xffffffffu, s)) != hipSuccess)
                return e;
        } else {
            launch_qkprep<false>(Q, s);
        }
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    QkArgs a{};
    a.qdig = qdig;
    a.kdig = (const int8_t *)kprep + align256((size_t)krows * 16);
    a.qinfo = qinfo;
    a.kinfo = (const int4 *)kprep;
    a.scores = scores;
    a.keys = rowmax_keys;
    a.nfix = nfix;
    a.fixlist = fixlist;
    a.fixcap = (int)(bh * ntiles * nKB);  // the list region holds one entry per item
    a.qslot = C.qslot;
    a.slots = C.slots;
    a.slotcap = (int)C.slotcap;
    a.scale = g.scale;
    a.Dp64 = (int)Dp64;
    a.ni = (int)ni;
    a.ni_pad = (int)ni_pad;
    a.i0 = (int)i0;
    a.kv_lo = (int)kv_lo;
    a.kv_hi = (int)kv_hi;
    a.kv_pad = (int)kv_pad;
    a.Hq = (int)g.Hq;
    a.Hkv = (int)g.Hkv;
    a.group = (int)(g.Hq / g.Hkv);
    a.causal = g.causal;
    a.W = (int)(kv_hi - kv_lo);
    a.key_rows = (int)key_rows;
    a.key_row0 = (int)key_row0;
    a.nKB = (int)nKB;
    a.ntiles = (int)ntiles;
    a.ngroups = (int)((ntiles + kQkWaves - 1) / kQkWaves);
    {
        ProfScope prof_("scores", s);
        // causal launches pair groups; parts of the key range spread the rest over the chip
        const int64_t gy = g.causal ? (a.ngroups + 1) / 2 : a.ngroups;
        const int64_t parts = std::max<int64_t>(1, std::min<int64_t>(8, (768 + gy * bh - 1) / (gy * bh)));
        dim3 grid((unsigned)parts, (unsigned)gy, (unsigned)bh);
        switch (Dp64 / 64) {
            case 1: hipLaunchKernelGGL(k_qk_mfma<1>, grid, dim3(64 * kQkWaves), 0, s, a); break;
            case 2: hipLaunchKernelGGL(k_qk_mfma<2>, grid, dim3(64 * kQkWaves), 0, s, a); break;
            case 3: hipLaunchKernelGGL(k_qk_mfma<3>, grid, dim3(64 * kQkWaves), 0, s, a); break;
            default: hipLaunchKernelGGL(k_qk_mfma<4>, grid, dim3(64 * kQkWaves), 0, s, a); break;
        }
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    ProfScope prof_("scores_fix", s);
    const int64_t items = bh * ntiles * nKB, nfw = std::min<int64_t>(items, 2048);
    const int64_t nvw = vj ? (vj->nKB + 3) / 4 * vj->nG * vj->nbhk : 0;  // V slice workgroups, 4 blocks each
    hipLaunchKernelGGL(k_qk_fix, dim3((unsigned)(nfw + nvw)), dim3(256), 0, s, a, (const bf16_t *)q.data, q.sB, q.sH,
                       q.sS, (const bf16_t *)k.data, k.sB, k.sH, k.sS, g.D, (int)nfw, vj ? *vj : VJob{});
    return hipGetLastError();
}

}  // namespace det
