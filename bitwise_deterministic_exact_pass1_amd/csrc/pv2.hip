// pv2.hip -- pass 2 of the exact softmax for recomputed bf16 scores (head
// dims up to 128), with every wave making weights and multiplying.
//
// The arithmetic is that of pv.hip (det-attn page, "Method": NUM_id =
// sum_j w_ij V_jd and DEN_i = sum_j w_ij exactly): scores recomputed from the
// Q and K digit rows on v_mfma_i32_16x16x64_i8, w = RN32(exp_det(s - m)),
// W = w 2^46 in six balanced digits, V on per-column grids in up to five, the
// class sums C_(a+b) += W_a x V_b exact in int32.  What differs is the split
// of the work.  A workgroup of eight waves owns a 32-row tile and walks the
// key range in blocks of 64 keys; per block, wave w
//   - scores the 16 x 16 item of rows 16 (w & 1) .. and keys 16 (w >> 1) ..
//     and turns it into W digits in LDS, and
//   - multiplies the whole block's W digits (32 rows x 64 keys) with the V
//     digits of its 16 output dims 16 w .. 16 w + 15 on
//     v_mfma_i32_16x16x64_i8 (two 16-row tiles), into its own class sums.
// Each SIMD then holds two waves that both run the fp64 exponentials and both
// issue matrix products, so one's arithmetic latency hides behind the
// other's work (a split into weight-making and multiplying waves leaves one
// dependent fp64 chain per SIMD), and the class sums of 32 rows x 16 dims
// take 72-80 registers.  Block kb's products run in the same step as block
// kb+1's weights, behind one barrier per block.
//
// Everything else follows pv.hip: deferred pairs (outside the exactness
// bound) as extra blocks scored by the fp64 chain, score slots of rows with
// many digits, the generic path and V remainders through k_pv_fix, the top
// class moved to int64 in LDS every 8192 keys, DEN as exact 128-bit row sums.
#include "pvcommon.hpp"

#include <algorithm>
#include <type_traits>

namespace det {

constexpr int kKB2 = 64;        // keys per block
constexpr int kW2 = 8;          // waves per workgroup
constexpr int kCarry2 = 128;    // blocks (8192 keys) between carry passes
constexpr int kDef2 = 1024;     // deferred pairs a tile can hold (more: the generic path)

template <int ND> struct Pv2Shared {
    static constexpr int RB = kQKmax * 64 * ND;  // digit bytes of one K (or Q) row
    static constexpr int KROW = RB + 16;         // LDS row: 16 lanes of a read hit 16 disjoint bank sets
    uint8_t kd[2][64 * KROW];                    // K digit rows of two blocks
    uint8_t qd[32 * KROW];                       // the tile's Q digit rows
    int4 ki[2][64];                              // key statistics (qkrow.hpp)
    int kg[2][64];                               // key grids
    int2 kh[2][4];                               // per 16-key quarter: largest digit count and bound
    // W digits of two blocks: [buffer][row tile][digit][operand lane * 16 + key % 16]
    uint8_t dig[2][2][kAw][1024];
    uint32_t mask[2][kW2];
    // per tile parity (a tile's finalize overlaps the next tile's start)
    unsigned long long den_hi[2][32], den_lo[2][32];  // exact sum of W per row: hi 2^32 + lo
    double d64[2][32];                                // RN64(DEN) of the row
    int bad[2];
    int dn[2];
    int2 dl[kDef2];     // deferred pairs of the current tile: {row in tile, key - kv_lo} (a tile's list
                        // is done with before its [C]; the next tile appends after its own [A])
    float dsc[64];      // their chain scores, per extra block
    int64_t top[kW2][8][64];  // int64 part of the top class: [wave][tile * 4 + register][lane]
};

// The products and weights of one tile for one wave: BVT V digits per group
// (4 serves groups of 1..4 digits: the higher digit planes are zero).
// Returns whether the tile needs the generic path.
template <bool FUSED, int ND, int BVT>
__device__ __forceinline__ bool pv2_tile(const PvArgs &A, const PvTile &T, int64_t bh, int64_t tile, int par,
                                         Pv2Shared<ND> &S) {
    constexpr int RB = Pv2Shared<ND>::RB, KROW = Pv2Shared<ND>::KROW;
    constexpr int NC = kAw + BVT - 1;                 // class sums
    constexpr int CPT = 64 * RB / 16 / (64 * kW2);    // 16-byte K chunks per thread and block
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    // 64-key blocks of the tile's keys [kv_lo, jhi) (K digit rows are padded to whole blocks)
    const int nblk = T.jhi > A.kv_lo ? (int)((T.jhi - A.kv_lo + kKB2 - 1) / kKB2) : 0;
    // ---- weight-making role: rows r, keys k0..k0+3 of each block
    const int qr0 = 16 * (w & 1), kc0 = 16 * (w >> 1);
    const int r = qr0 + (lane & 15), k0 = kc0 + 4 * (lane >> 4);
    const int64_t i = T.it0 + r;
    const bool rowok = i < T.i_end;
    const float m = rowok ? pv_rowmax(A, bh, i) : 0.0f;
    const int64_t jend = rowok ? (A.causal ? min64(T.jhi, i + 1) : T.jhi) : A.kv_lo;
    const int vis0 = (int)(jend - A.kv_lo - k0);
    auto nvis = [&](int kb) { return max(0, min(4, vis0 - kb * kKB2)); };
    // this lane's bytes in its row tile's W digit planes: operand lane (row % 16) + 16 (key / 16), bytes k0 % 16 ..
    const int dofs = (w & 1) * kAw * 1024 + ((lane & 15) + 16 * (w >> 1)) * 16 + 4 * (lane >> 4);
    int64_t wsum = 0, whi = 0;  // this lane's sum of W: whi 2^32 + wsum (wsum < 2^55 between folds)
    bool bad = false;
    // recomputed scores (ND > 0): the row's statistics and score slot, and the
    // largest digit count and bound of the wave's rows without a slot
    int4 qi = int4{0, 0, 0, 0};
    int slot = -1, qcnt = 0, qbnd = 0;
    bool slots = false;
    if constexpr (ND > 0) {
        const int64_t qrow = bh * A.src.ni_pad + (T.it0 - A.i0) + r;
        qi = A.src.qinfo[qrow];
        slot = A.src.qslot ? A.src.qslot[qrow] : -1;
        slots = __ballot(slot >= 0) != 0;
        int qc = slot < 0 ? qi.y : 0, qb = slot < 0 ? qi.z : 0;
#pragma unroll
        for (int off = 8; off > 0; off >>= 1) {
            qc = max(qc, __shfl_xor(qc, off, 64));
            qb = max(qb, __shfl_xor(qb, off, 64));
        }
        qcnt = __builtin_amdgcn_readfirstlane(qc);
        qbnd = __builtin_amdgcn_readfirstlane(qb);
    }
    // K digit rows of the head through a buffer resource (lane offsets in one
    // register, the block in the scalar offset: no per-lane addresses to keep)
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        ND > 0 ? (void *)((const uint8_t *)A.src.kdig + T.bhk * A.src.kv_pad * (int64_t)RB) : nullptr, (short)0,
        (int)(A.src.kv_pad * RB), 0x00020000);
    const __amdgpu_buffer_rsrc_t irs = __builtin_amdgcn_make_buffer_rsrc(
        ND > 0 ? (void *)(A.src.kinfo + T.bhk * A.src.kv_pad) : nullptr, (short)0, (int)(A.src.kv_pad * 16),
        0x00020000);
    // ---- multiplying role: dims 16 w .. 16 w + 15 of group G (32 dims) half h
    const int G = w >> 1, h = w & 1;
    const bool mine = 16 * w < A.D;
    const int64_t d = 16 * w + (lane & 15);
    // V digits of 64-key block kb, digit b, for this lane (column lane % 16,
    // keys 16 (lane / 16) ..): the 32-key slice 2 kb + lane / 32, its lane
    // 32 ((lane / 16) & 1) + 16 h + lane % 16 (vprep.hpp's layout), through a
    // buffer resource over the group's slices (a slice past the range reads
    // zero: its keys have zero weights)
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(A.vsl + ((T.bhk * T.nG + (mine ? G : 0)) * A.nKB) * kBmax * 64), (short)0,
        (int)(A.nKB * kBmax * 1024), 0x00020000);
    const int vlane = (((lane >> 5) * kBmax * 64) + 32 * ((lane >> 4) & 1) + 16 * h + (lane & 15)) * 16;
    auto v_load = [&](int kb, v4i (&Vr)[BVT]) {
#pragma unroll
        for (int b = 0; b < BVT; ++b)
            Vr[b] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(vrs, vlane + b * 1024,
                                                                                 2 * kb * kBmax * 1024, 0));
    };
    v4i VA[BVT];  // V digits of the block being multiplied
    v4i C[2][NC];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int c = 0; c < NC; ++c) C[t][c] = v4i{0, 0, 0, 0};
    const bool longt = nblk + kDef2 / kKB2 >= kCarry2;  // (extra blocks continue the count)
    if (longt) {
#pragma unroll
        for (int q = 0; q < 8; ++q) S.top[w][q][lane] = 0;
    }
    if (tid < 32) {
        S.den_hi[par][tid] = 0;
        S.den_lo[par][tid] = 0;
    }

    // ---- staging of K blocks and of the tile's Q rows
    struct KSet {
        v4i d[CPT > 0 ? CPT : 1];
        int4 st;
    };
    // chunk c = tid + 512 t of a block is bytes 16 (c % (RB/16)) of key c / (RB/16)
    auto k_load = [&](int kb, KSet &K) {
        if constexpr (ND == 0) return;
#pragma unroll
        for (int t = 0; t < CPT; ++t)
            K.d[t] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(krs, tid * 16,
                                                                                  kb * kKB2 * RB + t * 64 * kW2 * 16, 0));
        if (w == 0)
            K.st = __builtin_bit_cast(int4, __builtin_amdgcn_raw_buffer_load_b128(irs, lane * 16, kb * kKB2 * 16, 0));
    };
    auto k_store = [&](int buf, const KSet &K) {
        if constexpr (ND == 0) return;
#pragma unroll
        for (int t = 0; t < CPT; ++t) {
            const int c = tid + 64 * kW2 * t;
            *(v4i *)(S.kd[buf] + (c / (RB / 16)) * KROW + (c % (RB / 16)) * 16) = K.d[t];
        }
        if (w == 0) {  // the 64 keys' statistics, grids, and per 16-key quarter the largest count and bound
            int kc = K.st.y, kbd = K.st.z;
#pragma unroll
            for (int off = 8; off > 0; off >>= 1) {
                kc = max(kc, __shfl_xor(kc, off, 64));
                kbd = max(kbd, __shfl_xor(kbd, off, 64));
            }
            S.ki[buf][lane] = K.st;
            S.kg[buf][lane] = K.st.x;
            int q = lane >> 4;
            asm volatile("" : "+v"(q));  // (the address is formed here, not kept from the start)
            if ((lane & 15) == 0) S.kh[buf][q] = int2{kc, kbd};
        }
    };
    // kept scores (ND == 0): the lane's four scores of block kb through a
    // buffer resource based at the tile's first row (key kv_lo + j of row r at
    // byte (r W + j) 4; keys past a row's end read the next row or, past the
    // array, zero: those keys are invisible).  Recomputed scores: the slot
    // scores of rows that have one (slot s at byte (s kv_pad + j) 4).  Either
    // way the block step is the scalar offset.
    const int64_t row_first = bh * A.ni + (T.it0 - A.i0);
    const int64_t bytes_left = ND == 0 ? ((int64_t)gridDim.y * A.ni - row_first) * A.src.W * 4 : A.src.slot_bytes;
    const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
        ND == 0 ? (void *)(A.src.scores + row_first * A.src.W) : (void *)A.src.slots, (short)0,
        (int)min64(bytes_left, INT32_MAX), 0x00020000);
    const int voff = ND == 0 ? (r * (int)A.src.W + k0) * 4 : (slot >= 0 ? (slot * (int)A.src.kv_pad + k0) * 4 : 0);
    auto s_load = [&](int kb, float (&x)[4]) {
        if (ND == 0 || slots) {
#pragma unroll
            for (int u = 0; u < 4; ++u)
                x[u] = __builtin_bit_cast(float,
                                          __builtin_amdgcn_raw_buffer_load_b32(srs, voff + 4 * u, kb * kKB2 * 4, 0));
        }
    };

    // ---- the weights of block kb (K rows in buffer kb & 1) into W buffer kb & 1
    // ---- the weights of block kb (K rows in buffer kb & 1) into W buffer kb & 1
    auto make = [&](int kb, const float (&pre)[4]) {
        const int kbuf = kb & 1, nv = nvis(kb);
        if constexpr (ND == 0) {  // kept scores, loaded ahead into `pre`
            const uint32_t nz = wave_or_mask(block_weights<4>(pre, m, nv, &S.dig[kb & 1][0][0][0] + dofs, wsum, bad));
            if (lane == 0) S.mask[kb & 1][w] = nz;
            if (((kb + 1) % kCarry2) == 0) {
                whi += wsum >> 32;
                wsum &= 0xffffffffll;
            }
            return;
        }
        float stored[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        s_load(kb, stored);  // (rows with a score slot only: rare)
        const int2 kh = S.kh[kbuf][w >> 1];
        const int kcnt = __builtin_amdgcn_readfirstlane(kh.x), kbnd = __builtin_amdgcn_readfirstlane(kh.y);
        const bool crude = qcnt <= kQKmax && kcnt <= kQKmax && qbnd + kbnd <= 53;
        // pairs outside the exactness bound (rare): deferred, weight 0 here
        int chain = 0;
        if (!crude) {
            const int kk = kc0 + 4 * (lane >> 4);
            const int4 t0 = S.ki[kbuf][kk], t1 = S.ki[kbuf][kk + 1], t2 = S.ki[kbuf][kk + 2],
                       t3 = S.ki[kbuf][kk + 3];
            const int4 kis[4] = {t0, t1, t2, t3};
#pragma unroll
            for (int u = 0; u < 4; ++u)
                chain |= (u < nv && slot < 0 && qk_pair_class(qi, kis[u], kQKmax) == kPairChain) ? 1 << u : 0;
            if (chain) {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    if ((chain >> u) & 1) {
                        const int at = atomicAdd(&S.dn[par], 1);
                        if (at < kDef2) S.dl[at] = int2{r, kb * kKB2 + k0 + u};
                        else bad = true;
                    }
                }
            }
        }
        // the item's products (digit planes of the tile's Q rows and the block's K rows in LDS)
        v4i Cs[7];
#pragma unroll
        for (int c = 0; c < 7; ++c) Cs[c] = v4i{0, 0, 0, 0};
        const uint8_t *krow = S.kd[kbuf] + (kc0 + (lane & 15)) * KROW + 16 * (lane >> 4);
        const uint8_t *qrw = S.qd + (qr0 + (lane & 15)) * KROW + 16 * (lane >> 4);
        auto run = [&](auto nq) {
            constexpr int NQ = decltype(nq)::value;
#pragma unroll
            for (int n = 0; n < ND; ++n) {
                v4i Bq[NQ];
#pragma unroll
                for (int a = 0; a < NQ; ++a) Bq[a] = *(const v4i *)(qrw + a * 64 * ND + 64 * n);
#pragma unroll
                for (int c = 0; c < NQ; ++c) {
                    const v4i Ak = *(const v4i *)(krow + c * 64 * ND + 64 * n);
#pragma unroll
                    for (int a = 0; a < NQ; ++a)
                        Cs[a + c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(Ak, Bq[a], Cs[a + c], 0, 0, 0);
                }
            }
        };
        if (qcnt <= 3 && kcnt <= 3) run(std::integral_constant<int, 3>{});
        else run(std::integral_constant<int, kQKmax>{});
        const int4 kg4 = *(const int4 *)&S.kg[kbuf][kc0 + 4 * (lane >> 4)];
        const int kg[4] = {kg4.x, kg4.y, kg4.z, kg4.w};
        float sc[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            float v = (float)(A.src.scale * qk_dot_value<7>(Cs, u, qi.x + kg[u]));
            if (slots) v = slot >= 0 ? stored[u] : v;
            sc[u] = ((chain >> u) & 1) ? -__builtin_inff() : v;
        }
        // (the exponentials two keys at a time: fewer registers held)
        const uint32_t nz = wave_or_mask(block_weights<4, 2>(sc, m, nv, &S.dig[kb & 1][0][0][0] + dofs, wsum, bad));
        if (lane == 0) S.mask[kb & 1][w] = nz;
        if (((kb + 1) % kCarry2) == 0) {
            whi += wsum >> 32;
            wsum &= 0xffffffffll;
        }
    };

    // ---- block kb's products: W digits of buffer kb & 1 times this lane's V digits
    auto mult = [&](int kb, const v4i (&Vr)[BVT]) {
        if (!mine) return;
        const int buf = kb & 1;
        uint32_t mask = 0;
#pragma unroll
        for (int q = 0; q < kW2; ++q) mask |= S.mask[buf][q];
        mask = __builtin_amdgcn_readfirstlane(mask);
#pragma unroll
        for (int a = 0; a < kAw; ++a) {
            if (mask & (1u << a)) {
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const v4i Aw = *(const v4i *)(&S.dig[buf][t][a][0] + lane * 16);
#pragma unroll
                    for (int b = 0; b < BVT; ++b)
                        C[t][a + b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(Aw, Vr[b], C[t][a + b], 0, 0, 0);
                }
            }
        }
        if ((kb % kCarry2) == kCarry2 - 1) {
            // carry each class into the next so every partial sum stays far below
            // 2^31, and move the top class into its int64 part in LDS
#pragma unroll
            for (int t = 0; t < 2; ++t) {
#pragma unroll
                for (int c = 0; c < NC - 1; ++c) {
                    const v4i cc = C[t][c] >> 8;
                    C[t][c] -= cc << 8;
                    C[t][c + 1] += cc;
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) S.top[w][4 * t + q][lane] += C[t][NC - 1][q];
                C[t][NC - 1] = v4i{0, 0, 0, 0};
            }
        }
    };

    // ---- prologue: the tile's Q rows and K blocks 0 and 1 in LDS ([A]), block
    // 2 in registers; block 0's weights ([B])
    if constexpr (ND > 0) {
        const int8_t *qsrc = A.src.qdig + (bh * A.src.ni_pad + (T.it0 - A.i0)) * (int64_t)RB;
        for (int c = tid; c < 32 * RB / 16; c += 64 * kW2)
            *(v4i *)(S.qd + (c / (RB / 16)) * KROW + (c % (RB / 16)) * 16) = *(const v4i *)(qsrc + (int64_t)c * 16);
    }
    KSet kn;
    // kept scores of blocks 0 and 1 in the two register sets (each set takes
    // the block two further on once its weights are made)
    float s0[4] = {0.0f, 0.0f, 0.0f, 0.0f}, s1[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (nblk > 0) {
        KSet k1;
        if constexpr (ND == 0) {
            s_load(0, s0);
            if (nblk > 1) s_load(1, s1);
        }
        k_load(0, kn);
        if (nblk > 1) k_load(1, k1);
        k_store(0, kn);
        if (nblk > 1) k_store(1, k1);
        if (mine) v_load(0, VA);
    }
    __syncthreads();  // [A]
    if (nblk > 2) k_load(2, kn);
    if (nblk > 0) {
        make(0, s0);
        if constexpr (ND == 0)
            if (nblk > 2) s_load(2, s0);
    }
    __syncthreads();  // [B]
    // One step: block kb's products (its weights were made in the previous
    // step), then block kb+1's V digits into the same registers (they land
    // while the weights are made), block kb+1's weights, block kb+2's K rows
    // (in registers) into K buffer kb & 1 (block kb's, done with) and block
    // kb+3's into registers.
    // (kept scores: the loop is unrolled by two so the sets keep their roles)
    auto step = [&](int kb, float (&set)[4]) {
        mult(kb, VA);
        if (mine && kb + 1 < nblk) v_load(kb + 1, VA);
        if (kb + 1 < nblk) {
            make(kb + 1, set);
            if constexpr (ND == 0)
                if (kb + 3 < nblk) s_load(kb + 3, set);
        }
        if (kb + 2 < nblk) {
            k_store(kb & 1, kn);
            if (kb + 3 < nblk) k_load(kb + 3, kn);
        }
        __syncthreads();
    };
    if constexpr (ND == 0) {
        for (int kb = 0; kb < nblk; kb += 2) {
            step(kb, s1);
            if (kb + 1 < nblk) step(kb + 1, s0);
        }
    } else {
        for (int kb = 0; kb < nblk; ++kb) step(kb, s0);  // (no kept scores: the sets are unused)
    }

    // ---- deferred pairs, 64 at a time as the virtual keys of extra blocks:
    // their q and k rows into the K buffers ([E0]), their scores by the rule
    // itself, one lane of waves 0 and 1 per pair ([E1]), the weights of those
    // whose row is the lane's ([E2]); the multiplying role forms the V digits
    // of the pairs' keys from V itself as the slices do (the value toward zero
    // onto the column's grid; entries with bits below it are the remainders
    // added by k_pv_fix).  Block count and carry schedule continue.
    {
        const int ndef = min(S.dn[par], kDef2);
        const int D = (int)A.D;
        const bf16_t *qb = (const bf16_t *)A.src.q + T.b * A.src.qsB + T.hq * A.src.qsH;
        const bf16_t *kb0 = (const bf16_t *)A.src.k + T.b * A.src.ksB + (T.hq / A.group) * A.src.ksH;
        uint16_t *qs = (uint16_t *)S.kd[0], *ks = (uint16_t *)S.kd[1];
        const int g = (mine && d < A.D) ? A.colgrid[T.bhk * A.Dp32 + d] : 0;
        const int64_t vbase = T.b * A.vsB + (T.bhk % A.Hkv) * A.vsH + ((mine && d < A.D) ? d : 0);
        for (int x = 0; x < (ndef + 63) / 64; ++x) {
            for (int t = tid; t < 64 * D; t += 64 * kW2) {
                const int ee = t / D, dd = t - ee * D, e = 64 * x + ee;
                const int2 E = e < ndef ? S.dl[e] : int2{0, 0};  // (padding: the tile's first row and key)
                qs[t] = qb[(T.it0 + E.x) * A.src.qsS + dd].bits;
                ks[t] = kb0[(A.kv_lo + E.y) * A.src.ksS + dd].bits;
            }
            // V digits of the virtual keys for this lane's column
            if (mine) {
                uint64_t U[16];
#pragma unroll
                for (int p = 0; p < 16; ++p) {
                    const int e = 64 * x + 16 * (lane >> 4) + p;
                    const int64_t j = A.kv_lo + (e < ndef ? S.dl[e].y : 0);
                    const double v = A.vdtype == 0
                                         ? (double)((const float *)A.v)[vbase + j * A.vsS]
                                         : (double)elem<bf16_t>::to_f32(((const bf16_t *)A.v)[vbase + j * A.vsS]);
                    U[p] = (uint64_t)((int64_t)ldexp(d < A.D ? v : 0.0, -g) + 0x8080808080ll);
                }
#pragma unroll
                for (int b = 0; b < BVT; ++b) {
                    uint32_t w4[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        uint32_t pack = 0;
#pragma unroll
                        for (int u = 0; u < 4; ++u) pack |= ((uint32_t)(U[4 * q + u] >> (8 * b)) & 255u) << (8 * u);
                        w4[q] = pack ^ 0x80808080u;
                    }
                    VA[b] = v4i{(int)w4[0], (int)w4[1], (int)w4[2], (int)w4[3]};
                }
            }
            __syncthreads();  // [E0]
            if (tid < 64) {
                const int e = 64 * x + tid;
                double acc = 0.0;
#pragma unroll 8
                for (int dd = 0; dd < D; ++dd)
                    acc = fma((double)__uint_as_float((uint32_t)qs[tid * D + dd] << 16),
                              (double)__uint_as_float((uint32_t)ks[tid * D + dd] << 16), acc);
                S.dsc[tid] = e < ndef ? (float)(A.src.scale * acc) : -__builtin_inff();
            }
            __syncthreads();  // [E1]
            const int kbv = nblk + x;
            float sc[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int e = 64 * x + k0 + u;
                sc[u] = (e < ndef && S.dl[e].x == r) ? S.dsc[k0 + u] : -__builtin_inff();
            }
            const uint32_t nz =
                wave_or_mask(block_weights<4, 2>(sc, m, 4, &S.dig[kbv & 1][0][0][0] + dofs, wsum, bad));
            if (lane == 0) S.mask[kbv & 1][w] = nz;
            if (((kbv + 1) % kCarry2) == 0) {
                whi += wsum >> 32;
                wsum &= 0xffffffffll;
            }
            __syncthreads();  // [E2]
            mult(kbv, VA);
        }
    }

    // ---- exact row sums of W: the four lanes of a row, then the four waves of
    // a row tile add theirs in LDS (each wsum < 2^55; whi counts units of 2^32)
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
    if (w < 2 && lane < 16) {
        // DEN 2^46 = hi 2^32 + lo; RN64(DEN) correctly rounded from its 128 bits
        const int64_t hi = (int64_t)S.den_hi[par][r] + (int64_t)(S.den_lo[par][r] >> 32);
        const uint64_t lo = S.den_lo[par][r] & 0xffffffffull;
        S.d64[par][r] = i128_to_f64(hi >> 32, ((uint64_t)hi << 32) | lo, -kSw);
        if (A.stat_den && !generic && rowok) {  // (generic tiles write theirs in k_pv_fix)
            A.stat_den[bh * A.stat_rows + i] = S.d64[par][r];
            A.stat_m[bh * A.stat_rows + i] = m;
        }
    }
    __syncthreads();  // [D]: RN64(DEN) of every row is in LDS
    if (generic) {
        if (tid == 0) A.flags[bh * A.ntiles + tile] = kTileGeneric;
        return true;
    }
    if (tid == 0) A.flags[bh * A.ntiles + tile] = kTileDone;
    if (!mine) return false;

    // ---- the lane's outputs: dim d, rows 16 t + 4 (lane / 16) + q
    // carry the classes into bytes: C_0..C_(NC-2) in [0, 256), C_(NC-1) signed
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int c = 0; c < NC - 1; ++c) {
            const v4i cc = C[t][c] >> 8;
            C[t][c] &= 255;
            C[t][c + 1] += cc;
        }
    auto top = [&](int t, int q) -> int64_t {
        return (int64_t)C[t][NC - 1][q] + (longt ? S.top[w][4 * t + q][lane] : 0);
    };
    const int gcol = d < A.D ? A.colgrid[T.bhk * A.Dp32 + d] : 0;
    const bool dok = d < A.D;
    if (FUSED && ((T.rem >> G) & 1)) {
        // this group's remainders are added by k_pv_fix: its exact NUM goes to
        // the tile's 32-row digit scratch (cleared here), each row's RN64(DEN)
        // beside it, and is finalized there after the remainders
        const int64_t nplane = A.ntiles * 32 * (int64_t)gridDim.y * A.D;
        int64_t *nb = A.fb_num + (bh * A.ntiles + tile) * 32 * A.D;
        for (int t = lane; t < 32 * 16 * kNumDigits; t += 64) {
            const int k = t >> 9, rr = (t >> 4) & 31, c = t & 15;
            if (16 * w + c < A.D) nb[k * nplane + rr * A.D + 16 * w + c] = 0;
        }
        if (lane < 32) ((double *)A.fb_den)[(bh * A.ntiles + tile) * 32 + lane] = S.d64[par][lane];
        __threadfence();
    }
    const int nrows = (int)min64(32, T.i_end - T.it0);
    int ostride = (int)A.osS;
    asm volatile("" : "+s"(ostride));
    int64_t pbase = bh * A.rows_per_bh + (T.it0 - A.row0);
    asm volatile("" : "+s"(pbase));
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        float out[4];
        bool big = false;
        // NUM = P_hi 2^48 + P_lo with P_lo = bytes C_0..C_5 and P_hi = the classes
        // above (the top one signed): both exact in binary64 while |P_hi| < 2^53,
        // and then fma(P_hi, 2^48, P_lo) is the correctly rounded NUM; a larger
        // P_hi takes the 128-bit conversion
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int rr = 16 * t + 4 * (lane >> 4) + q;
            const uint64_t plo = (uint64_t)((uint32_t)C[t][0][q] | ((uint32_t)C[t][1][q] << 8) |
                                            ((uint32_t)C[t][2][q] << 16) | ((uint32_t)C[t][3][q] << 24)) |
                                 ((uint64_t)((uint32_t)C[t][4][q] | ((uint32_t)C[t][5][q] << 8)) << 32);
            int64_t phi = top(t, q);
#pragma unroll
            for (int c = NC - 2; c >= 6; --c) phi = phi * 256 + C[t][c][q];
            big |= (uint64_t)(phi + ((int64_t)1 << 53)) >= ((uint64_t)1 << 54);
            const double n64 = ldexp(fma((double)phi, 0x1p48, (double)plo), gcol - kSw);
            out[q] = FUSED ? (float)(n64 / S.d64[par][rr]) : 0.0f;
            (void)rr;
        }
        auto num_i128 = [&](int q, int64_t &hi, uint64_t &lo) {
            // value = P_hi 2^48 + P_lo as hi 2^64 + lo
            int64_t phi = top(t, q);
#pragma unroll
            for (int c = NC - 2; c >= 6; --c) phi = phi * 256 + C[t][c][q];
            const uint64_t plo = (uint64_t)((uint32_t)C[t][0][q] | ((uint32_t)C[t][1][q] << 8) |
                                            ((uint32_t)C[t][2][q] << 16) | ((uint32_t)C[t][3][q] << 24)) |
                                 ((uint64_t)((uint32_t)C[t][4][q] | ((uint32_t)C[t][5][q] << 8)) << 32);
            lo = ((uint64_t)phi << 48) | plo;
            hi = phi >> 16;
        };
        if (FUSED && ((T.rem >> G) & 1)) {
            if (dok) {
#pragma unroll 1
                for (int q = 0; q < 4; ++q) {
                    int64_t hi;
                    uint64_t lo;
                    num_i128(q, hi, lo);
                    const int rr = 16 * t + 4 * (lane >> 4) + q;
                    const __int128 num = (__int128)(((unsigned __int128)(uint64_t)hi << 64) | lo);
                    const int64_t nplane = A.ntiles * 32 * (int64_t)gridDim.y * A.D;
                    int64_t *nb = A.fb_num + (bh * A.ntiles + tile) * 32 * A.D;
                    add_i128_digits<kNumDigits>(num, gcol - kSw - kNumElo, nb + rr * A.D + d, nplane);
                }
            }
            continue;
        }
        if (FUSED) {
            if (big) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    int64_t hi;
                    uint64_t lo;
                    num_i128(q, hi, lo);
                    const int rr = 16 * t + 4 * (lane >> 4) + q;
                    out[q] = (float)(i128_to_f64(hi, lo, gcol - kSw) / S.d64[par][rr]);
                }
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) asm volatile("" ::"v"(out[q]));
            float *ob = A.o + T.b * A.osB + T.hq * A.osH + T.it0 * A.osS;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int rr = 16 * t + 4 * (lane >> 4) + q;
                if (rr < nrows && dok) ob[rr * ostride + (int)d] = out[q];
            }
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int rr = 16 * t + 4 * (lane >> 4) + q;
                if (rr >= nrows || !dok) continue;
                int64_t hi;
                uint64_t lo;
                num_i128(q, hi, lo);
                const __int128 num = (__int128)(((unsigned __int128)(uint64_t)hi << 64) | lo);
                const int64_t prow = pbase + rr;
                add_i128_digits<kNumDigits>(num, gcol - kSw - kNumElo, A.num + prow * A.D + d,
                                            A.plane_rows * A.D);
            }
        }
    }
    if (!FUSED && w == 0 && lane < 32 && lane < nrows) {
        const int64_t hi2 = (int64_t)S.den_hi[par][lane] + (int64_t)(S.den_lo[par][lane] >> 32);
        const int64_t lo2 = (int64_t)(S.den_lo[par][lane] & 0xffffffffull);
        add_i128_digits<kDenDigits>(((__int128)hi2 << 32) + lo2, -kSw - kDenElo, A.den + pbase + lane,
                                    A.plane_rows);
    }
    return false;
}

// One workgroup per tile, or for causal attention per pair of tiles (x,
// ntiles-1-x) whose key counts add up to the same total for every pair.
template <bool FUSED, int ND>
__global__ __launch_bounds__(64 * kW2, 2) void k_pv2(PvArgs A) {
    __shared__ __align__(16) Pv2Shared<ND> S;
    const GridPos gp = xcd_grouped_pos();
    const int64_t bh = gp.y, x = gp.x;
    const int npass = (A.causal && x != A.ntiles - 1 - x) ? 2 : 1;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll 1
    for (int pass = 0; pass < npass; ++pass) {
        const int64_t tile = (A.causal && pass == 0) ? A.ntiles - 1 - x : x;
        const PvTile T = pv_tile_of(A, bh, tile);
        if (T.badv) {
            if (threadIdx.x == 0) A.flags[bh * A.ntiles + tile] = kTileGeneric;
            continue;
        }
        if (threadIdx.x == 0) {  // (the previous pass's last barrier ordered its uses of these)
            S.bad[pass] = 0;
            S.dn[pass] = 0;
        }
        __syncthreads();
        // the wave's V digit count (4 stands for 1..4)
        const int64_t G = w >> 1;
        const int bv = 16 * w < A.D ? A.grpB[T.bhk * T.nG + G] : 0;
        if (bv > 4) pv2_tile<FUSED, ND, 5>(A, T, bh, tile, pass, S);
        else pv2_tile<FUSED, ND, 4>(A, T, bh, tile, pass, S);
    }
}

template <bool FUSED>
hipError_t launch_pv2_t(const PvArgs &a, int64_t bh, int nd, hipStream_t s) {
    dim3 grid((unsigned)(a.causal ? (a.ntiles + 1) / 2 : a.ntiles), (unsigned)bh);
    if (nd == 0) hipLaunchKernelGGL((k_pv2<FUSED, 0>), grid, dim3(64 * kW2), 0, s, a);
    else if (nd == 1) hipLaunchKernelGGL((k_pv2<FUSED, 1>), grid, dim3(64 * kW2), 0, s, a);
    else hipLaunchKernelGGL((k_pv2<FUSED, 2>), grid, dim3(64 * kW2), 0, s, a);
    return hipGetLastError();
}
template hipError_t launch_pv2_t<true>(const PvArgs &, int64_t, int, hipStream_t);
template hipError_t launch_pv2_t<false>(const PvArgs &, int64_t, int, hipStream_t);

}  // namespace det
