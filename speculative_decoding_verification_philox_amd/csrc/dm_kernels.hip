// dm_kernels.hip -- HIP kernels of the DropMatch verify step for gfx950.
//
//   k_prep        dropout masks from Philox, masked hidden rows in GEMM order
//                 (k_prep_packed: the same in matrix-core operand order)
//   k_pack_w      one-time reorder of the LM-head weight into panel order
//   k_gemm_panel  LM-head GEMM over panel-ordered W: one wave streams one
//                 panel of 64 vocabulary rows straight into MFMA operands,
//                 with a softmax-statistics epilogue per row and per centroid
//   k_gemm_tile   the same for many rows: four panels x one tile of up to
//                 160 rows per workgroup (a wave per panel), W streamed into
//                 a register ring, the masked rows shared through an LDS
//                 ring, two workgroups per CU, XCD-aware order
//   k_gemm_skinny LM-head GEMM over row-major W (all rows of a tile in one
//                 workgroup; W streamed from HBM straight into MFMA operands),
//                 same epilogue
//   k_combine     merges the per-vocabulary-group statistics
//   k_filter      top-k / top-p thresholds of the lossless targets (only when
//                 a filter is set)
//   k_vocab       Jensen-Shannon terms and the residual race over the
//                 vocabulary
//   k_finish      acceptance rule per drafted position, first-rejection
//                 scan and the emitted token, one workgroup per sequence
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dm_common.hpp"
#include "dm_launch.hpp"

namespace dmv {

typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// =====================================================================
// k_prep: Hm[rho, :] = h[b, t, :] * keep(b, t, i, :) for every GEMM row,
// plus the row's metadata for the LM-head epilogue.  A thread handles eight
// elements (two Philox blocks); grid = rows x (d / 2048).
// DropMatch Sec. 3.1 Eq. (1): independent Bernoulli(1 - p_drop) keeps per
// (position, head, element), drawn from Philox stream 0 with counter
// (j / 4, b * (gamma + 1) + t, i, 0).  The inverted-dropout scale of Eq. (2)
// is applied to the fp32 accumulator later, so masked values stay exact.
// Hm is written row-major, for the row-major-W kernel.
// =====================================================================
template <bool BF16>
__global__ __launch_bounds__(256) void k_prep(const Plan P, const void* __restrict__ h, void* __restrict__ Hm,
                                              RowMeta* __restrict__ meta, uint32_t* __restrict__ dbg_mask) {
    const int rho = blockIdx.x;
    const RowInfo ri = row_info(P, rho);
    if (blockIdx.y == 0 && threadIdx.x == 0) {
        RowMeta mt;
        const bool valid = ri.b >= 0;
        mt.canon = valid ? (ri.b * P.T1 + ri.t) * P.K + ri.i : -1;
        mt.scale = valid ? (ri.lossy ? seq_scale(P, ri.b) : P.scale_undropped) : 0.0f;
        mt.store = valid && (P.store_all || !ri.lossy || (bit_of(P.js_bits, ri.b) && ri.t < seq_G(P, ri.b)));
        mt.inv_k = valid && ri.lossy ? seq_inv_k(P, ri.b) : 0.0f;
        meta[rho] = mt;
    }
    // this thread: elements 8 e .. 8 e + 7 of the row
    const int e = blockIdx.y * blockDim.x + threadIdx.x;
    const int n8 = P.d >> 3;
    if (e >= n8) return;  // n8 is a multiple of 8: groups of four neighbours leave together
    constexpr int esz = BF16 ? 2 : 4;
    constexpr int NV = esz / 2;  // 16-byte pieces per 8 elements
    uint32_t bits = 0u;          // bit k: keep element 8 e + k
    if (ri.b >= 0) {
        if (ri.lossy) {
            const uint32_t pidx = (uint32_t)(ri.b * P.T1 + ri.t);
            const uint32_t thr = seq_thresh(P, ri.b);
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const u32x4 rr = philox10(u32x4{(uint32_t)(2 * e + q), pidx, (uint32_t)ri.i, kStreamMask}, P.key0, P.key1);
                bits |= (uint32_t)(rr.x >= thr) << (4 * q);
                bits |= (uint32_t)(rr.y >= thr) << (4 * q + 1);
                bits |= (uint32_t)(rr.z >= thr) << (4 * q + 2);
                bits |= (uint32_t)(rr.w >= thr) << (4 * q + 3);
            }
        } else {
            bits = 0xffu;
        }
    }
    const size_t src_row = ri.b >= 0 ? (size_t)(ri.b * P.T1 + ri.t) * P.d : 0;
    const uint8_t* src = (const uint8_t*)h + (src_row + (size_t)e * 8) * esz;
    const size_t row_bytes = (size_t)P.d * esz;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        v4u x = ri.b >= 0 ? *(const v4u*)(src + 16 * v) : v4u{0, 0, 0, 0};
        if (BF16) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t lo = (bits >> (2 * k)) & 1u, hi = (bits >> (2 * k + 1)) & 1u;
                x[k] = (lo ? (x[k] & 0x0000ffffu) : 0u) | (hi ? (x[k] & 0xffff0000u) : 0u);
            }
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) x[k] = ((bits >> (4 * v + k)) & 1u) ? x[k] : 0u;
        }
        const size_t o = (size_t)e * 8 * esz + 16 * v;  // byte offset within the row
        *(v4u*)((uint8_t*)Hm + (size_t)rho * row_bytes + o) = x;
    }
    if (dbg_mask) {
        // four neighbouring threads hold the 32 bits of one mask word
        uint32_t word = bits << (8 * (e & 3));
        word |= __shfl_xor(word, 1, 64);
        word |= __shfl_xor(word, 2, 64);
        if (ri.b >= 0 && (e & 3) == 0) dbg_mask[((size_t)(ri.b * P.T1 + ri.t) * P.K + ri.i) * (P.d >> 5) + (e >> 2)] = word;
    }
}

// =====================================================================
// k_prep_packed: the same masked rows, written in matrix-core operand order
// (per tile: [fragment kb][sub-tile m][lane][16 B], lane 16 a + r holding
// bytes 64 kb + 16 a .. + 16 of sub-tile row r) for the panel-order kernels.
// One thread per 16-byte piece of the output (PPT = 1), or, for large plans,
// per PPT = 4 pieces of one row in consecutive fragments, so the row lookup
// and the index arithmetic are paid once per four (the Philox rounds stay
// one block per four elements).  Consecutive threads write consecutive
// bytes; the source row piece is gathered from h (L2-resident).
// =====================================================================
// Pieces from which the launch gives each thread four of them: at the
// batched 70B (2^20.3 pieces, 1280 blocks) the masking took 14.7 against
// 18.0 us; at the 60-node tree (2^18.3 pieces, 320 blocks, too few to hide
// latency) 9.1 against 7.8 us, so that plan keeps one piece per thread.
constexpr size_t kPrepFourMin = (size_t)1 << 19;

template <bool BF16, int PPT>
__global__ __launch_bounds__(256) void k_prep_packed(const Plan P, const void* __restrict__ h, void* __restrict__ Hm,
                                                     RowMeta* __restrict__ meta, uint32_t* __restrict__ dbg_mask) {
    constexpr int esz = BF16 ? 2 : 4;
    constexpr int EPP = 16 / esz;  // elements per 16-byte piece
    const size_t qt = (size_t)blockIdx.x * 256 + threadIdx.x;
    const uint32_t msub = (uint32_t)P.msub, nkq = (uint32_t)(P.nkb / PPT);
    if (qt >= (size_t)P.R_phys * nkq * 4) return;
    const int lane = (int)(qt & 63);
    // (tile * nkq + kq) * msub + m: at most R_phys * nkb / 16 fragments, far
    // below 2^32, so the index splits in 32-bit arithmetic
    const uint32_t frag = (uint32_t)(qt >> 6);
    const uint32_t tk = frag / msub;
    const int m = (int)(frag - tk * msub);
    const uint32_t tile_u = tk / nkq;
    const int kb0 = (int)(tk - tile_u * nkq) * PPT;  // this thread's first fragment
    const int tile = (int)tile_u;
    const int r = 16 * m + (lane & 15);
    const int rho = tile * P.MT + r;
    const RowInfo ri = row_info(P, rho);
    if (kb0 == 0 && (lane >> 4) == 0) {
        RowMeta mt;
        const bool valid = ri.b >= 0;
        mt.canon = valid ? (ri.b * P.T1 + ri.t) * P.K + ri.i : -1;
        mt.scale = valid ? (ri.lossy ? seq_scale(P, ri.b) : P.scale_undropped) : 0.0f;
        mt.store = valid && (P.store_all || !ri.lossy || (bit_of(P.js_bits, ri.b) && ri.t < seq_G(P, ri.b)));
        mt.inv_k = valid && ri.lossy ? seq_inv_k(P, ri.b) : 0.0f;
        meta[rho] = mt;
    }
    const uint32_t pidx = ri.b >= 0 ? (uint32_t)(ri.b * P.T1 + ri.t) : 0u;
    const uint32_t thr = ri.b >= 0 && ri.lossy ? seq_thresh(P, ri.b) : 0u;
    const uint8_t* hrow = (const uint8_t*)h + ((size_t)pidx * P.d) * esz;
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
        const int kb = kb0 + j;
        const int o = kb * 64 + (lane >> 4) * 16;  // byte offset within the row
        const int e0 = o / esz;                   // first element of the piece
        uint32_t bits = 0u;                       // bit k: keep element e0 + k
        if (ri.b >= 0) {
            if (ri.lossy) {
#pragma unroll
                for (int qq = 0; qq < EPP / 4; ++qq) {
                    const u32x4 rr = philox10(u32x4{(uint32_t)(e0 / 4 + qq), pidx, (uint32_t)ri.i, kStreamMask},
                                              P.key0, P.key1);
                    bits |= (uint32_t)(rr.x >= thr) << (4 * qq);
                    bits |= (uint32_t)(rr.y >= thr) << (4 * qq + 1);
                    bits |= (uint32_t)(rr.z >= thr) << (4 * qq + 2);
                    bits |= (uint32_t)(rr.w >= thr) << (4 * qq + 3);
                }
            } else {
                bits = (1u << EPP) - 1u;
            }
        }
        v4u x = v4u{0, 0, 0, 0};
        if (ri.b >= 0) x = *(const v4u*)(hrow + o);
        if (BF16) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t lo = (bits >> (2 * k)) & 1u, hi = (bits >> (2 * k + 1)) & 1u;
                x[k] = (lo ? (x[k] & 0x0000ffffu) : 0u) | (hi ? (x[k] & 0xffff0000u) : 0u);
            }
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) x[k] = ((bits >> k) & 1u) ? x[k] : 0u;
        }
        const size_t q = (((size_t)tile * P.nkb + kb) * msub + m) * 64 + lane;  // consecutive lanes, consecutive pieces
        *(v4u*)((uint8_t*)Hm + q * 16) = x;
        if (dbg_mask && ri.b >= 0)  // keep bits of this piece into their mask word (the word starts zeroed)
            atomicOr(&dbg_mask[((size_t)(ri.b * P.T1 + ri.t) * P.K + ri.i) * (P.d >> 5) + (e0 >> 5)],
                     bits << (e0 & 31));
    }
}

// =====================================================================
// k_pack_w: row-major W -> panel order (see dm_verify_pack_w).  One thread
// per 16-byte piece of the packed buffer.
// =====================================================================
__global__ __launch_bounds__(256) void k_pack_w(const uint8_t* __restrict__ W, uint8_t* __restrict__ Wp, int V,
                                                int nkb, size_t n16) {
    const size_t q = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (q >= n16) return;
    const int lane = (int)(q & 63), g = (int)((q >> 6) & 3);
    const size_t rest = q >> 8;
    const int kb = (int)(rest % (size_t)nkb);
    const size_t panel = rest / (size_t)nkb;
    const size_t row = panel * 64 + (size_t)g * 16 + (lane & 15);
    const size_t row_bytes = (size_t)nkb * 64;
    v4u x = v4u{0, 0, 0, 0};
    if (row < (size_t)V) x = *(const v4u*)(W + row * row_bytes + (size_t)kb * 64 + (lane >> 4) * 16);
    *(v4u*)(Wp + q * 16) = x;
}

// Centroid weight of lossy position p: 1 / K_b of its sequence.  Rows of
// heads past K_b are padding rows whose values are exactly 0, so a sum over
// all K slots in head order equals the sum over the K_b heads.
__device__ __forceinline__ float lossy_pos_inv_k(const Plan& P, int p) {
    if (!P.ragged || p >= P.n_lossy_pos) return P.inv_k;
    int b, t;
    class_pos(P, 0, p, &b, &t);
    return seq_inv_k(P, b);
}

// =====================================================================
// k_gemm_panel: L[rho, v] = scale(rho) * sum_j W[v, j] * Hm[rho, j]
// (DropMatch Eq. (3), the shared head W) for one tile of up to 64 rows and
// one panel of 64 vocabulary rows per wave, W in panel order; a workgroup's
// four waves take four neighbouring panels of one tile.
//
// Main loop: the wave streams its panel front to back, 1 KiB per load
// instruction (non-temporal: W is read once), four strips of 16 vocabulary
// rows per 64-byte fragment; the tile's masked rows come from the packed Hm
// (L2-resident, shared by every wave).  The next fragment's loads are in
// flight while the current one feeds v_mfma_f32_16x16x32_bf16 (16x16x4 for
// fp32).  No LDS and no barrier in the loop.  A grid of fewer waves than the
// GPU has SIMDs (DEEP) keeps three stages in flight instead: with the
// bandwidth not shared, each wave is bound by the latency of its loads.
//
// Epilogue, straight from the accumulators: lane 16 a + c holds column
// 16 g + c of rows 16 m + 4 a + j.  Rows later passes need are stored; per
// row, (max, sum exp, argmax) over the panel's 64 columns comes from the
// lane's four columns and DPP reductions over the 16 lanes of its row.  A
// position's K head rows sit in one lane group (slot layout), so its
// centroid (the mean of the heads, DropMatch Eq. (5)) is formed in-lane and
// reduced the same way.  The four waves' results are merged in panel order
// through LDS into part[target][panel group].
// =====================================================================
constexpr int kPanelWaves = 4;
constexpr int kPanelStrips = 4;
constexpr int kPanelNK = 1;  // fragments per pipeline stage
constexpr int kPanelDeepRing = 4;  // register ring of the few-wave variant

// Reductions over the 16 lanes of a DPP row (lanes 16 a .. 16 a + 15): swap
// neighbours, then pairs, then mirror within each half row, then within the
// row; every lane ends with the same value, formed in the same order.
constexpr int kDppXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;  // row_half_mirror
constexpr int kDppMirror = 0x140;      // row_mirror

// Every lane of these patterns reads a lane of its own row, so bound_ctrl
// changes nothing; it lets the compiler fold the move into the ALU op.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
    return __builtin_amdgcn_mov_dpp(x, CTRL, 0xF, 0xF, true);
}
__device__ __forceinline__ int row16_min(int x) {
    x = min(x, dpp_i<kDppXor1>(x));
    x = min(x, dpp_i<kDppXor2>(x));
    x = min(x, dpp_i<kDppHalfMirror>(x));
    return min(x, dpp_i<kDppMirror>(x));
}

constexpr float kLog2e = 1.44269504088896341f;

// A compile-time bool carried as an argument, so one generic lambda gives
// two specialised epilogues.
template <bool B>
struct BoolTag {
    static constexpr bool value = B;
};

// Order-preserving map from a float's bits to a signed integer, its own
// inverse: on non-NaN values integer order is float order (-0 sorts just
// below +0, and the two compare equal afterwards).  The 16-lane max runs on
// these keys because the integer max takes the DPP lane move as an operand
// modifier, where a float max would first quiet a possible NaN.
__device__ __forceinline__ int fkey(float x) {
    const int b = __float_as_int(x);
    return b ^ (int)((uint32_t)(b >> 31) >> 1);
}
__device__ __forceinline__ float fkey_inv(int k) { return __int_as_float(k ^ (int)((uint32_t)(k >> 31) >> 1)); }

// 4 x 4 transpose inside each quad of lanes (lanes 4n .. 4n + 3; k = the
// lane's place in its quad): on entry lane k holds t[j] = element (j, k) of
// the quad's block, on exit t[i] = element (k, i).  Two butterfly steps:
// lanes k and k ^ 1 swap the elements whose index differs from k in bit 0,
// then lanes k and k ^ 2 those differing in bit 1.
__device__ __forceinline__ void quad_transpose(float (&t)[4], int k) {
    const bool odd = k & 1, hi = k & 2;
#pragma unroll
    for (int e = 0; e < 4; e += 2) {
        const float recv = dpp_f<kDppXor1>(odd ? t[e] : t[e + 1]);
        if (odd)
            t[e] = recv;
        else
            t[e + 1] = recv;
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const float recv = dpp_f<kDppXor2>(hi ? t[e] : t[e + 2]);
        if (hi)
            t[e] = recv;
        else
            t[e + 2] = recv;
    }
}

// (max, sum exp, lowest argmax) of J rows, each held as G values per lane by
// the 16 lanes of a DPP row (lane c holds columns col0 + 16 g); the J
// reductions are independent, so their DPP steps interleave.
//
// FULL: every column is a vocabulary entry, so no lane-out test is needed
// and the values are finite; e^(x - m) is taken as 2^(x log2 e - m log2 e).
// Otherwise columns with ok[g] false are left out by selects (they add
// exactly 0 to the sum and -inf to the max), and a row with no column at all
// gives the empty statistic.
template <int J, int G, bool FULL>
__device__ __forceinline__ void row16_stats(const float (&x)[J][G], const bool (&ok)[G], int col0, Stat (&out)[J]) {
    float m[J], s[J];
    int k[J], idx[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        float mm = (FULL || ok[0]) ? x[j][0] : -INFINITY;
#pragma unroll
        for (int g = 1; g < G; ++g) mm = fmaxf(mm, (FULL || ok[g]) ? x[j][g] : -INFINITY);
        k[j] = fkey(mm);
    }
#pragma unroll
    for (int j = 0; j < J; ++j) k[j] = max(k[j], dpp_i<kDppXor1>(k[j]));
#pragma unroll
    for (int j = 0; j < J; ++j) k[j] = max(k[j], dpp_i<kDppXor2>(k[j]));
#pragma unroll
    for (int j = 0; j < J; ++j) k[j] = max(k[j], dpp_i<kDppHalfMirror>(k[j]));
#pragma unroll
    for (int j = 0; j < J; ++j) k[j] = max(k[j], dpp_i<kDppMirror>(k[j]));
#pragma unroll
    for (int j = 0; j < J; ++j) {
        m[j] = fkey_inv(k[j]);
        s[j] = 0.0f;
        idx[j] = 0x7fffffff;
        if (FULL) {
            const float ml = m[j] * kLog2e;
#pragma unroll
            for (int g = 0; g < G; ++g) s[j] += __builtin_amdgcn_exp2f(fmaf(x[j][g], kLog2e, -ml));
            // the lowest column attaining the max: the last write is the smallest g
#pragma unroll
            for (int g = G - 1; g >= 0; --g) idx[j] = x[j][g] == m[j] ? col0 + 16 * g : idx[j];
        } else {
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float e = __expf(x[j][g] - m[j]);
                s[j] += ok[g] ? e : 0.0f;
                idx[j] = (ok[g] && x[j][g] == m[j]) ? min(idx[j], col0 + 16 * g) : idx[j];
            }
        }
    }
#pragma unroll
    for (int j = 0; j < J; ++j) {
        s[j] = s[j] + dpp_f<kDppXor1>(s[j]);
        idx[j] = min(idx[j], dpp_i<kDppXor1>(idx[j]));
    }
#pragma unroll
    for (int j = 0; j < J; ++j) {
        s[j] = s[j] + dpp_f<kDppXor2>(s[j]);
        idx[j] = min(idx[j], dpp_i<kDppXor2>(idx[j]));
    }
#pragma unroll
    for (int j = 0; j < J; ++j) {
        s[j] = s[j] + dpp_f<kDppHalfMirror>(s[j]);
        idx[j] = min(idx[j], dpp_i<kDppHalfMirror>(idx[j]));
    }
#pragma unroll
    for (int j = 0; j < J; ++j) {
        s[j] = s[j] + dpp_f<kDppMirror>(s[j]);
        idx[j] = min(idx[j], dpp_i<kDppMirror>(idx[j]));
    }
#pragma unroll
    for (int j = 0; j < J; ++j) out[j] = Stat{m[j], s[j], idx[j]};
}

// Running centroid of the lossy positions in a lane group: the group's head
// slots are visited in order, slot lam being head i of position `slot` (i and
// slot advance with lam, i wrapping at K; both uniform).  The head rows are
// summed in head order as they go by (the order every kernel uses for the
// centroid, see centroid_logit) and the position's statistics are taken at
// its last head.  ACC(lam, g) yields the scaled row value of slot lam and
// INVW(p) the centroid weight (1 / K_b) of the lane group's p-th position.
#define DM_CENTROID_PASS(NSLOT, ACC, INVW, write, dst)                          \
    do {                                                                            \
        float csum_[G];                                                             \
        int i_ = 0, slot_ = 0;                                                      \
        _Pragma("unroll") for (int lam_ = 0; lam_ < (NSLOT); ++lam_) {              \
            if (i_ == 0) {                                                          \
                _Pragma("unroll") for (int g_ = 0; g_ < G; ++g_) csum_[g_] = ACC(lam_, g_); \
            } else {                                                                \
                _Pragma("unroll") for (int g_ = 0; g_ < G; ++g_) csum_[g_] += ACC(lam_, g_); \
            }                                                                       \
            if (i_ == P.K - 1) {                                                    \
                if (slot_ < P.ppg) {                                                \
                    const float inv_ = INVW(slot_);                              \
                    float xc_[1][G];                                                \
                    _Pragma("unroll") for (int g_ = 0; g_ < G; ++g_) xc_[0][g_] = csum_[g_] * inv_; \
                    Stat st_[1];                                                    \
                    row16_stats<1, G, FULL>(xc_, ok, col0, st_);                    \
                    if (write) (dst)[slot_] = st_[0];                               \
                }                                                                   \
                i_ = 0;                                                             \
                ++slot_;                                                            \
            } else {                                                                \
                ++i_;                                                               \
            }                                                                       \
        }                                                                           \
    } while (0)

// The same pass with the head count KC fixed at compile time: a position's
// KC slots are summed in head order exactly as above, and then the
// statistics of all NSLOT / KC positions of the lane group are reduced
// together, so their DPP steps interleave instead of running one position
// after another.
#define DM_CENTROID_K(KC, NSLOT, ACC, INVW, write, dst)                        \
    do {                                                                           \
        constexpr int NP_ = (NSLOT) / (KC);                                        \
        if constexpr (NP_ > 0) {                                                   \
            float xc_[NP_ > 0 ? NP_ : 1][G];                                       \
            _Pragma("unroll") for (int p_ = 0; p_ < NP_; ++p_) {                    \
                const float inv_ = INVW(p_);                                     \
                _Pragma("unroll") for (int g_ = 0; g_ < G; ++g_) {                 \
                    float s_ = ACC(p_ * (KC), g_);                                  \
                    _Pragma("unroll") for (int i_ = 1; i_ < (KC); ++i_) s_ += ACC(p_ * (KC) + i_, g_); \
                    xc_[p_][g_] = s_ * inv_;                                        \
                }                                                                  \
            }                                                                      \
            Stat st_[NP_ > 0 ? NP_ : 1];                                           \
            row16_stats<NP_, G, FULL>(xc_, ok, col0, st_);                          \
            if (write) {                                                           \
                _Pragma("unroll") for (int p_ = 0; p_ < NP_; ++p_) (dst)[p_] = st_[p_]; \
            }                                                                      \
        }                                                                          \
    } while (0)

// Centroid statistics of a lane group: the common head counts take the
// interleaved pass on full panels, every other case the running one.
#define DM_CENTROIDS(NSLOT, ACC, INVW, write, dst)                             \
    do {                                                                           \
        if (FULL && P.K == 5)                                                      \
            DM_CENTROID_K(5, NSLOT, ACC, INVW, write, dst);                     \
        else if (FULL && P.K == 8)                                                 \
            DM_CENTROID_K(8, NSLOT, ACC, INVW, write, dst);                     \
        else                                                                       \
            DM_CENTROID_PASS(NSLOT, ACC, INVW, write, dst);                    \
    } while (0)

template <bool BF16, int MSUB, bool DEEP>
__global__ __launch_bounds__(kPanelWaves * 64, DEEP ? 1 : 2) void k_gemm_panel(const Plan P, const uint8_t* __restrict__ Wp,
                                                                 const uint8_t* __restrict__ Hp,
                                                                 const RowMeta* __restrict__ meta,
                                                                 float* __restrict__ logits,
                                                                 Stat* __restrict__ part) {
    constexpr int ROWS = 16 * MSUB, G = kPanelStrips, NK = kPanelNK;
    constexpr int SLOTS = ROWS + 64;  // rows, then centroid slots (at most 4 groups x 16)
    __shared__ Stat s_st[kPanelWaves][SLOTS];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int tile = blockIdx.y;
    const int panel_raw = blockIdx.x * kPanelWaves + wave;
    const bool active = panel_raw < P.n_panels;  // a wave past the last panel only joins the merge
    const int panel = active ? panel_raw : P.n_panels - 1;
    const int nkb = P.nkb;

    // metadata of tile row `lane`, fetched now, read through shuffles later
    RowMeta my = RowMeta{-1, 0.0f, 0, 0.0f};
    if (lane < ROWS) my = meta[(size_t)tile * ROWS + lane];

    v4f acc[G][MSUB];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int m = 0; m < MSUB; ++m) acc[g][m] = v4f{0.f, 0.f, 0.f, 0.f};
    if (active) {
        const uint8_t* wp = Wp + (size_t)panel * nkb * G * 1024 + lane * 16;
        const uint8_t* ap = Hp + (size_t)tile * nkb * MSUB * 1024 + lane * 16;
        auto mma = [&](const v4u (&w)[G], const v4u (&a)[MSUB]) {
#pragma unroll
            for (int g = 0; g < G; ++g)
#pragma unroll
                for (int m = 0; m < MSUB; ++m) {
                    if (BF16) {
                        acc[g][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(v8bf, a[m]), __builtin_bit_cast(v8bf, w[g]), acc[g][m], 0, 0, 0);
                    } else {
                        const v4f a4 = __builtin_bit_cast(v4f, a[m]);
                        const v4f b4 = __builtin_bit_cast(v4f, w[g]);
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            acc[g][m] = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[e], b4[e], acc[g][m], 0, 0, 0);
                    }
                }
        };
        if constexpr (DEEP) {
            // Few waves on the whole GPU: each is bound by load latency, not
            // by a share of the bandwidth, so it keeps D - 1 stages in flight
            // while multiplying one (same stages, same order of products).
            constexpr int D = kPanelDeepRing;
            v4u wb[D][G], ab[D][MSUB];
            auto load = [&](int slot, int kb) {
#pragma unroll
                for (int g = 0; g < G; ++g)
                    wb[slot][g] = __builtin_nontemporal_load((const v4u*)(wp + ((size_t)kb * G + g) * 1024));
#pragma unroll
                for (int m = 0; m < MSUB; ++m) ab[slot][m] = *(const v4u*)(ap + ((size_t)kb * MSUB + m) * 1024);
            };
            // prologue: stages 0 .. D - 2 (a row shorter than that re-reads its
            // last fragment, never multiplied)
#pragma unroll
            for (int st = 0; st < D - 1; ++st) load(st, min(st, nkb - 1));
            // steady state: every load a live stage and the same number of
            // loads per step, so each wait is the fixed count issued after
            int kb0 = 0;
            for (; kb0 + 2 * D - 1 <= nkb; kb0 += D) {
#pragma unroll
                for (int k = 0; k < D; ++k) {
                    load((k + D - 1) % D, kb0 + k + D - 1);  // the slot multiplied one step ago
                    __builtin_amdgcn_sched_barrier(0);
                    mma(wb[k], ab[k]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            // tail: at most 2 D - 2 stages, D - 1 of them already loaded
#pragma unroll
            for (int k = 0; k < 2 * D - 2; ++k) {
                if (kb0 + k < nkb) {
                    if (kb0 + k + D - 1 < nkb) load((k + D - 1) % D, kb0 + k + D - 1);
                    mma(wb[k % D], ab[k % D]);
                }
            }
        } else {
            v4u wc[NK][G], ac[NK][MSUB], wn[NK][G], an[NK][MSUB];
            auto load = [&](v4u (&w)[NK][G], v4u (&a)[NK][MSUB], int kb0) {
#pragma unroll
                for (int k = 0; k < NK; ++k) {
#pragma unroll
                    for (int g = 0; g < G; ++g)
                        w[k][g] = __builtin_nontemporal_load((const v4u*)(wp + ((size_t)(kb0 + k) * G + g) * 1024));
#pragma unroll
                    for (int m = 0; m < MSUB; ++m) a[k][m] = *(const v4u*)(ap + ((size_t)(kb0 + k) * MSUB + m) * 1024);
                }
            };
            load(wc, ac, 0);
            for (int kb0 = 0; kb0 < nkb; kb0 += NK) {
                if (kb0 + NK < nkb) load(wn, an, kb0 + NK);
#pragma unroll
                for (int k = 0; k < NK; ++k)
#pragma unroll
                    for (int g = 0; g < G; ++g)
#pragma unroll
                        for (int m = 0; m < MSUB; ++m) {
                            if (BF16) {
                                acc[g][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                    __builtin_bit_cast(v8bf, ac[k][m]), __builtin_bit_cast(v8bf, wc[k][g]), acc[g][m], 0,
                                    0, 0);
                            } else {
                                const v4f a = __builtin_bit_cast(v4f, ac[k][m]);
                                const v4f b = __builtin_bit_cast(v4f, wc[k][g]);
#pragma unroll
                                for (int e = 0; e < 4; ++e)
                                    acc[g][m] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], acc[g][m], 0, 0, 0);
                            }
                        }
#pragma unroll
                for (int k = 0; k < NK; ++k) {
#pragma unroll
                    for (int g = 0; g < G; ++g) wc[k][g] = wn[k][g];
#pragma unroll
                    for (int m = 0; m < MSUB; ++m) ac[k][m] = an[k][m];
                }
            }
        }
    }

    // ---------------- epilogue ----------------
    const int grp = lane >> 4, c = lane & 15;
    const int col0 = panel * 64 + c;
    bool ok[G];
#pragma unroll
    for (int g = 0; g < G; ++g) ok[g] = active && col0 + 16 * g < P.V;
    const int npt = P.GR * P.ppg;
    const bool lossy_tile = tile < P.tiles_lossy;
    // FULL: the panel lies wholly inside the vocabulary (every panel but
    // possibly the last), so its statistics need no per-column selects
    auto epilogue = [&](auto full) __attribute__((always_inline)) {
        constexpr bool FULL = decltype(full)::value;
#pragma unroll
        for (int m = 0; m < MSUB; ++m) {
            // the lane group's four rows of sub-tile m together
            float sc[4], x[4][G];
            int canon[4], store[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * m + 4 * grp + j;
                sc[j] = __shfl(my.scale, r, 64);
                canon[j] = __shfl(my.canon, r, 64);
                store[j] = __shfl(my.store, r, 64);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    x[j][g] = acc[g][m][j] * sc[j];
                    acc[g][m][j] = x[j][g];
                }
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (canon[j] >= 0 && store[j]) {  // the whole 16-lane row agrees
#pragma unroll
                    for (int g = 0; g < G; ++g)
                        if (FULL || ok[g]) logits[(size_t)canon[j] * P.V + col0 + 16 * g] = x[j][g];
                }
            Stat st[4];
            row16_stats<4, G, FULL>(x, ok, col0, st);
            if (c == 0) {
#pragma unroll
                for (int j = 0; j < 4; ++j) s_st[wave][16 * m + 4 * grp + j] = canon[j] >= 0 ? st[j] : stat_empty();
            }
        }
        if (lossy_tile) {
#define DM_ACC(lam, g) acc[g][(lam) >> 2][(lam) & 3]
            // a ragged batch's weight sits in the metadata of the position's first head row
#define DM_INVW(p) (P.ragged ? __shfl(my.inv_k, 16 * (((p) * P.K) >> 2) + 4 * grp + (((p) * P.K) & 3), 64) : P.inv_k)
            DM_CENTROIDS(4 * MSUB, DM_ACC, DM_INVW, c == 0, &s_st[wave][ROWS + grp * P.ppg]);
#undef DM_INVW
#undef DM_ACC
        }
    };
    if (active && (panel + 1) * 64 <= P.V)
        epilogue(BoolTag<true>{});
    else
        epilogue(BoolTag<false>{});
    __syncthreads();
    // merge the workgroup's panels in panel order: part[target][panel group]
    const int nloc = ROWS + (lossy_tile ? npt : 0);
    for (int t = threadIdx.x; t < nloc; t += blockDim.x) {
        Stat st = s_st[0][t];
#pragma unroll
        for (int w = 1; w < kPanelWaves; ++w) st = stat_merge(st, s_st[w][t]);
        int target = tile * ROWS + t;
        if (t >= ROWS) {
            const int p = tile * npt + (t - ROWS);
            if (p >= P.n_lossy_pos) continue;
            target = P.R_phys + p;
        }
        part[(size_t)target * P.n_vgroups + blockIdx.x] = st;
    }
}

// =====================================================================
// k_gemm_tile: the LM head for many rows (the matrix-core-bound regime):
// L[rho, v] = scale(rho) * sum_j W[v, j] * Hm[rho, j] (DropMatch Eq. (3)
// with the shared head W).  One workgroup computes one group of four panels
// (256 vocabulary columns) against one row tile of 16 * MSUB rows; wave w
// owns panel w of the group.
//
// A stage is one 64-byte slice of the reduction index.  Its masked-row
// fragments (MSUB of 1 KiB, each read by all four waves) are copied from
// global memory straight into a D-deep LDS ring (direct global-to-LDS
// loads, 16 bytes per lane, dealt round-robin to the waves).  Its weight
// fragments are read by one wave only, so each wave streams its panel's four
// fragments (4 KiB, already in operand order) from global memory straight
// into a D-deep register ring: the weight never passes through LDS.  Every
// wave issues the same loads at every stage (a wave short of a masked-row
// fragment copies one into a spare LDS area; stages past the end re-read the
// last one into slots never read), so every wait is an exact count.  Up to
// eight sub-tiles, per stage a wave issues the loads of the stage D - 1
// ahead, multiplies the current one (4 x MSUB v_mfma_f32_16x16x32_bf16;
// 16x16x4 for fp32), waits until its loads of the next stage have landed and
// meets the other waves at a bare s_barrier (the workgroup fence of an
// ordinary barrier would also wait for the loads of the later stages still
// in flight).  At nine and ten sub-tiles the registers hold only two stages
// of W beyond the accumulators, so the stages go in pairs: one pair in
// flight while the other is multiplied, and one barrier per pair.
//
// Two workgroups share a CU, each meeting only its own barrier, so one feeds
// the matrix cores while the other waits.  Blocks are mapped so that the
// tiles sharing a panel group run together on one XCD (workgroups go to the
// eight XCDs in turn), where the group's W is read from HBM once and then
// from that XCD's L2.
//
// The epilogue (in the ring's memory): statistics per row and per centroid
// over each wave's 64 columns, merged across the four panels into
// part[target][panel group]; stored rows written 16 bytes per lane (a
// transpose inside each quad of lanes turns the matrix-core output, four
// rows of one column per lane, into four columns of one row).
// =====================================================================
constexpr int kTileWaves = 4;  // 64-column panels per workgroup, one wave each

// The LDS ring holds D = 4 stages.  Up to eight sub-tiles the register ring
// of W holds four single stages (16 VGPRs each, three in flight) and the
// waves meet once per stage; at nine and ten sub-tiles, where the 16 * MSUB
// accumulators leave room for 64 ring registers only, it holds two pairs of
// stages (one pair in flight) and the waves meet once per pair.
template <int MSUB>
struct TileShape {
    static constexpr int D = 4;
    static constexpr bool PAIRS = MSUB >= 9;
    static constexpr int NA = (MSUB + kTileWaves - 1) / kTileWaves;  // masked-row loads per wave per stage
    static constexpr int STAGE = MSUB * 1024;
    static constexpr int SPARE = D * STAGE;  // where a wave short of a fragment loads one
    static constexpr int RING = SPARE + 1024;
    static constexpr int EPI = kTileWaves * 2 * 16 * MSUB * (int)sizeof(Stat) + 16 * MSUB * (int)sizeof(RowMeta);
    static constexpr int LDS = RING > EPI ? RING : EPI;
};

#define DM_AS_GLOBAL __attribute__((address_space(1)))
#define DM_AS_LDS __attribute__((address_space(3)))

// s_waitcnt vmcnt(N), other counters left alone (gfx9 encoding: vmcnt bits
// 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt is six bits");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Barrier between ring stages: this wave's LDS reads are complete
// (lgkmcnt 0) and its loads of the next stage have landed (waited for by
// the caller).  The memory clobber keeps the compiler from moving any memory
// access across it.
__device__ __forceinline__ void ring_barrier() {
    __builtin_amdgcn_s_waitcnt((0xF) | (0x3 << 14) | (0x7 << 4));  // lgkmcnt(0)
    asm volatile("s_barrier" ::: "memory");
}

template <bool BF16, int MSUB>
__global__ __launch_bounds__(kTileWaves * 64, 2) void k_gemm_tile(const Plan P, const uint8_t* __restrict__ Wp,
                                                                  const uint8_t* __restrict__ Hp,
                                                                  const RowMeta* __restrict__ meta,
                                                                  float* __restrict__ logits,
                                                                  Stat* __restrict__ part) {
    using TS = TileShape<MSUB>;
    constexpr int ROWS = 16 * MSUB, G = 4, D = TS::D, NA = TS::NA;
    constexpr size_t ST_BYTES = (size_t)kTileWaves * 2 * ROWS * sizeof(Stat);
    __shared__ __align__(16) uint8_t ring[TS::LDS];

    // the wave index is uniform: in scalar registers, so are the panel and
    // every load offset derived from it
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n_groups = (P.n_panels + 3) >> 2;
    const int per_xcd = (n_groups + 7) >> 3;
    const int xcd = blockIdx.x & 7, k_local = blockIdx.x >> 3;
    const int group = xcd * per_xcd + k_local / P.n_tiles;
    const int tile = k_local % P.n_tiles;
    if (group >= n_groups) return;  // the whole block, before any barrier
    const int nkb = P.nkb;
    const int my_panel = group * 4 + wave;
    // a panel past the last one streams the last panel; its products are never used
    const uint8_t* wsrc = Wp + (size_t)min(my_panel, P.n_panels - 1) * nkb * (G * 1024) + lane * 16;
    const uint8_t* asrc = Hp + (size_t)tile * nkb * TS::STAGE + lane * 16;

    // the four W fragments of stage st (clamped to the last stage) into w
    auto load_w = [&](v4u (&w)[G], int st) {
        const uint8_t* s = wsrc + (size_t)min(st, nkb - 1) * (G * 1024);
#pragma unroll
        for (int g = 0; g < G; ++g) w[g] = *(const v4u*)(s + g * 1024);
    };
    // fragments wave, wave + 4, ... of stage st (clamped) into LDS ring stage `slot`
    auto load_a = [&](int st, int slot) {
        const uint8_t* s = asrc + (size_t)min(st, nkb - 1) * TS::STAGE;
        uint8_t* base = ring + slot * TS::STAGE;
#pragma unroll
        for (int j = 0; j < NA; ++j) {
            const int f = wave + kTileWaves * j;
            const bool real = f < MSUB;
            __builtin_amdgcn_global_load_lds((const DM_AS_GLOBAL void*)(s + (real ? f : wave) * 1024),
                                             (DM_AS_LDS void*)(real ? base + f * 1024 : ring + TS::SPARE), 16, 0,
                                             0);
        }
    };

    v4f acc[G][MSUB];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int m = 0; m < MSUB; ++m) acc[g][m] = v4f{0.f, 0.f, 0.f, 0.f};
    auto mma = [&](const v4u (&w)[G], const uint8_t* abase) {
        // masked-row fragments one ahead: the next one's LDS read is in
        // flight while the current one's products issue
        v4u a_next = *(const v4u*)abase;
#pragma unroll
        for (int m = 0; m < MSUB; ++m) {
            const v4u afr = a_next;
            if (m + 1 < MSUB) a_next = *(const v4u*)(abase + (m + 1) * 1024);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int g = 0; g < G; ++g) {
                if (BF16) {
                    acc[g][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(v8bf, afr), __builtin_bit_cast(v8bf, w[g]), acc[g][m], 0, 0, 0);
                } else {
                    const v4f a4 = __builtin_bit_cast(v4f, afr);
                    const v4f b4 = __builtin_bit_cast(v4f, w[g]);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc[g][m] = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[e], b4[e], acc[g][m], 0, 0, 0);
                }
            }
        }
    };

    if constexpr (TS::PAIRS) {
        // Pair q of stages (2q, 2q + 1) sits in register slot q % 2 and LDS
        // stages 2 (q % 2), + 1.  Each block waits for every load (only the
        // current pair's are in flight), meets the other waves (so the other
        // slot's LDS stages are free), issues the next pair and multiplies
        // the current one.  The wait opens the block, so the compiler sees it
        // on every path into the products and adds none of its own.
        v4u wr[2][2][G];
        auto load_pair = [&](int slot, int q) {
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                load_w(wr[slot][h2], 2 * q + h2);
                load_a(2 * q + h2, 2 * slot + h2);
            }
        };
        const int npairs = (nkb + 1) / 2;
        load_pair(0, 0);
        for (int pr = 0; pr < npairs; pr += 2) {
#pragma unroll
            for (int slot = 0; slot < 2; ++slot) {
                const int q = pr + slot;
                wait_vmcnt<0>();
                ring_barrier();
                load_pair(slot ^ 1, q + 1);
                if (2 * q < nkb) mma(wr[slot][0], ring + (2 * slot) * TS::STAGE + lane * 16);
                if (2 * q + 1 < nkb) mma(wr[slot][1], ring + (2 * slot + 1) * TS::STAGE + lane * 16);
            }
        }
    } else {
        // One uniform loop: trips of D stages, so the register ring's slots
        // are fixed.  Stage st issues the loads of stage st + D - 1 and
        // multiplies stage st; the loop starts D - 1 stages early (loads
        // only) and runs past the last stage (clamped loads, no products).
        // Without a separate prologue the compiler sees the same loads on
        // every path into the loop, so its own waits for the register ring
        // stay exact counts.
        v4u wr[D][G];
        const int n_trips = (nkb + 2 * D - 2) / D;
        for (int trip = 0; trip < n_trips; ++trip) {
#pragma unroll
            for (int k = 0; k < D; ++k) {
                const int st = trip * D + k - (D - 1);
                load_w(wr[(k + D - 1) % D], st + D - 1);
                load_a(st + D - 1, (st + D - 1) % D);
                if (st >= 0 && st < nkb) mma(wr[k], ring + (st % D) * TS::STAGE + lane * 16);
                wait_vmcnt<(D - 2) * (G + NA)>();
                ring_barrier();
            }
        }
    }
    wait_vmcnt<0>();
    __syncthreads();  // every load landed, every ring read done: the ring is free

    // ---------------- epilogue ----------------
    Stat* s_st = reinterpret_cast<Stat*>(ring);                     // [wave][2 * ROWS]
    RowMeta* s_meta = reinterpret_cast<RowMeta*>(ring + ST_BYTES);  // [ROWS]
    for (int r = threadIdx.x; r < ROWS; r += blockDim.x) s_meta[r] = meta[(size_t)tile * ROWS + r];
    __syncthreads();
    Stat* my_st = s_st + (size_t)wave * 2 * ROWS;
    {
        const int grp = lane >> 4, c16 = lane & 15;
        const int col0 = my_panel * 64 + c16;
        bool ok[G];
#pragma unroll
        for (int g = 0; g < G; ++g) ok[g] = my_panel < P.n_panels && col0 + 16 * g < P.V;
        // One epilogue for every real panel, free of per-column tests (a second,
        // tested copy would cost this one its registers).  The one panel the
        // vocabulary cuts (`cut`, a uniform branch no other wave takes) sets
        // its columns past the vocabulary to -inf, which the statistics and
        // the centroid sums ignore, and stores none of them.
        if (my_panel < P.n_panels) {
            constexpr bool FULL = true;
            const bool cut = (my_panel + 1) * 64 > P.V;
            // 16-byte stores of whole quads: rows 16-byte aligned (V % 4 == 0,
            // so a quad's four columns are all inside or all past the vocabulary)
            const bool vstore = (P.V & 3) == 0 && (reinterpret_cast<uintptr_t>(logits) & 15) == 0;
#pragma unroll
            for (int m = 0; m < MSUB; ++m) {
                // the lane group's four rows of sub-tile m: metadata read together,
                // statistics reduced together
                RowMeta mt[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) mt[j] = s_meta[16 * m + 4 * grp + j];
                float x[4][G];
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int g = 0; g < G; ++g) x[j][g] = acc[g][m][j] * mt[j].scale;
                if (cut) {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
#pragma unroll
                        for (int g = 0; g < G; ++g) x[j][g] = ok[g] ? x[j][g] : -INFINITY;
                }
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int g = 0; g < G; ++g) acc[g][m][j] = x[j][g];
                if (vstore) {
                    // rows kept for the vocabulary pass, 16 bytes per lane: after a
                    // transpose inside each quad of lanes, lane 16 grp + 4 q + k holds
                    // columns 16 g + 4 q .. + 3 of row 4 grp + k of the sub-tile
                    const int k = c16 & 3;
                    const RowMeta me = s_meta[16 * m + 4 * grp + k];
#pragma unroll
                    for (int g = 0; g < G; ++g) {
                        float t[4] = {x[0][g], x[1][g], x[2][g], x[3][g]};
                        quad_transpose(t, k);
                        if (me.canon >= 0 && me.store && (!cut || my_panel * 64 + 16 * g + 4 * (c16 >> 2) < P.V))
                            *(v4f*)(logits + (size_t)me.canon * P.V + my_panel * 64 + 16 * g + 4 * (c16 >> 2)) =
                                v4f{t[0], t[1], t[2], t[3]};
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (mt[j].canon >= 0 && mt[j].store) {  // the whole 16-lane row agrees
#pragma unroll
                            for (int g = 0; g < G; ++g)
                                if (!cut || ok[g]) logits[(size_t)mt[j].canon * P.V + col0 + 16 * g] = x[j][g];
                        }
                }
                Stat st[4];
                row16_stats<4, G, FULL>(x, ok, col0, st);
                if (c16 == 0) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) my_st[16 * m + 4 * grp + j] = mt[j].canon >= 0 ? st[j] : stat_empty();
                }
            }
            if (tile < P.tiles_lossy) {
#define DM_ACC(lam, g) acc[g][(lam) >> 2][(lam) & 3]
                // a ragged batch's weight sits in the metadata of the position's first head row
#define DM_INVW(p) (P.ragged ? s_meta[16 * (((p) * P.K) >> 2) + 4 * grp + (((p) * P.K) & 3)].inv_k : P.inv_k)
                DM_CENTROIDS(4 * MSUB, DM_ACC, DM_INVW, c16 == 0, &my_st[ROWS + grp * P.ppg]);
#undef DM_INVW
#undef DM_ACC
            }
        } else {
            // a panel past the last one: no columns, empty statistics for the merge
            for (int t = lane; t < 2 * ROWS; t += 64) my_st[t] = stat_empty();
        }
    }
    __syncthreads();
    // merge the four panels in panel order: part[target][panel group]
    const int npt = P.GR * P.ppg;
    const int nloc = ROWS + (tile < P.tiles_lossy ? npt : 0);
    for (int t = threadIdx.x; t < nloc; t += blockDim.x) {
        const Stat* col = s_st + t;
        Stat st = col[0];
#pragma unroll
        for (int c = 1; c < kTileWaves; ++c) st = stat_merge(st, col[(size_t)c * 2 * ROWS]);
        int target = tile * ROWS + t;
        if (t >= ROWS) {
            const int p = tile * npt + (t - ROWS);
            if (p >= P.n_lossy_pos) continue;
            target = P.R_phys + p;
        }
        part[(size_t)target * P.n_vgroups + group] = st;
    }
}

// =====================================================================
// k_gemm_skinny: L[rho, v] = scale(rho) * sum_j W[v, j] * Hm[rho, j]
// (DropMatch Eq. (3) with the shared head W), for one tile of ROWS = 16*MSUB
// rows per workgroup and a contiguous range of 16-row vocabulary strips.
//
// Main loop: each wave streams NS strips of W straight from HBM into MFMA
// B operands (v_mfma_f32_16x16x32_bf16; fp32 inputs use 16x16x4), one
// 128-byte slice of every row per iteration, prefetching the next slice.
// The Hm tile (the A operand, shared by all waves) is staged through LDS in
// 512-byte-per-row chunks, double buffered.  Any permutation of the
// reduction index applied to both operands leaves the sums unchanged, so
// each lane loads 16 contiguous bytes of a row for both A and B.
//
// Epilogue: the accumulators pass through LDS; the wave stores the rows
// that later passes need (coalesced along the vocabulary), and computes,
// over its columns, (max, sum exp, argmax) per row and per centroid (the
// mean of a position's K head rows, DropMatch Eq. (5)).  The waves'
// statistics are merged in a fixed order into one partial per workgroup.
// =====================================================================
constexpr int kChunkBytes = 512;
constexpr int kIterBytes = 128;
constexpr int kIPC = kChunkBytes / kIterBytes;
constexpr int kLdsRow = kChunkBytes + 16;
constexpr int kSkinnyNS = 4;
constexpr int kSkinnyWaves = 8;

template <int MSUB, int NS, int WAVES>
struct SkinnyLds {
    static constexpr int ROWS = 16 * MSUB;
    static constexpr int COLS = 16 * NS;
    static constexpr int PITCH = COLS + 1;
    static constexpr int STAGE = 2 * ROWS * kLdsRow;
    static constexpr int EPI = WAVES * ROWS * PITCH * 4;
    static constexpr int MAIN = STAGE > EPI ? STAGE : EPI;
    static constexpr int NSTAT = ROWS + 4 * 16;  // rows + centroid slots
    static constexpr int STATS = WAVES * NSTAT * (int)sizeof(Stat);
};

template <bool BF16, int MSUB, int NS, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void k_gemm_skinny(const Plan P, const uint8_t* __restrict__ W,
                                                            const uint8_t* __restrict__ Hm,
                                                            float* __restrict__ logits, Stat* __restrict__ part) {
    typedef SkinnyLds<MSUB, NS, WAVES> L;
    constexpr int ROWS = L::ROWS, COLS = L::COLS, PITCH = L::PITCH;
    __shared__ __align__(16) uint8_t smem[L::MAIN];
    __shared__ Stat sstat[WAVES][L::NSTAT];
    __shared__ float s_scale[ROWS];
    __shared__ int s_canon[ROWS];
    __shared__ int s_store[ROWS];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int tile = blockIdx.y, vg = blockIdx.x;
    const int nstr = (P.V + 15) >> 4;
    const int s_lo = (int)((long long)vg * nstr / P.n_vgroups);
    const int s_hi = (int)((long long)(vg + 1) * nstr / P.n_vgroups);
    const int ws0 = s_lo + wave * NS;
    const size_t row_bytes = (size_t)P.d * (BF16 ? 2 : 4);
    const int n_iter = (int)(row_bytes / kIterBytes);
    const int n_chunks = (n_iter + kIPC - 1) / kIPC;

    if (threadIdx.x < ROWS) {
        RowInfo ri = row_info(P, tile * ROWS + threadIdx.x);
        bool valid = ri.b >= 0;
        s_scale[threadIdx.x] = valid ? (ri.lossy ? seq_scale(P, ri.b) : P.scale_undropped) : 0.0f;
        s_canon[threadIdx.x] = valid ? (ri.b * P.T1 + ri.t) * P.K + ri.i : -1;
        s_store[threadIdx.x] =
            valid && (P.store_all || !ri.lossy || (bit_of(P.js_bits, ri.b) && ri.t < seq_G(P, ri.b)));
    }

    const uint8_t* wp[NS];
    bool sact[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int strip = ws0 + s;
        sact[s] = strip < s_hi;
        int v = strip * 16 + (lane & 15);
        v = v < P.V ? v : P.V - 1;
        wp[s] = W + (size_t)v * row_bytes + (lane >> 4) * 16;
    }
    const uint8_t* Ab = Hm + (size_t)tile * ROWS * row_bytes;

    constexpr int UNITS = ROWS * (kChunkBytes / 16);
    constexpr int UPT = (UNITS + WAVES * 64 - 1) / (WAVES * 64);
    v4u areg[UPT];
    auto load_a = [&](int c) {
#pragma unroll
        for (int u = 0; u < UPT; ++u) {
            const int idx = threadIdx.x + u * WAVES * 64;
            const int r = idx >> 5, col = (idx & 31) * 16;
            const size_t off = (size_t)c * kChunkBytes + col;
            areg[u] = (idx < UNITS && off < row_bytes) ? *(const v4u*)(Ab + (size_t)r * row_bytes + off)
                                                        : v4u{0, 0, 0, 0};
        }
    };
    auto store_a = [&](int buf) {
#pragma unroll
        for (int u = 0; u < UPT; ++u) {
            const int idx = threadIdx.x + u * WAVES * 64;
            if (idx < UNITS) {
                const int r = idx >> 5, col = (idx & 31) * 16;
                *(v4u*)(smem + buf * ROWS * kLdsRow + r * kLdsRow + col) = areg[u];
            }
        }
    };

    v4f acc[NS][MSUB];
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int m = 0; m < MSUB; ++m) acc[s][m] = v4f{0.f, 0.f, 0.f, 0.f};

    load_a(0);
    store_a(0);
    __syncthreads();

    v4u wc[NS][2], wn[NS][2];
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int f = 0; f < 2; ++f) wc[s][f] = sact[s] ? *(const v4u*)(wp[s] + f * 64) : v4u{0, 0, 0, 0};

    for (int c = 0; c < n_chunks; ++c) {
        const int it0 = c * kIPC;
        const int nit = n_iter - it0 < kIPC ? n_iter - it0 : kIPC;
        if (c + 1 < n_chunks) load_a(c + 1);
        const uint8_t* abuf = smem + (c & 1) * ROWS * kLdsRow;
        for (int ii = 0; ii < nit; ++ii) {
            const int it = it0 + ii;
            if (it + 1 < n_iter) {
#pragma unroll
                for (int s = 0; s < NS; ++s)
#pragma unroll
                    for (int f = 0; f < 2; ++f)
                        if (sact[s]) wn[s][f] = *(const v4u*)(wp[s] + (size_t)(it + 1) * kIterBytes + f * 64);
            }
            v4u afr[MSUB][2];
#pragma unroll
            for (int m = 0; m < MSUB; ++m)
#pragma unroll
                for (int f = 0; f < 2; ++f)
                    afr[m][f] = *(const v4u*)(abuf + (16 * m + (lane & 15)) * kLdsRow + ii * kIterBytes + f * 64 +
                                              (lane >> 4) * 16);
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                if (!sact[s]) continue;
#pragma unroll
                for (int f = 0; f < 2; ++f)
#pragma unroll
                    for (int m = 0; m < MSUB; ++m) {
                        if (BF16) {
                            acc[s][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                __builtin_bit_cast(v8bf, afr[m][f]), __builtin_bit_cast(v8bf, wc[s][f]), acc[s][m],
                                0, 0, 0);
                        } else {
                            v4f a = __builtin_bit_cast(v4f, afr[m][f]);
                            v4f b = __builtin_bit_cast(v4f, wc[s][f]);
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                acc[s][m] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], acc[s][m], 0, 0, 0);
                        }
                    }
            }
#pragma unroll
            for (int s = 0; s < NS; ++s)
#pragma unroll
                for (int f = 0; f < 2; ++f) wc[s][f] = wn[s][f];
        }
        if (c + 1 < n_chunks) store_a((c + 1) & 1);
        __syncthreads();
    }

    // ---------------- epilogue ----------------
    float* et = (float*)smem + wave * ROWS * PITCH;
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int m = 0; m < MSUB; ++m)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * m + 4 * (lane >> 4) + j;
                et[r * PITCH + s * 16 + (lane & 15)] = acc[s][m][j] * s_scale[r];
            }
    __syncthreads();

    const int vbase = ws0 * 16;
    // stores of the rows the later passes read, one coalesced row at a time
    {
        const int cs = lane >> 4;
        const int v = vbase + lane;
        const bool ok = (lane < COLS) && (ws0 + cs < s_hi) && v < P.V;
        if (ok) {
            for (int r = 0; r < ROWS; ++r)
                if (s_store[r]) logits[(size_t)s_canon[r] * P.V + v] = et[r * PITCH + lane];
        }
    }
    int ncol = (s_hi - ws0) * 16;
    ncol = ncol < COLS ? ncol : COLS;
    if (vbase + ncol > P.V) ncol = P.V - vbase;
    if (ncol < 0) ncol = 0;
    // per-row statistics over this wave's columns: lane = row
    if (lane < ROWS) {
        Stat st = stat_empty();
        for (int c = 0; c < ncol; ++c) stat_push(st, et[lane * PITCH + c], vbase + c);
        sstat[wave][lane] = st;
    }
    // per-centroid statistics: lane = lossy position slot of this tile
    const int npt = P.GR * P.ppg;
    const bool lossy_tile = tile < P.tiles_lossy;
    if (lossy_tile && lane < npt) {
        const int g = lane / P.ppg, slot = lane - g * P.ppg;
        const int p = tile * npt + lane;
        Stat st = stat_empty();
        if (p < P.n_lossy_pos) {
            const float inv_k = lossy_pos_inv_k(P, p);
            for (int c = 0; c < ncol; ++c) {
                float lb = centroid_logit(P.K, inv_k,
                                          [&](int i) { return et[tile_row(0, g, slot * P.K + i) * PITCH + c]; });
                stat_push(st, lb, vbase + c);
            }
        }
        sstat[wave][ROWS + lane] = st;
    }
    __syncthreads();
    const int nloc = ROWS + (lossy_tile ? npt : 0);
    for (int t = threadIdx.x; t < nloc; t += blockDim.x) {
        Stat st = stat_empty();
#pragma unroll
        for (int w = 0; w < WAVES; ++w) st = stat_merge(st, sstat[w][t]);
        int target;
        if (t < ROWS) {
            target = tile * ROWS + t;
        } else {
            const int p = tile * npt + (t - ROWS);
            if (p >= P.n_lossy_pos) continue;
            target = P.R_phys + p;
        }
        part[(size_t)target * P.n_vgroups + vg] = st;
    }
}

// =====================================================================
// k_combine: final (max, log Z, argmax) per head row and per centroid.
// One block per target: threads merge the per-vocabulary-group partials
// (four loads in flight each), then a butterfly per wave and a fixed-order
// merge of the waves, so repeated runs give identical bits.  Block 0 also
// zeroes the call's residual-race slots, which k_vocab fills next: every
// call starts from empty slots whatever an earlier call left there.
// =====================================================================
constexpr int kCombineThreads = 256;
constexpr float kLn2Combine = 0.69314718055994531f;

__global__ __launch_bounds__(kCombineThreads) void k_combine(const Plan P, const Stat* __restrict__ part,
                                                             RowStat* __restrict__ rowstat,
                                                             RowStat* __restrict__ centstat,
                                                             unsigned long long* __restrict__ race_best,
                                                             int32_t* __restrict__ dbg_head_arg,
                                                             float* __restrict__ dbg_head_logz,
                                                             int32_t* __restrict__ dbg_cent_arg,
                                                             float* __restrict__ dbg_cent_logz) {
    __shared__ Stat s_w[kCombineThreads / 64];
    const int t = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (t == 0)
        for (int i = threadIdx.x; i < P.B; i += kCombineThreads) {
            race_best[kRaceSlotStride * i] = 0ull;
            race_best[kRaceSlotStride * i + 1] = 0ull;
        }
    int b, pos_t, head = 0;
    const bool is_row = t < P.R_phys;
    bool lossless = false;
    if (is_row) {
        const RowInfo ri = row_info(P, t);
        if (ri.b < 0) return;  // padding row: the whole block leaves
        b = ri.b;
        pos_t = ri.t;
        head = ri.i;
        lossless = !ri.lossy;
    } else {
        class_pos(P, 0, t - P.R_phys, &b, &pos_t);
    }
    const Stat* src = part + (size_t)t * P.n_vgroups;
    Stat st = stat_empty();
    for (int vg = threadIdx.x; vg < P.n_vgroups; vg += 4 * kCombineThreads) {
        Stat x[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int k = vg + u * kCombineThreads;
            x[u] = k < P.n_vgroups ? src[k] : stat_empty();
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) st = stat_merge(st, x[u]);
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) st = stat_merge(st, stat_shfl_xor(st, off));
    if (lane == 0) s_w[wave] = st;
    __syncthreads();
    if (threadIdx.x != 0) return;
    st = s_w[0];
#pragma unroll
    for (int w = 1; w < kCombineThreads / 64; ++w) st = stat_merge(st, s_w[w]);
    const float logz = st.m + __logf(st.s);
    const RowStat rs{st.m, logz, st.idx, logz - kLn2Combine};
    const int pidx = b * P.T1 + pos_t;
    if (is_row) {
        const int canon = pidx * P.K + head;
        rowstat[canon] = rs;
        if (dbg_head_arg) dbg_head_arg[canon] = rs.idx;
        if (dbg_head_logz) dbg_head_logz[canon] = rs.logz;
    }
    if (!is_row || lossless) {
        centstat[pidx] = rs;
        if (dbg_cent_arg) dbg_cent_arg[pidx] = rs.idx;
        if (dbg_cent_logz) dbg_cent_logz[pidx] = rs.logz;
    }
}

// =====================================================================
// k_vocab: the vocabulary pass.
//
// Blocks [0, blk_js): one JS position x one vocabulary chunk.  Partial sums
//   over the chunk of JS(p^(i) || p-bar) for every head i and of
//   JS(q_hat || p-bar) (DropMatch Eq. (6): natural-log Jensen-Shannon
//   divergence, M = (P + Q) / 2, 0 ln 0 = 0).
// Blocks [blk_js, blk_js + blk_race): one lossless sequence x one chunk.
//   Each block first repeats the sequence's min(1, p/q) tests to find the
//   first rejection A, then runs the exponential race over its chunk for
//   the emitted token (the residual (p_A - q_A)+ after a rejection, p_gamma
//   when every draft passed; "Why speculative decoding preserves
//   distributions...", Sec. 2 and the verify round of Sec. 5).  Chunk
//   winners meet in a 64-bit atomic max per sequence.
// =====================================================================
constexpr int kVocabThreads = 256;
constexpr int kVocabWaves = kVocabThreads / 64;
constexpr int kJsPerThread = 8;  // the JS chunk is kVocabThreads * kJsPerThread entries
constexpr float kLn2 = 0.69314718055994531f;
// steps of 4 entries per thread that cover one race block's chunk
constexpr int kRaceSteps = kRaceChunkMax / (4 * kVocabThreads);
static_assert(kRaceSteps * 4 * kVocabThreads == kRaceChunkMax, "race chunk: whole steps");

// e^x and ln x on the hardware base-2 units (v_exp_f32, v_log_f32), for
// arguments whose results stay in the normal fp32 range.
__device__ __forceinline__ float hw_exp(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }
__device__ __forceinline__ float hw_log(float x) { return __builtin_amdgcn_logf(x) * kLn2; }

// Smallest mixture the JS terms evaluate ln of; an entry whose two
// probabilities sum to less contributes below 1e-36 and is left at that.
constexpr float kMixFloor = 1e-37f;

// Adds twice one vocabulary entry's share of JS(P || Q) to acc.  With
// a = ln P, b = ln Q and ln M = ln(P + Q) - ln 2 = ln 2 (L - 1), L =
// log2(P + Q), the share is (P (a - ln M) + Q (b - ln M)) / 2.  The caller
// passes the shifted logs a1 = a + ln 2 and b1 = b + ln 2, so that
// a - ln M = a1 - ln 2 L (one fused multiply-add); the factor 1/2 is
// applied once to the chunk sum.  A zero probability contributes nothing as
// long as its log argument is finite.  Branch-free.
__device__ __forceinline__ float js_acc2(float acc, float a1, float Pa, float b1, float Pb) {
    const float L = __builtin_amdgcn_logf(fmaxf(Pa + Pb, kMixFloor));
    return fmaf(Pb, fmaf(-kLn2, L, b1), fmaf(Pa, fmaf(-kLn2, L, a1), acc));
}

// P = e^a from the shifted log a1 = a + ln 2: 2^(a1 log2 e - 1).
__device__ __forceinline__ float exp_shifted(float a1) { return __builtin_amdgcn_exp2f(fmaf(a1, kLog2e, -1.0f)); }

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

__device__ __forceinline__ unsigned long long race_pack(float key, int v) {
    return ((unsigned long long)__float_as_uint(key) << 32) | (unsigned long long)(0xffffffffu - (uint32_t)v);
}

__device__ __forceinline__ unsigned long long u64_max(unsigned long long a, unsigned long long b) {
    return a > b ? a : b;
}

// Lossless decision at drafted position t: u_t * q(x) < p(x) with p the
// undropped target distribution and u_t from Philox stream 1.
__device__ __forceinline__ bool lossless_accept(const Plan& P, int b, int t, const int32_t* draft,
                                                const float* q_hat, const float* logits,
                                                const RowStat* rowstat, const FiltStat* filt) {
    const int32_t x = draft[b * P.G + t];
    if (!(x >= 0 && x < P.V)) return false;
    const int pidx = b * P.T1 + t;
    const float lx = logits[(size_t)pidx * P.K * P.V + x];
    float px;
    if (P.filter) {
        // the processed target: 0 off the kept set, renormalised on it
        const FiltStat f = filt[pidx];
        px = lx >= f.thresh ? __expf(lx - f.logz) : 0.0f;
    } else {
        px = __expf(lx - rowstat[pidx * P.K].logz);
    }
    const float qx = q_hat[(size_t)(b * P.G + t) * P.V + x];
    const u32x4 r = philox10(u32x4{0u, (uint32_t)pidx, 0u, kStreamAccept}, P.key0, P.key1);
    const float u = (float)(r.x >> 8) * 5.9604644775390625e-08f;  // 2^-24
    return u * qx < px;
}

// First rejection of a sequence from a wave's per-lane reject flags.
__device__ __forceinline__ int first_reject(bool reject, int G) {
    const unsigned long long rej = __ballot(reject);
    return rej ? __ffsll((long long)rej) - 1 : G;
}

// The round on a token tree ("Speculative Decoding: Draft, Then Verify",
// "Variants"; DropMatch Sec. 4.4), one wave, lane t = draft t = node t+1:
// `pass` is the rule's decision for the draft at its parent, `up` the
// parent position (valid iff 0 <= up <= t).  A node is on a kept path iff
// it and every node above it passed; the deepest such node wins, the
// smallest index on equal depths.  Pointer jumping: each lane folds in the
// pass flag and length of the segment above it, doubling the segment every
// step, so six steps cover any path of up to 64 nodes.  Returns the depth
// and writes the winner's position (0 = the root) to *pos.
__device__ __forceinline__ int tree_walk(bool live, bool pass, int up, int lane, int* pos) {
    const bool up_ok = live && up >= 0 && up <= lane;
    int anc = up_ok ? up - 1 : -1;  // draft index of the parent node, -1 = the root
    int ok = (up_ok && pass) ? 1 : 0;
    int depth = 1;
#pragma unroll
    for (int step = 0; step < 6; ++step) {
        const int src = anc < 0 ? lane : anc;
        const int ok_a = __shfl(ok, src, 64);
        const int depth_a = __shfl(depth, src, 64);
        const int anc_a = __shfl(anc, src, 64);
        if (anc >= 0) {
            ok &= ok_a;
            depth += depth_a;
            anc = anc_a;
        }
    }
    // deepest first, then the smallest lane: one max over (depth, 63 - lane)
    int key = ok ? (depth << 6) | (63 - lane) : 0;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) key = max(key, __shfl_xor(key, off, 64));
    *pos = key ? 64 - (key & 63) : 0;
    return key >> 6;
}

// JS partial sums of one (position, chunk): kJsPerThread entries per
// thread, every load issued before any arithmetic, all non-temporal (each
// logit and q_hat entry is read once per call).  Rows 16-byte aligned:
// thread x takes float4s at 4x and 4x + 1024 of the chunk, so each wave's
// load covers 1 KiB contiguous; otherwise entries x, x + 256, ....  KMAX
// bounds K so the registers stay small.
template <int KMAX, bool VEC4>
__device__ __forceinline__ void js_block(const Plan& P, int blk, const float* __restrict__ q_hat,
                                         const float* __restrict__ logits, const RowStat* __restrict__ rowstat,
                                         const RowStat* __restrict__ centstat, float* __restrict__ jspart,
                                         float (*s_red)[kMaxK + 1]) {
    constexpr int E = kJsPerThread;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int K = P.K, G = P.G, T1 = P.T1, V = P.V;
    const int jp = blk / P.js_chunks, c = blk - jp * P.js_chunks;
    const int js_rank = jp / G, t = jp - js_rank * G;
    const int b = select_of(P.js_bits, P.B, js_rank, true);
    if (t >= seq_G(P, b)) return;  // past a ragged sequence's drafts: the whole block leaves
    const int Kb = seq_K(P, b);    // heads of this sequence (K is the layout stride)
    const float inv_k = seq_inv_k(P, b);
    const int pidx = b * T1 + t;
    const float* lrow = logits + (size_t)pidx * K * V;
    const float* qrow = q_hat + (size_t)(b * G + t) * V;
    const int v0 = c * P.js_chunk;

    // Loads past the end of the vocabulary read a valid entry instead, so no
    // lane branches; such an entry takes live = 0, which zeroes every
    // probability it contributes (the values it read stay finite).
    float l[E][KMAX], q[E];
    bool live[E];
    if constexpr (VEC4) {
#pragma unroll
        for (int u = 0; u < E; u += 4) {
            const int vu = v0 + u * kVocabThreads + 4 * threadIdx.x;  // a wave reads 1 KiB contiguous
            const bool ok = vu < V;  // V % 4 == 0: a float4 is wholly in or out
            const int vv = ok ? vu : V - 4;
#pragma unroll
            for (int i = 0; i < KMAX; ++i) {
                v4f x = v4f{0.f, 0.f, 0.f, 0.f};
                if (i < Kb) x = __builtin_nontemporal_load((const v4f*)(lrow + (size_t)i * V + vv));  // Kb is uniform
#pragma unroll
                for (int e = 0; e < 4; ++e) l[u + e][i] = x[e];
            }
            const v4f y = __builtin_nontemporal_load((const v4f*)(qrow + vv));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                q[u + e] = y[e];
                live[u + e] = ok;
            }
        }
    } else {
#pragma unroll
        for (int u = 0; u < E; ++u) {
            const int vu = v0 + u * kVocabThreads + threadIdx.x;
            const bool ok = vu < V;
            const int vv = ok ? vu : V - 1;
#pragma unroll
            for (int i = 0; i < KMAX; ++i) {
                float x = 0.0f;
                if (i < Kb) x = __builtin_nontemporal_load(lrow + (size_t)i * V + vv);
                l[u][i] = x;
            }
            q[u] = __builtin_nontemporal_load(qrow + vv);
            live[u] = ok;
        }
    }
    float logz[KMAX];
#pragma unroll
    for (int i = 0; i < KMAX; ++i) logz[i] = i < Kb ? rowstat[pidx * K + i].logz1 : 0.0f;  // log Z - ln 2
    const float logz_c = centstat[pidx].logz1;

    float acc[KMAX + 1];
#pragma unroll
    for (int i = 0; i <= KMAX; ++i) acc[i] = 0.0f;
#pragma unroll
    for (int u = 0; u < E; ++u) {
        const float lv = live[u] ? 1.0f : 0.0f;  // 0 past the end of the vocabulary
        // the centroid logit, same operations in the same order as the
        // LM-head epilogue's
        float lsum = l[u][0];
#pragma unroll
        for (int i = 1; i < KMAX; ++i)
            if (i < Kb) lsum += l[u][i];
        const float bb = lsum * inv_k - logz_c;  // ln p-bar + ln 2
        const float pb = exp_shifted(bb) * lv;
#pragma unroll
        for (int i = 0; i < KMAX; ++i)
            if (i < Kb) {
                const float a = l[u][i] - logz[i];  // ln p + ln 2
                acc[i] = js_acc2(acc[i], a, exp_shifted(a) * lv, bb, pb);
            }
        const float qq = live[u] ? fmaxf(q[u], 0.0f) : 0.0f;
        acc[KMAX] = js_acc2(acc[KMAX], fmaf(__builtin_amdgcn_logf(fmaxf(qq, kMixFloor)), kLn2, kLn2), qq, bb, pb);
    }
#pragma unroll
    for (int i = 0; i <= KMAX; ++i)
        if (i < Kb || i == KMAX) {
            const float x = wave_sum(acc[i]);
            if (lane == 0) s_red[wave][i == KMAX ? kMaxK : i] = x;
        }
    __syncthreads();
    if ((int)threadIdx.x < Kb || (int)threadIdx.x == K) {  // heads, then the draft in slot K
        const int i = threadIdx.x == K ? kMaxK : threadIdx.x;
        float x = 0.0f;
#pragma unroll
        for (int w = 0; w < kVocabWaves; ++w) x += s_red[w][i];
        jspart[((size_t)jp * (K + 1) + threadIdx.x) * P.js_chunks + c] = 0.5f * x;
    }
}

// KMAX bounds the heads the JS blocks hold in registers; the launch picks
// the smallest of 5, 8 and kMaxK that covers K, so a kernel's register
// budget (and with it how many waves a CU keeps in flight) follows K.
// VEC4: the rows are read as float4 (16-byte aligned, V % 4 == 0).  The
// scalar path is an instance of its own because a kernel's register count
// is the largest over its code: in one instance with the float4 path it
// held K <= 5 at 66 VGPRs (7 waves per SIMD) instead of 62 (8 waves).
template <int KMAX, bool VEC4>
__global__ __launch_bounds__(kVocabThreads) void k_vocab(
    const Plan P, const int32_t* __restrict__ draft, const float* __restrict__ q_hat,
    const float* __restrict__ logits, const RowStat* __restrict__ rowstat, const RowStat* __restrict__ centstat,
    float* __restrict__ jspart, unsigned long long* __restrict__ race_best, const FiltStat* __restrict__ filt) {
    __shared__ float s_red[kVocabWaves][kMaxK + 1];
    __shared__ int s_A;
    __shared__ unsigned long long s_best[2][kVocabWaves];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int K = P.K, G = P.G, T1 = P.T1, V = P.V;
    int blk = blockIdx.x;
    (void)wave;

    if (blk < P.blk_js) {
        js_block<KMAX, VEC4>(P, blk, q_hat, logits, rowstat, centstat, jspart, s_red);
        return;
    }
    blk -= P.blk_js;

    const int r = blk / P.race_chunks, c = blk - r * P.race_chunks;
    const int b = select_of(P.lossless_bits, P.B, r, true);
    const int Gb = seq_G(P, b);
    if (wave == 0) {
        const bool reject = lane < Gb && !lossless_accept(P, b, lane, draft, q_hat, logits, rowstat, filt);
        const int A = first_reject(reject, Gb);
        if (lane == 0) s_A = A;
    }
    __syncthreads();
    const int A = s_A;
    const int pidx = b * T1 + A;
    float logz = rowstat[pidx * K].logz, thresh = -INFINITY;
    if (P.filter) {
        const FiltStat f = filt[pidx];
        logz = f.logz;
        thresh = f.thresh;
    }
    const float* lrow = logits + (size_t)pidx * K * V;
    const float* qrow = A < Gb ? q_hat + (size_t)(b * G + A) * V : nullptr;
    unsigned long long best_r = 0ull, best_p = 0ull;
    const int v0 = c * P.race_chunk;
    const int v1 = min(v0 + P.race_chunk, V);  // race_chunk <= kRaceChunkMax, a multiple of 1024
    // every load of the chunk first (non-temporal: read once per call); an
    // entry past the chunk reads a valid one and is skipped below
    float lv[kRaceSteps][4], qv[kRaceSteps][4];
#pragma unroll
    for (int it = 0; it < kRaceSteps; ++it) {
        const int vq = v0 + 4 * threadIdx.x + it * 4 * kVocabThreads;
        if constexpr (VEC4) {  // V % 4 == 0, so v1 % 4 == 0: a float4 is wholly in or out
            const int vv = vq < v1 ? vq : V - 4;
            const v4f x = __builtin_nontemporal_load((const v4f*)(lrow + vv));
            const v4f y = qrow ? __builtin_nontemporal_load((const v4f*)(qrow + vv)) : v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                lv[it][k] = x[k];
                qv[it][k] = y[k];
            }
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int vv = vq + k < v1 ? vq + k : V - 1;
                lv[it][k] = __builtin_nontemporal_load(lrow + vv);
                qv[it][k] = qrow ? __builtin_nontemporal_load(qrow + vv) : 0.0f;
            }
        }
    }
#pragma unroll
    for (int it = 0; it < kRaceSteps; ++it) {
        const int vq = v0 + 4 * threadIdx.x + it * 4 * kVocabThreads;
        if (vq >= v1) break;  // later steps are past the chunk too
        const u32x4 rr = philox10(u32x4{(uint32_t)(vq >> 2), (uint32_t)pidx, 0u, kStreamRace}, P.key0, P.key1);
        const uint32_t words[4] = {rr.x, rr.y, rr.z, rr.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int v = vq + k;
            if (v >= v1) continue;
            const float p = lv[it][k] >= thresh ? __expf(lv[it][k] - logz) : 0.0f;
            const float w = qrow ? fmaxf(p - qv[it][k], 0.0f) : p;
            // U in (0, 1): top 23 bits plus one half, times 2^-23, a normal
            // number, so the hardware log2 needs no range reduction; the
            // keys take one reciprocal of E = -ln U
            const float U = ((float)(words[k] >> 9) + 0.5f) * 1.1920928955078125e-07f;
            const float inv_e = __builtin_amdgcn_rcpf(-kLn2 * __builtin_amdgcn_logf(U));
            if (w > 0.0f) best_r = u64_max(best_r, race_pack(w * inv_e, v));
            if (p > 0.0f) best_p = u64_max(best_p, race_pack(p * inv_e, v));
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        best_r = u64_max(best_r, __shfl_xor(best_r, off, 64));
        best_p = u64_max(best_p, __shfl_xor(best_p, off, 64));
    }
    // the waves' winners meet in LDS, so a block takes one atomic per slot
    if (lane == 0) {
        s_best[0][wave] = best_r;
        s_best[1][wave] = best_p;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
#pragma unroll
        for (int w = 1; w < kVocabWaves; ++w) {
            best_r = u64_max(best_r, s_best[0][w]);
            best_p = u64_max(best_p, s_best[1][w]);
        }
        if (best_r) atomicMax(&race_best[kRaceSlotStride * b], best_r);
        if (best_p) atomicMax(&race_best[kRaceSlotStride * b + 1], best_p);
    }
}

// =====================================================================
// k_finish: one block per sequence.  Applies the sequence's rule at every
// drafted position (lane t decides position t), finds the first rejection A
// ("Speculative Decoding: Draft, Then Verify", the draft-then-verify loop,
// steps 3 and 4) and emits one token: the centroid argmax at A for the
// DropMatch rules, the race winner for lossless sequences.
//
// The kernel is latency-bound, so it is built around few memory round trips:
// what the decisions read that does not depend on the JS sums (draft tokens,
// head and centroid argmaxes, race slots) is fetched first, while groups of
// four lanes reduce each (position, head-or-draft) JS sum over the
// vocabulary chunks, sixteen loads in flight per lane, in a fixed order.
// =====================================================================
constexpr int kFinishThreads = 256;
constexpr int kFinishLanesPerSum = 4;
constexpr int kFinishLoads = 16;  // JS chunk partials in flight per lane

__global__ __launch_bounds__(kFinishThreads) void k_finish(const Plan P, const int32_t* __restrict__ draft,
                                                           const float* __restrict__ q_hat,
                                                           const int32_t* __restrict__ tree_parent,
                                                           const float* __restrict__ logits,
                                                           const RowStat* __restrict__ rowstat,
                                                           const RowStat* __restrict__ centstat,
                                                           const float* __restrict__ jspart,
                                                           unsigned long long* __restrict__ race_best,
                                                           const FiltStat* __restrict__ filt,
                                                           int32_t* __restrict__ accept_len,
                                                           int32_t* __restrict__ out_token,
                                                           int32_t* __restrict__ accept_pos,
                                                           uint32_t* __restrict__ data_status,
                                                           uint8_t* __restrict__ dbg_flags,
                                                           float* __restrict__ dbg_js_heads,
                                                           float* __restrict__ dbg_js_draft) {
    __shared__ float s_js[kMaxGamma + 1][kMaxK + 1];
    const int b = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int K = P.K, G = P.G, T1 = P.T1;  // layout strides
    const int Gb = seq_G(P, b), Kb = seq_K(P, b);  // this sequence's drafts and heads
    const bool lossless = bit_of(P.lossless_bits, b);
    const bool js = bit_of(P.js_bits, b);
    const bool tree = bit_of(P.tree_bits, b);

    // wave 0, lane t: the inputs of the decision for draft t, made by the
    // heads at position t (a chain) or at the draft's parent (a tree)
    int x = -1, cent_idx = 0, up = -1;
    int head_idx[kMaxK];
#pragma unroll
    for (int i = 0; i < kMaxK; ++i) head_idx[i] = -1;
    unsigned long long best_r = 0ull, best_p = 0ull;
    if (wave == 0) {
        if (lane < Gb) x = draft[b * G + lane];
        if (tree && lane < Gb) up = tree_parent[b * G + lane];
        if (!lossless) {
            if (lane <= Gb) cent_idx = centstat[b * T1 + lane].idx;
            // a parent outside [0, t] rejects the draft; read position t instead
            const int at = (tree && up >= 0 && up <= lane) ? up : lane;
            if (lane < Gb) {
#pragma unroll
                for (int i = 0; i < kMaxK; ++i)
                    if (i < Kb) head_idx[i] = rowstat[(b * T1 + at) * K + i].idx;
            }
        } else if (lane == 0) {
            best_r = race_best[kRaceSlotStride * b];
            best_p = race_best[kRaceSlotStride * b + 1];
        }
    }

    if (js && G > 0) {
        // group g of four lanes sums (position, head-or-draft) pair base + g
        // over the chunks: lane s of the group takes chunks s, s + 4, ... in
        // order, then the four partial sums meet in a fixed butterfly
        const int jp0 = rank_of(P.js_bits, b, true) * G;
        const int n_idx = G * (K + 1);
        const int grp = threadIdx.x / kFinishLanesPerSum, sub = threadIdx.x % kFinishLanesPerSum;
        constexpr int kGroups = kFinishThreads / kFinishLanesPerSum;
        for (int base = 0; base < n_idx; base += kGroups) {
            const int idx = base + grp;
            const float* src = jspart + ((size_t)jp0 * (K + 1) + min(idx, n_idx - 1)) * P.js_chunks;
            float acc = 0.0f;
            for (int c0 = 0; c0 < P.js_chunks; c0 += kFinishLanesPerSum * kFinishLoads) {
                float v[kFinishLoads];
#pragma unroll
                for (int q = 0; q < kFinishLoads; ++q) {
                    const int cc = c0 + sub + kFinishLanesPerSum * q;
                    v[q] = (idx < n_idx && cc < P.js_chunks) ? src[cc] : 0.0f;
                }
#pragma unroll
                for (int q = 0; q < kFinishLoads; ++q) acc += v[q];
            }
            acc += __shfl_xor(acc, 1, 64);
            acc += __shfl_xor(acc, 2, 64);
            if (sub == 0 && idx < n_idx) s_js[idx / (K + 1)][idx % (K + 1)] = acc;
        }
    }
    __syncthreads();
    if (wave != 0) return;
    bool accept = false;
    if (lane < Gb) {
        if (lossless) {
            accept = lossless_accept(P, b, lane, draft, q_hat, logits, rowstat, filt);
        } else {
            int count = 0;
#pragma unroll
            for (int i = 0; i < kMaxK; ++i) count += (i < Kb && head_idx[i] == x) ? 1 : 0;
            const bool valid = x >= 0 && x < P.V;
            if (js) {
                float jmax = -INFINITY;
                for (int i = 0; i < Kb; ++i) jmax = fmaxf(jmax, s_js[lane][i]);
                const float jq = s_js[lane][K];
                accept = valid && (jq <= jmax || 2 * count > Kb);  // Algorithm 1: Eq. (6), else Eq. (7)
                if (dbg_js_draft) dbg_js_draft[b * G + lane] = jq;
                if (dbg_js_heads)
                    for (int i = 0; i < Kb; ++i) dbg_js_heads[(size_t)(b * G + lane) * K + i] = s_js[lane][i];
            } else {
                accept = valid && count > 0;  // DropMatch Eq. (4)
                if (tree && !(up >= 0 && up <= lane)) accept = false;
            }
        }
        if (dbg_flags) dbg_flags[b * G + lane] = accept ? 1 : 0;
    }
    // inputs the device found out of range (each such draft was rejected)
    const bool bad_draft = lane < Gb && !(x >= 0 && x < P.V);
    const bool bad_parent = tree && lane < Gb && !(up >= 0 && up <= lane);
    const unsigned long long any_bad_draft = __ballot(bad_draft), any_bad_parent = __ballot(bad_parent);
    int A, pos;
    if (tree) {
        A = tree_walk(lane < Gb, accept, up, lane, &pos);
    } else {
        A = first_reject(lane < Gb && !accept, Gb);
        pos = A;
    }
    const int token_lossy = __shfl(cent_idx, pos, 64);  // greedy on the centroid at the last kept node
    if (lane == 0) {
        accept_len[b] = A;
        if (accept_pos) accept_pos[b] = pos;
        if (data_status) data_status[b] = (any_bad_draft ? 1u : 0u) | (any_bad_parent ? 2u : 0u);
        if (lossless) {
            const unsigned long long best = best_r ? best_r : best_p;
            out_token[b] = best ? (int32_t)(0xffffffffu - (uint32_t)(best & 0xffffffffull)) : 0;
        } else {
            out_token[b] = token_lossy;
        }
    }
}

// =====================================================================
// k_filter: the processed target distribution of every lossless position.
// "Why speculative decoding preserves distributions but may not be faster",
// Sec. 1: p must already include top-k, top-p and the renormalisation;
// "Speculative Decoding: Draft, Then Verify", "The same sampling settings":
// the test and the residual use the processed p.  The pages name the filters
// without fixing ties; the readings: top-k keeps every token whose logit is
// >= the k-th largest, top-p keeps the tokens of that set whose strictly
// larger renormalised mass is below top_p.  Both are thresholds on the
// logit, found exactly by a radix search over the lexicographic order
// (distance bin, 32-bit key), which is the order of the logits:
//   F = floor((max - l) * 2048), clamped to 16 bits, is a monotone function
//   of the logit; level 0 bins its high byte (1/8 logit per bin), level 1
//   its low byte, levels 2-5 the bytes of the order-preserving key.
// The distance bins spread a row over many bins (few LDS atomic collisions)
// and shrink the candidate range fast: once the range holds at most
// kFilterCache tokens they are gathered into LDS and the remaining levels
// read only that copy.  When the top-k set itself fits, it is gathered
// whole and the top-p search never reads the row again.
// Histograms count tokens and add their masses e^(l - logZ) in 2^-60 fixed
// point, so every sum is exact and independent of the order of the atomics.
// One block per position writes the logit threshold, the log normaliser of
// the kept set and its size.
// =====================================================================
constexpr int kFilterThreads = 1024;
constexpr int kFilterHists = 4;     // histogram copies (wave % 4) to spread the atomics
constexpr int kFilterCache = 8192;  // candidate tokens held in LDS
constexpr int kFilterUnroll = 8;    // row loads in flight per thread

__device__ __forceinline__ uint32_t order_key(float f) {
    const uint32_t u = __float_as_uint(f + 0.0f);  // -0 -> +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}
__device__ __forceinline__ int dist_index(float l, float m) {
    return (int)fminf(fmaxf((m - l) * 2048.0f, 0.0f), 65535.0f);
}
__device__ __forceinline__ unsigned long long fixed_mass(float l, float logz) {
    return (unsigned long long)(__expf(l - logz) * 1.152921504606846976e18f);  // 2^60
}
__device__ __forceinline__ unsigned long long shfl_up_u64(unsigned long long x, int d) {
    const unsigned lo = __shfl_up((unsigned)x, d, 64), hi = __shfl_up((unsigned)(x >> 32), d, 64);
    return ((unsigned long long)hi << 32) | lo;
}
__device__ __forceinline__ unsigned long long shfl_u64(unsigned long long x, int src) {
    const unsigned lo = __shfl((unsigned)x, src, 64), hi = __shfl((unsigned)(x >> 32), src, 64);
    return ((unsigned long long)hi << 32) | lo;
}

struct FilterSel {
    int bin;
    unsigned cnt_above, cnt_bin;
    unsigned long long mass_above, mass_bin, total;
};

struct FilterLds {
    unsigned cnt[kFilterHists][256];
    unsigned long long mass[kFilterHists][256];
    uint32_t c_key[kFilterCache];
    unsigned long long c_mass[kFilterCache];
    int n_cache;
    FilterSel sel;
};

// The candidate range of a search: tokens with key >= lo and, from level 1
// on, distance bytes and key bytes equal to the ones chosen so far.
struct FilterRange {
    uint32_t lo;
    int level, hi_byte, lo_byte;
    uint32_t prefix;
    __device__ bool contains(int F, uint32_t key) const {
        if (key < lo) return false;
        if (level >= 1 && (F >> 8) != hi_byte) return false;
        if (level >= 2 && (F & 255) != lo_byte) return false;
        if (level >= 3 && (key >> (32 - 8 * (level - 2))) != prefix) return false;
        return true;
    }
    __device__ int bin(int F, uint32_t key) const {
        if (level == 0) return 255 - (F >> 8);
        if (level == 1) return 255 - (F & 255);
        return (int)((key >> (24 - 8 * (level - 2))) & 255u);
    }
};

// Wave 0: merges the histogram copies and picks the bin.  Count mode: the
// bin holding rank kk (1-based, from the top) of the range.  Mass mode: the
// lowest non-empty bin whose tokens above it (base + bins above) weigh less
// than the target; at the first level the target is top_p times the total.
__device__ void filter_select(FilterLds& L, bool mass_mode, unsigned kk, unsigned long long base,
                              unsigned long long target, double top_p, bool first) {
    const int lane = threadIdx.x & 63;
    unsigned c[4];
    unsigned long long m[4];
    unsigned tc = 0;
    unsigned long long tm = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int bin = 255 - 4 * lane - e;  // lane 0 holds the top bins
        c[e] = 0;
        m[e] = 0;
#pragma unroll
        for (int w = 0; w < kFilterHists; ++w) {
            c[e] += L.cnt[w][bin];
            m[e] += L.mass[w][bin];
        }
        tc += c[e];
        tm += m[e];
    }
    unsigned ic = tc;
    unsigned long long im = tm;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const unsigned oc = __shfl_up(ic, d, 64);
        const unsigned long long om = shfl_up_u64(im, d);
        if (lane >= d) {
            ic += oc;
            im += om;
        }
    }
    const unsigned long long total = shfl_u64(im, 63);
    if (mass_mode && first) target = (unsigned long long)(top_p * (double)total);
    unsigned ac = ic - tc;
    unsigned long long am = im - tm;
    int found = -1;
    unsigned f_ac = 0, f_c = 0;
    unsigned long long f_am = 0, f_m = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const bool hit = mass_mode ? (c[e] > 0 && base + am < target) : (ac < kk && kk <= ac + c[e]);
        if (hit) {  // mass mode keeps the last (lowest) qualifying bin of the lane
            found = 255 - 4 * lane - e;
            f_ac = ac;
            f_am = am;
            f_c = c[e];
            f_m = m[e];
        }
        ac += c[e];
        am += m[e];
    }
    const unsigned long long any = __ballot(found >= 0);
    const int src = any ? 63 - __clzll((long long)any) : 0;  // the lowest bins sit in the highest lane
    if (lane == src) L.sel = FilterSel{found, f_ac, f_c, f_am, f_m, total};
}

// Calls f(F, key, mass) for every token of the row in `range`, reading the
// row with kFilterUnroll loads in flight per thread (16-byte loads when the
// rows are 16-byte aligned: the pass is bound by the bytes in flight).
template <typename Fn>
__device__ __forceinline__ void for_row(const float* __restrict__ row, int V, bool vec4, float m, float logz,
                                        const FilterRange& range, Fn f) {
    if (vec4) {
        const v4f* row4 = reinterpret_cast<const v4f*>(row);
        const int V4 = V >> 2;
        for (int u0 = 0; u0 < V4; u0 += kFilterThreads * kFilterUnroll) {
            v4f x[kFilterUnroll];
#pragma unroll
            for (int j = 0; j < kFilterUnroll; ++j) {
                const int u = u0 + j * kFilterThreads + threadIdx.x;
                x[j] = u < V4 ? row4[u] : v4f{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int j = 0; j < kFilterUnroll; ++j) {
                const int u = u0 + j * kFilterThreads + threadIdx.x;
                if (u >= V4) continue;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t key = order_key(x[j][e]);
                    const int F = dist_index(x[j][e], m);
                    if (range.contains(F, key)) f(F, key, fixed_mass(x[j][e], logz));
                }
            }
        }
        return;
    }
    for (int v0 = 0; v0 < V; v0 += kFilterThreads * kFilterUnroll) {
        float l[kFilterUnroll];
#pragma unroll
        for (int j = 0; j < kFilterUnroll; ++j) {
            const int v = v0 + j * kFilterThreads + threadIdx.x;
            l[j] = v < V ? row[v] : -INFINITY;
        }
#pragma unroll
        for (int j = 0; j < kFilterUnroll; ++j) {
            const int v = v0 + j * kFilterThreads + threadIdx.x;
            if (v >= V) continue;
            const uint32_t key = order_key(l[j]);
            const int F = dist_index(l[j], m);
            if (range.contains(F, key)) f(F, key, fixed_mass(l[j], logz));
        }
    }
}

// Copies the row's tokens in `range` (at most kFilterCache) into the cache,
// with the same loads in flight as for_row; slots are claimed once per wave
// and value.
__device__ void filter_gather(FilterLds& L, const float* __restrict__ row, int V, bool vec4, float m, float logz,
                              const FilterRange& range) {
    const int lane = threadIdx.x & 63;
    if (threadIdx.x == 0) L.n_cache = 0;
    __syncthreads();
    auto put = [&](bool valid, float l) {
        const uint32_t key = order_key(l);
        const bool mem = valid && range.contains(dist_index(l, m), key);
        const unsigned long long bal = __ballot(mem);
        if (bal) {
            int slot0 = 0;
            if (lane == 0) slot0 = atomicAdd(&L.n_cache, __popcll(bal));
            slot0 = __shfl(slot0, 0, 64);
            if (mem) {
                const int slot = slot0 + __popcll(bal & ((1ull << lane) - 1ull));
                L.c_key[slot] = key;
                L.c_mass[slot] = fixed_mass(l, logz);
            }
        }
    };
    if (vec4) {
        const v4f* row4 = reinterpret_cast<const v4f*>(row);
        const int V4 = V >> 2;
        for (int u0 = 0; u0 < V4; u0 += kFilterThreads * kFilterUnroll) {
            v4f x[kFilterUnroll];
#pragma unroll
            for (int j = 0; j < kFilterUnroll; ++j) {
                const int u = u0 + j * kFilterThreads + threadIdx.x;
                x[j] = u < V4 ? row4[u] : v4f{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int j = 0; j < kFilterUnroll; ++j) {
                const bool valid = u0 + j * kFilterThreads + (int)threadIdx.x < V4;
#pragma unroll
                for (int e = 0; e < 4; ++e) put(valid, x[j][e]);
            }
        }
    } else {
        for (int v0 = 0; v0 < V; v0 += kFilterThreads * kFilterUnroll) {
            float x[kFilterUnroll];
#pragma unroll
            for (int j = 0; j < kFilterUnroll; ++j) {
                const int v = v0 + j * kFilterThreads + threadIdx.x;
                x[j] = v < V ? row[v] : 0.0f;
            }
#pragma unroll
            for (int j = 0; j < kFilterUnroll; ++j) put(v0 + j * kFilterThreads + (int)threadIdx.x < V, x[j]);
        }
    }
    __syncthreads();
}

// One radix search over the tokens with key >= lo.  `cached`: the cache
// already holds exactly those tokens.  Returns the final key and the count
// and fixed-point mass of the tokens at or above it.
__device__ void filter_search(FilterLds& L, const float* __restrict__ row, int V, bool vec4, float m, float logz,
                              uint32_t lo, bool cached, bool mass_mode, unsigned kk, double top_p, uint32_t* key_out,
                              unsigned* cnt_out, unsigned long long* mass_out) {
    const int hist = (threadIdx.x >> 6) & (kFilterHists - 1);
    FilterRange range{lo, 0, 0, 0, 0u};
    unsigned base_c = 0;
    unsigned long long base_m = 0, target = 0;
    for (int level = 0; level < 6; ++level) {
        range.level = level;
        for (int i = threadIdx.x; i < kFilterHists * 256; i += kFilterThreads) {
            (&L.cnt[0][0])[i] = 0u;
            (&L.mass[0][0])[i] = 0ull;
        }
        __syncthreads();
        auto add = [&](int F, uint32_t key, unsigned long long ms) {
            const int bin = range.bin(F, key);
            atomicAdd(&L.cnt[hist][bin], 1u);
            atomicAdd(&L.mass[hist][bin], ms);
        };
        if (cached) {
            for (int i = threadIdx.x; i < L.n_cache; i += kFilterThreads) {
                const uint32_t key = L.c_key[i];
                const int F = dist_index(key_value(key), m);
                if (range.contains(F, key)) add(F, key, L.c_mass[i]);
            }
        } else {
            for_row(row, V, vec4, m, logz, range, add);
        }
        __syncthreads();
        if (threadIdx.x < 64) filter_select(L, mass_mode, kk, base_m, target, top_p, level == 0);
        __syncthreads();
        const FilterSel sel = L.sel;
        if (level == 0 && mass_mode) target = (unsigned long long)(top_p * (double)sel.total);
        base_c += sel.cnt_above;
        base_m += sel.mass_above;
        if (!mass_mode) kk -= sel.cnt_above;
        if (level == 0) range.hi_byte = 255 - sel.bin;
        else if (level == 1) range.lo_byte = 255 - sel.bin;
        else range.prefix = (range.prefix << 8) | (uint32_t)sel.bin;
        if (level == 5) {
            *key_out = range.prefix;
            *cnt_out = base_c + sel.cnt_bin;
            *mass_out = base_m + sel.mass_bin;
        } else if (!cached && sel.cnt_bin <= (unsigned)kFilterCache) {
            // the next range is the chosen bin: small enough to keep in LDS
            FilterRange next = range;
            next.level = level + 1;
            filter_gather(L, row, V, vec4, m, logz, next);
            cached = true;
        }
    }
}

__global__ __launch_bounds__(kFilterThreads) void k_filter(const Plan P, const float* __restrict__ logits,
                                                           const RowStat* __restrict__ rowstat,
                                                           FiltStat* __restrict__ filt,
                                                           int32_t* __restrict__ dbg_count,
                                                           float* __restrict__ dbg_logz) {
    __shared__ FilterLds L;
    const int r = blockIdx.x / P.T1, t = blockIdx.x - r * P.T1;
    const int b = select_of(P.lossless_bits, P.B, r, true);
    if (t > seq_G(P, b)) return;  // past a ragged sequence's drafts: the whole block leaves
    const int pidx = b * P.T1 + t;
    const float* row = logits + (size_t)pidx * P.K * P.V;
    const RowStat rs = rowstat[pidx * P.K];
    const bool use_k = P.top_k > 0 && P.top_k < P.V;
    const bool use_p = P.top_p > 0.0f && P.top_p < 1.0f;
    const bool vec4 = P.vec4 && (reinterpret_cast<uintptr_t>(row) & 15u) == 0;

    uint32_t key = 0u, lo = 0u;
    unsigned cnt = (unsigned)P.V;
    unsigned long long mass = 0ull;
    bool cached = false;
    if (use_k) {
        filter_search(L, row, P.V, vec4, rs.m, rs.logz, 0u, false, false, (unsigned)P.top_k, 0.0, &key, &cnt,
                      &mass);
        lo = key;
        if (use_p && cnt <= (unsigned)kFilterCache) {
            // the whole top-k set fits: the top-p search reads only its copy
            filter_gather(L, row, P.V, vec4, rs.m, rs.logz, FilterRange{lo, 0, 0, 0, 0u});
            cached = true;
        }
    }
    if (use_p)
        filter_search(L, row, P.V, vec4, rs.m, rs.logz, lo, cached, true, 0u, (double)P.top_p, &key, &cnt, &mass);
    if (threadIdx.x == 0) {
        const float lz = (float)((double)rs.logz + log((double)mass * 8.673617379884035e-19));  // 2^-60
        filt[pidx] = FiltStat{key_value(key), lz, (int)cnt, 0};
        if (dbg_count) dbg_count[pidx] = (int)cnt;
        if (dbg_logz) dbg_logz[pidx] = lz;
    }
}

__global__ void k_fill_i32(int32_t* __restrict__ p, int n, int32_t v) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

// =====================================================================
// launch wrappers
// =====================================================================
hipError_t launch_prep(const Plan& P, const void* h, void* Hm, RowMeta* meta, uint32_t* dbg_mask, hipStream_t st) {
    if (P.w_packed) {
        const size_t n16 = (size_t)P.R_phys * P.nkb * 4;
        // large plans: four consecutive pieces of a row per thread, so the
        // row lookup and index arithmetic are paid once per four; small
        // plans keep one piece per thread (latency: more threads in flight)
        const bool four = P.nkb % 4 == 0 && n16 >= kPrepFourMin;
        const dim3 grid((unsigned)(((four ? n16 / 4 : n16) + 255) / 256));
        if (P.dtype == 1) {
            if (four)
                hipLaunchKernelGGL((k_prep_packed<true, 4>), grid, dim3(256), 0, st, P, h, Hm, meta, dbg_mask);
            else
                hipLaunchKernelGGL((k_prep_packed<true, 1>), grid, dim3(256), 0, st, P, h, Hm, meta, dbg_mask);
        } else {
            if (four)
                hipLaunchKernelGGL((k_prep_packed<false, 4>), grid, dim3(256), 0, st, P, h, Hm, meta, dbg_mask);
            else
                hipLaunchKernelGGL((k_prep_packed<false, 1>), grid, dim3(256), 0, st, P, h, Hm, meta, dbg_mask);
        }
        return hipGetLastError();
    }
    const dim3 grid(P.R_phys, ((P.d >> 3) + 255) / 256);
    if (P.dtype == 1)
        hipLaunchKernelGGL(k_prep<true>, grid, dim3(256), 0, st, P, h, Hm, meta, dbg_mask);
    else
        hipLaunchKernelGGL(k_prep<false>, grid, dim3(256), 0, st, P, h, Hm, meta, dbg_mask);
    return hipGetLastError();
}

hipError_t launch_pack_w(const void* W, void* Wp, int V, int nkb, size_t n16, hipStream_t st) {
    const size_t blocks = (n16 + 255) / 256;
    hipLaunchKernelGGL(k_pack_w, dim3((unsigned)blocks), dim3(256), 0, st, (const uint8_t*)W, (uint8_t*)Wp, V, nkb,
                       n16);
    return hipGetLastError();
}

// The few-wave panel variant: fewer waves than the GPU has SIMDs (256 CUs x
// 4), so no wave competes for bandwidth and latency bounds each one.
static bool panel_deep(const Plan& P) { return (long long)P.n_panels * P.n_tiles < 1024; }

template <bool BF16>
static hipError_t launch_panel_t(const Plan& P, const void* Wp, const void* Hp, const RowMeta* meta, float* logits,
                                 Stat* part, hipStream_t st) {
    dim3 grid((P.n_panels + kPanelWaves - 1) / kPanelWaves, P.n_tiles), block(kPanelWaves * 64);
    const uint8_t* w = (const uint8_t*)Wp;
    const uint8_t* a = (const uint8_t*)Hp;
    if (panel_deep(P)) {
        switch (P.msub) {
            case 1: hipLaunchKernelGGL((k_gemm_panel<BF16, 1, true>), grid, block, 0, st, P, w, a, meta, logits, part); break;
            case 2: hipLaunchKernelGGL((k_gemm_panel<BF16, 2, true>), grid, block, 0, st, P, w, a, meta, logits, part); break;
            case 3: hipLaunchKernelGGL((k_gemm_panel<BF16, 3, true>), grid, block, 0, st, P, w, a, meta, logits, part); break;
            default: hipLaunchKernelGGL((k_gemm_panel<BF16, 4, true>), grid, block, 0, st, P, w, a, meta, logits, part); break;
        }
        return hipGetLastError();
    }
    switch (P.msub) {
        case 1: hipLaunchKernelGGL((k_gemm_panel<BF16, 1, false>), grid, block, 0, st, P, w, a, meta, logits, part); break;
        case 2: hipLaunchKernelGGL((k_gemm_panel<BF16, 2, false>), grid, block, 0, st, P, w, a, meta, logits, part); break;
        case 3: hipLaunchKernelGGL((k_gemm_panel<BF16, 3, false>), grid, block, 0, st, P, w, a, meta, logits, part); break;
        default: hipLaunchKernelGGL((k_gemm_panel<BF16, 4, false>), grid, block, 0, st, P, w, a, meta, logits, part); break;
    }
    return hipGetLastError();
}

template <bool BF16>
static hipError_t launch_skinny_t(const Plan& P, const void* W, const void* Hm, float* logits, Stat* part,
                                  hipStream_t st) {
    dim3 grid(P.n_vgroups, P.n_tiles), block(kSkinnyWaves * 64);
    const uint8_t* w = (const uint8_t*)W;
    const uint8_t* a = (const uint8_t*)Hm;
    switch (P.msub) {
        case 1: hipLaunchKernelGGL((k_gemm_skinny<BF16, 1, kSkinnyNS, kSkinnyWaves>), grid, block, 0, st, P, w, a, logits, part); break;
        case 2: hipLaunchKernelGGL((k_gemm_skinny<BF16, 2, kSkinnyNS, kSkinnyWaves>), grid, block, 0, st, P, w, a, logits, part); break;
        case 3: hipLaunchKernelGGL((k_gemm_skinny<BF16, 3, kSkinnyNS, kSkinnyWaves>), grid, block, 0, st, P, w, a, logits, part); break;
        default: hipLaunchKernelGGL((k_gemm_skinny<BF16, 4, kSkinnyNS, kSkinnyWaves>), grid, block, 0, st, P, w, a, logits, part); break;
    }
    return hipGetLastError();
}

template <bool BF16>
static hipError_t launch_tile_t(const Plan& P, const void* Wp, const void* Hp, const RowMeta* meta, float* logits,
                                Stat* part, hipStream_t st) {
    const int n_groups = (P.n_panels + 3) / 4;
    const int per_xcd = (n_groups + 7) / 8;
    dim3 grid(8 * per_xcd * P.n_tiles), block(kTileWaves * 64);
    const uint8_t* w = (const uint8_t*)Wp;
    const uint8_t* a = (const uint8_t*)Hp;
    switch (P.msub) {
        case 4: hipLaunchKernelGGL((k_gemm_tile<BF16, 4>), grid, block, 0, st, P, w, a, meta, logits, part); break;
        case 5: hipLaunchKernelGGL((k_gemm_tile<BF16, 5>), grid, block, 0, st, P, w, a, meta, logits, part); break;
        case 6: hipLaunchKernelGGL((k_gemm_tile<BF16, 6>), grid, block, 0, st, P, w, a, meta, logits, part); break;
        case 7: hipLaunchKernelGGL((k_gemm_tile<BF16, 7>), grid, block, 0, st, P, w, a, meta, logits, part); break;
        case 8: hipLaunchKernelGGL((k_gemm_tile<BF16, 8>), grid, block, 0, st, P, w, a, meta, logits, part); break;
        case 9: hipLaunchKernelGGL((k_gemm_tile<BF16, 9>), grid, block, 0, st, P, w, a, meta, logits, part); break;
        case 10:
            hipLaunchKernelGGL((k_gemm_tile<BF16, 10>), grid, block, 0, st, P, w, a, meta, logits, part);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_gemm(const Plan& P, const void* W, const void* Hm, const RowMeta* meta, float* logits, Stat* part,
                       hipStream_t st) {
    if (P.w_packed && P.tile_kernel)
        return P.dtype == 1 ? launch_tile_t<true>(P, W, Hm, meta, logits, part, st)
                            : launch_tile_t<false>(P, W, Hm, meta, logits, part, st);
    if (P.w_packed)
        return P.dtype == 1 ? launch_panel_t<true>(P, W, Hm, meta, logits, part, st)
                            : launch_panel_t<false>(P, W, Hm, meta, logits, part, st);
    return P.dtype == 1 ? launch_skinny_t<true>(P, W, Hm, logits, part, st)
                        : launch_skinny_t<false>(P, W, Hm, logits, part, st);
}

int skinny_strips_per_group() { return kSkinnyNS * kSkinnyWaves; }

hipError_t launch_combine(const Plan& P, const Stat* part, RowStat* rowstat, RowStat* centstat,
                          unsigned long long* race_best, int32_t* dbg_head_arg, float* dbg_head_logz,
                          int32_t* dbg_cent_arg, float* dbg_cent_logz, hipStream_t st) {
    const int n = P.R_phys + P.n_lossy_pos;
    hipLaunchKernelGGL(k_combine, dim3(n), dim3(kCombineThreads), 0, st, P, part, rowstat, centstat, race_best,
                       dbg_head_arg, dbg_head_logz, dbg_cent_arg, dbg_cent_logz);
    return hipGetLastError();
}

hipError_t launch_filter(const Plan& P, const float* logits, const RowStat* rowstat, FiltStat* filt,
                         int32_t* dbg_count, float* dbg_logz, hipStream_t st) {
    if (!P.filter || P.n_lossless_seq == 0) return hipSuccess;
    hipLaunchKernelGGL(k_filter, dim3(P.n_lossless_seq * P.T1), dim3(kFilterThreads), 0, st, P, logits, rowstat, filt,
                       dbg_count, dbg_logz);
    return hipGetLastError();
}

hipError_t launch_vocab(const Plan& P, const int32_t* draft, const float* q_hat, const int32_t* tree_parent,
                        const float* logits, const RowStat* rowstat, const RowStat* centstat, float* jspart,
                        unsigned long long* race_best, const FiltStat* filt, int32_t* accept_len, int32_t* out_token,
                        int32_t* accept_pos, uint32_t* data_status, uint8_t* dbg_flags, float* dbg_js_heads,
                        float* dbg_js_draft, hipStream_t st) {
    if (P.blk_js + P.blk_race > 0) {
        const dim3 grid(P.blk_js + P.blk_race), block(kVocabThreads);
        auto kernel = P.vec4 ? k_vocab<kMaxK, true> : k_vocab<kMaxK, false>;
        if (P.K <= 5)
            kernel = P.vec4 ? k_vocab<5, true> : k_vocab<5, false>;
        else if (P.K <= 8)
            kernel = P.vec4 ? k_vocab<8, true> : k_vocab<8, false>;
        hipLaunchKernelGGL(kernel, grid, block, 0, st, P, draft, q_hat, logits, rowstat, centstat, jspart, race_best,
                           filt);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_finish, dim3(P.B), dim3(kFinishThreads), 0, st, P, draft, q_hat, tree_parent, logits,
                       rowstat, centstat, jspart, race_best, filt, accept_len, out_token, accept_pos, data_status,
                       dbg_flags, dbg_js_heads, dbg_js_draft);
    return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t* p, int n, int32_t v, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_fill_i32, dim3((n + 255) / 256), dim3(256), 0, st, p, n, v);
    return hipGetLastError();
}

}  // namespace dmv
