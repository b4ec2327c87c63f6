// dm_common.hpp -- internal definitions shared by the host side and the
// kernels of libdmverify: the per-call plan, the LM-head row layout, the
// device Philox4x32-10, and softmax-statistic merging.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dmv {

constexpr int kMaxBatch = 256;
constexpr int kMaxK = 16;
constexpr int kMaxGamma = 63;  // drafts (tree nodes) per sequence: positions fit one wave
constexpr int kMaskWords = kMaxBatch / 32;
constexpr int kMaxDropValues = 8;  // distinct per-sequence dropout probabilities in one call
// 64-bit words per sequence in the residual-race slots: its two slots alone
// in a 128-byte line, so the atomics of different sequences never share one
constexpr int kRaceSlotStride = 16;
constexpr int kRaceChunkMax = 4096;  // vocabulary entries of one residual-race block

enum Mode : int { kLossless = 0, kNaive = 1, kJs = 2, kTreeNaive = 3 };

// Row layout of the LM-head GEMM ("slot layout").
//
// The GEMM's M dimension is cut into tiles of MT rows.  Inside a tile the
// MFMA output layout gives each lane `GR` row groups; a lane holds the rows of
// one group for one vocabulary column.  Each group has S row slots, and a
// position occupies K consecutive slots of one group (one per dropout head),
// so every head of a position lands in the same lane as its siblings.  Lossy
// positions fill tiles first (ppg = S / K per group), lossless positions
// (one undropped row each) fill the tiles after them.
//
// geom 0: 16x16 MFMA output, a tile is MT = 16 * msub rows, GR = 4 groups,
//         row r of the tile = 16 m + 4 g + j  (slot lambda = 4 m + j).
// geom 1: 32x32 MFMA output, a tile is MT = 32 * msub rows, GR = 2 groups,
//         row r = 32 m + 8 a + 4 g + c        (slot lambda = 16 m + 4 a + c).
struct Plan {
    // problem
    int B, T1, G, K, V, d;
    int dtype;           // 0 f32, 1 bf16
    float scale;         // 1 / ((1 - p_drop) temperature), the dropout rows
    float inv_k;         // 1 / K, the centroid's mean weight
    uint32_t thresh;     // keep iff Philox word >= thresh
    uint32_t key0, key1; // Philox key (seed low, high)
    // sequences
    uint32_t lossless_bits[kMaskWords];
    uint32_t js_bits[kMaskWords];
    uint32_t tree_bits[kMaskWords];  // naive matching on a token tree
    int n_lossy_seq, n_lossless_seq, n_js_seq;
    // sampling settings: row scales include 1 / temperature; the filter
    // (top-k, top-p) applies to lossless rows when `filter` is set
    float scale_undropped;
    int filter, top_k;
    float top_p;
    // ragged batches: per-sequence drafts and heads, and the dropout of each
    // sequence as an index into a small table of (threshold, scale); G, K
    // above are the largest, which fix the layout
    int ragged;
    uint8_t seq_gamma[kMaxBatch], seq_k[kMaxBatch], seq_pi[kMaxBatch];
    uint32_t p_thresh[kMaxDropValues];
    float p_scale[kMaxDropValues];
    // ragged batches lay out live positions only: class 0 (lossy) and 1
    // (lossless) number their positions sequence by sequence in batch
    // order; rk_seq[c][r] is the r-th sequence of class c and rk_start[c][r]
    // its first position (rk_start[c][n] the class's position count)
    uint8_t rk_seq[2][kMaxBatch];
    uint16_t rk_start[2][kMaxBatch + 1];
    // slot layout
    int geom, msub, MT, GR, S;
    int ppg;                // lossy positions per group (S / K)
    int n_lossy_pos, n_lossless_pos;
    int tiles_lossy, n_tiles, R_phys;
    // stored logits: rows of [B * T1 * K, V]
    int store_all;
    // LM-head weight order: 0 row-major, 1 panels of 64 rows (dm_verify_pack_w)
    int w_packed;
    int tile_kernel;  // 1: panel-ordered W past one small tile (k_gemm_tile), else 0
    int nkb;       // 64-byte fragments per weight row (row bytes / 64)
    int n_panels;  // ceil(V / 64)
    // vocabulary split of the GEMM's statistic partials
    int n_vgroups;
    // vocabulary pass: JS blocks, then race blocks
    int n_js_pos, js_chunks, js_chunk;
    int vec4;  // logits and q_hat rows are 16-byte aligned (V % 4 == 0)
    int race_chunks, race_chunk;
    int blk_js, blk_race;
};

// Per-sequence drafts, heads, dropout threshold and row scale, and the
// centroid weight 1 / K_b (the same fp32 value everywhere it is used).
__host__ __device__ inline int seq_G(const Plan& P, int b) { return P.ragged ? P.seq_gamma[b] : P.G; }
__host__ __device__ inline int seq_K(const Plan& P, int b) { return P.ragged ? P.seq_k[b] : P.K; }
__host__ __device__ inline uint32_t seq_thresh(const Plan& P, int b) {
    return P.ragged ? P.p_thresh[P.seq_pi[b]] : P.thresh;
}
__host__ __device__ inline float seq_scale(const Plan& P, int b) { return P.ragged ? P.p_scale[P.seq_pi[b]] : P.scale; }
__host__ __device__ inline float seq_inv_k(const Plan& P, int b) {
    return P.ragged ? 1.0f / (float)P.seq_k[b] : P.inv_k;
}

// ------------------------------------------------------------------ layout
__host__ __device__ inline bool bit_of(const uint32_t* bits, int b) {
    return (bits[b >> 5] >> (b & 31)) & 1u;
}

// Number of set bits of `bits` below position b (or of clear bits, for the
// complement set), within [0, B).
__host__ __device__ inline int rank_of(const uint32_t* bits, int b, bool set) {
    int r = 0;
    for (int w = 0; w < (b >> 5); ++w) {
        uint32_t x = set ? bits[w] : ~bits[w];
        r += __builtin_popcount(x);
    }
    uint32_t x = set ? bits[b >> 5] : ~bits[b >> 5];
    uint32_t below = (b & 31) ? (x & ((1u << (b & 31)) - 1u)) : 0u;
    return r + __builtin_popcount(below);
}

// Position of the k-th (0-based) set bit of x; x has more than k set bits.
__host__ __device__ inline int select_in_word(uint32_t x, int k) {
    int pos = 0;
    for (int w = 16; w >= 1; w >>= 1) {
        const uint32_t low = x & ((1u << w) - 1u);
        const int c = __builtin_popcount(low);
        if (k >= c) {
            k -= c;
            x >>= w;
            pos += w;
        } else {
            x = low;
        }
    }
    return pos;
}

// The sequence index of the `rank`-th member of the set (set bits when `set`,
// clear bits otherwise) among sequences [0, B); -1 if there is none.
__host__ __device__ inline int select_of(const uint32_t* bits, int B, int rank, bool set) {
    if (rank < 0) return -1;
    const int nw = (B + 31) >> 5;
    for (int w = 0; w < nw; ++w) {
        uint32_t x = set ? bits[w] : ~bits[w];
        const int valid = B - 32 * w;  // sequences covered by this word
        if (valid < 32) x &= (1u << valid) - 1u;
        const int c = __builtin_popcount(x);
        if (rank < c) return 32 * w + select_in_word(x, rank);
        rank -= c;
    }
    return -1;
}

__host__ __device__ inline int tile_row(int geom, int g, int lambda) {
    if (geom == 0) return 16 * (lambda >> 2) + 4 * g + (lambda & 3);
    return 32 * (lambda >> 4) + 8 * ((lambda & 15) >> 2) + 4 * g + (lambda & 3);
}

__host__ __device__ inline void tile_slot(int geom, int r, int* g, int* lambda) {
    if (geom == 0) {
        *g = (r & 15) >> 2;
        *lambda = 4 * (r >> 4) + (r & 3);
    } else {
        int rr = r & 31;
        *g = (rr & 7) >> 2;
        *lambda = 16 * (r >> 5) + 4 * (rr >> 3) + (rr & 3);
    }
}

// Per physical GEMM row, written by k_prep for the LM-head epilogue.
struct RowMeta {
    int canon;    // (b * T1 + t) * K + i, or -1 for a padding row
    float scale;  // 1 / ((1 - p_drop) T) for a dropout row, 1 / T undropped, 0 padding
    int store;    // 1 if the row's logits are kept for the vocabulary pass
    float inv_k;  // 1 / K_b of a dropout row's sequence (its position's centroid weight), 0 otherwise
};

// What a physical GEMM row holds.
struct RowInfo {
    int b, t, i;   // sequence, position, head; b < 0 for a padding row
    int lossy;     // 1 if the row is masked and scaled
    int lossy_pos; // index of the lossy position (centroid slot), -1 otherwise
};

// Sequence b and position t of live position p of class cls (0 lossy, 1
// lossless).  A uniform batch has gamma + 1 positions per sequence; a ragged
// one gamma_b + 1, found by a binary search of the class's starts.
__host__ __device__ inline void class_pos(const Plan& P, int cls, int p, int* b, int* t) {
    if (!P.ragged) {
        *b = select_of(P.lossless_bits, P.B, p / P.T1, cls == 1);
        *t = p % P.T1;
        return;
    }
    const uint16_t* start = P.rk_start[cls];
    int lo = 0, hi = (cls ? P.n_lossless_seq : P.n_lossy_seq) - 1;  // the last r with start[r] <= p
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if ((int)start[mid] <= p)
            lo = mid;
        else
            hi = mid - 1;
    }
    *b = P.rk_seq[cls][lo];
    *t = p - (int)start[lo];
}

__host__ __device__ inline RowInfo row_info(const Plan& P, int rho) {
    RowInfo ri{-1, 0, 0, 0, -1};
    int tile = rho / P.MT, r = rho - tile * P.MT;
    int g, lam;
    tile_slot(P.geom, r, &g, &lam);
    if (tile < P.tiles_lossy) {
        int slot = lam / P.K;
        if (slot >= P.ppg) return ri;
        int p = (tile * P.GR + g) * P.ppg + slot;
        if (p >= P.n_lossy_pos) return ri;
        class_pos(P, 0, p, &ri.b, &ri.t);
        ri.i = lam - slot * P.K;
        ri.lossy = 1;
        ri.lossy_pos = p;
        // a ragged sequence's head slots past its heads are padding
        if (P.ragged && ri.i >= P.seq_k[ri.b]) return RowInfo{-1, 0, 0, 0, -1};
    } else {
        int q = ((tile - P.tiles_lossy) * P.GR + g) * P.S + lam;
        if (q >= P.n_lossless_pos) return ri;
        class_pos(P, 1, q, &ri.b, &ri.t);
        ri.i = 0;
        ri.lossy = 0;
    }
    return ri;
}

// Physical row of head i of lossy position p.
__host__ __device__ inline int lossy_row(const Plan& P, int p, int i) {
    int grp = p / P.ppg, slot = p - grp * P.ppg;
    int tile = grp / P.GR, g = grp - tile * P.GR;
    return tile * P.MT + tile_row(P.geom, g, slot * P.K + i);
}

// Physical row of lossless position q.
__host__ __device__ inline int lossless_row(const Plan& P, int q) {
    int grp = q / P.S, lam = q - grp * P.S;
    int tile = P.tiles_lossy + grp / P.GR, g = grp % P.GR;
    return tile * P.MT + tile_row(P.geom, g, lam);
}

// ------------------------------------------------------------ Philox4x32-10
// Salmon, Moraes, Dror, Shaw (SC'11): ten rounds; each round multiplies
// counter words 0 and 2 by the two Philox multipliers, XORs the high halves
// with the crossed counter words and the round key, and the key advances by
// the two Weyl increments.
struct u32x4 {
    uint32_t x, y, z, w;
};

__device__ __forceinline__ u32x4 philox10(u32x4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint32_t m0 = 0xD2511F53u, m1 = 0xCD9E8D57u;
        // one 32 x 32 -> 64-bit product gives both halves (v_mad_u64_u32)
        const uint64_t p0 = (uint64_t)m0 * c.x, p1 = (uint64_t)m1 * c.z;
        const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        c = u32x4{hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0};
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return c;
}

// Stream tags (counter word 3).
constexpr uint32_t kStreamMask = 0u, kStreamAccept = 1u, kStreamRace = 2u;

// ------------------------------------------------------------- statistics
// Softmax statistics of a set of logits: running max m, s = sum exp(l - m)
// and the smallest index attaining m.
struct Stat {
    float m;
    float s;
    int idx;
};

__device__ __forceinline__ Stat stat_empty() { return Stat{-INFINITY, 0.0f, 0x7fffffff}; }

__device__ __forceinline__ void stat_push(Stat& a, float v, int idx) {
    if (v > a.m) {
        a.s = a.s * __expf(a.m - v) + 1.0f;
        a.m = v;
        a.idx = idx;
    } else {
        a.s += __expf(v - a.m);
        if (v == a.m && idx < a.idx) a.idx = idx;
    }
}

__device__ __forceinline__ Stat stat_merge(Stat a, Stat b) {
    if (b.m == -INFINITY) return a;
    if (a.m == -INFINITY) return b;
    Stat r;
    if (a.m > b.m) {
        r.m = a.m;
        r.s = a.s + b.s * __expf(b.m - a.m);
        r.idx = a.idx;
    } else if (b.m > a.m) {
        r.m = b.m;
        r.s = b.s + a.s * __expf(a.m - b.m);
        r.idx = b.idx;
    } else {
        r.m = a.m;
        r.s = a.s + b.s;
        r.idx = a.idx < b.idx ? a.idx : b.idx;
    }
    return r;
}

__device__ __forceinline__ Stat stat_shfl_xor(Stat a, int off) {
    Stat o;
    o.m = __shfl_xor(a.m, off, 64);
    o.s = __shfl_xor(a.s, off, 64);
    o.idx = __shfl_xor(a.idx, off, 64);
    return o;
}

// Final per-row statistics.
struct RowStat {
    float m;
    float logz;
    int idx;
    float logz1;  // logz - ln 2: the vocabulary pass takes its JS terms from logs shifted by ln 2
};

// The processed target of one lossless position: v is kept iff its logit is
// >= thresh; logz = log of the sum of e^l over the kept tokens.
struct FiltStat {
    float thresh;
    float logz;
    int count;
    int pad;
};

// Mean of the K head logits of one position: the DropMatch centroid logit,
// summed in head order and scaled by inv_k = 1 / K.  Every kernel that forms
// it uses this order and this scaling, so the values agree bit for bit.
template <class Get>
__device__ __forceinline__ float centroid_logit(int K, float inv_k, Get get) {
    float s = get(0);
    for (int i = 1; i < K; ++i) s += get(i);
    return s * inv_k;
}

// ----------------------------------------------------------- bf16 helpers
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

}  // namespace dmv
