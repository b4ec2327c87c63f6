// dm_kernels.hip -- HIP kernels of the DropMatch verify step for gfx950.
//
//   k_prep        dropout masks from Philox, masked hidden rows in GEMM order
//   k_gemm_skinny LM-head GEMM for short M (all rows of a tile in one
//                 workgroup; W streamed from HBM straight into MFMA operands),
//                 with a softmax-statistics epilogue per row and per centroid
//   k_combine     merges the per-vocabulary-group statistics
//   k_js          Jensen-Shannon terms over the vocabulary
//   k_decide      acceptance rules, first-reject scan, lossy emit
//   k_race        exponential race over the residual (lossless emit)
//   k_emit        picks the race winner
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dm_common.hpp"
#include "dm_launch.hpp"

namespace dmv {

typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// =====================================================================
// k_prep: Hm[rho, :] = h[b, t, :] * keep(b, t, i, :) for every GEMM row.
// DropMatch Sec. 3.1 Eq. (1): independent Bernoulli(1 - p_drop) keeps per
// (position, head, element), drawn from Philox stream 0 with counter
// (j / 4, b * (gamma + 1) + t, i, 0).  The inverted-dropout scale of Eq. (2)
// is applied to the fp32 accumulator later, so masked values stay exact.
// One block per GEMM row; a thread handles 32 consecutive elements.
// =====================================================================
template <bool BF16>
__global__ __launch_bounds__(256) void k_prep(const Plan P, const void* __restrict__ h, void* __restrict__ Hm,
                                              uint32_t* __restrict__ dbg_mask) {
    const int rho = blockIdx.x;
    const RowInfo ri = row_info(P, rho);
    const int nchunk = P.d >> 5;
    const int esz = BF16 ? 2 : 4;
    const size_t src_row = ri.b >= 0 ? (size_t)(ri.b * P.T1 + ri.t) * P.d : 0;
    for (int c = threadIdx.x; c < nchunk; c += blockDim.x) {
        uint32_t bits = 0u;
        if (ri.b >= 0) {
            if (ri.lossy) {
                const uint32_t pidx = (uint32_t)(ri.b * P.T1 + ri.t);
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    u32x4 r = philox10(u32x4{(uint32_t)(c * 8 + q), pidx, (uint32_t)ri.i, kStreamMask}, P.key0, P.key1);
                    bits |= (uint32_t)(r.x >= P.thresh) << (4 * q);
                    bits |= (uint32_t)(r.y >= P.thresh) << (4 * q + 1);
                    bits |= (uint32_t)(r.z >= P.thresh) << (4 * q + 2);
                    bits |= (uint32_t)(r.w >= P.thresh) << (4 * q + 3);
                }
            } else {
                bits = 0xffffffffu;
            }
        }
        const uint8_t* src = (const uint8_t*)h + (src_row + (size_t)c * 32) * esz;
        uint8_t* dst = (uint8_t*)Hm + ((size_t)rho * P.d + (size_t)c * 32) * esz;
        if (BF16) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                v4u x = ri.b >= 0 ? *(const v4u*)(src + 16 * v) : v4u{0, 0, 0, 0};
                uint32_t m8 = (bits >> (8 * v)) & 0xffu;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    uint32_t w = x[k];
                    uint32_t lo = (m8 >> (2 * k)) & 1u, hi = (m8 >> (2 * k + 1)) & 1u;
                    w = (lo ? (w & 0x0000ffffu) : 0u) | (hi ? (w & 0xffff0000u) : 0u);
                    x[k] = w;
                }
                *(v4u*)(dst + 16 * v) = x;
            }
        } else {
#pragma unroll
            for (int v = 0; v < 8; ++v) {
                v4u x = ri.b >= 0 ? *(const v4u*)(src + 16 * v) : v4u{0, 0, 0, 0};
#pragma unroll
                for (int k = 0; k < 4; ++k) x[k] = ((bits >> (4 * v + k)) & 1u) ? x[k] : 0u;
                *(v4u*)(dst + 16 * v) = x;
            }
        }
        if (dbg_mask && ri.b >= 0)
            dbg_mask[((size_t)(ri.b * P.T1 + ri.t) * P.K + ri.i) * nchunk + c] = bits;
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
        s_scale[threadIdx.x] = valid ? (ri.lossy ? P.scale : 1.0f) : 0.0f;
        s_canon[threadIdx.x] = valid ? (ri.b * P.T1 + ri.t) * P.K + ri.i : -1;
        s_store[threadIdx.x] =
            valid && (P.store_all || !ri.lossy || (bit_of(P.js_bits, ri.b) && ri.t < P.G));
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
            for (int c = 0; c < ncol; ++c) {
                float lb = centroid_logit(P.K, [&](int i) { return et[tile_row(0, g, slot * P.K + i) * PITCH + c]; });
                stat_push(st, lb, vbase + c);
            }
        }
        sstat[wave][ROWS + lane] = st;
    }
    __syncthreads();
    const int n_targets = P.R_phys + P.n_lossy_pos;
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
        part[(size_t)vg * n_targets + target] = st;
    }
}

// =====================================================================
// k_combine: final (max, log Z, argmax) per head row and per centroid.
// =====================================================================
__global__ __launch_bounds__(256) void k_combine(const Plan P, const Stat* __restrict__ part,
                                                 RowStat* __restrict__ rowstat, RowStat* __restrict__ centstat,
                                                 int32_t* __restrict__ dbg_head_arg, float* __restrict__ dbg_head_logz,
                                                 int32_t* __restrict__ dbg_cent_arg,
                                                 float* __restrict__ dbg_cent_logz) {
    const int n_targets = P.R_phys + P.n_lossy_pos;
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= n_targets) return;
    int b, pos_t, head = 0;
    bool is_row = t < P.R_phys, lossless = false;
    if (is_row) {
        RowInfo ri = row_info(P, t);
        if (ri.b < 0) return;
        b = ri.b;
        pos_t = ri.t;
        head = ri.i;
        lossless = !ri.lossy;
    } else {
        const int p = t - P.R_phys;
        b = select_of(P.lossless_bits, P.B, p / P.T1, false);
        pos_t = p % P.T1;
    }
    Stat st = stat_empty();
    for (int vg = 0; vg < P.n_vgroups; ++vg) st = stat_merge(st, part[(size_t)vg * n_targets + t]);
    RowStat rs{st.m, st.m + logf(st.s), st.idx};
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
// k_js: partial sums over a vocabulary chunk of JS(p^(i) || p-bar) for each
// head and of JS(q_hat || p-bar) (DropMatch Eq. (6); natural-log divergence
// with M = (P + Q) / 2).  Each term is evaluated in log space:
//   log M = max(a, b) + log1p(exp(-|a - b|)) - ln 2,
//   term  = (e^a (a - log M) + e^b (b - log M)) / 2.
// =====================================================================
__device__ __forceinline__ float js_term(float a, float b) {
    const float mx = fmaxf(a, b), dl = fabsf(a - b);
    const float lm = mx + log1pf(__expf(-dl)) - 0.69314718055994531f;
    return 0.5f * (__expf(a) * (a - lm) + __expf(b) * (b - lm));
}

__device__ __forceinline__ float js_term_q(float q, float b) {
    if (!(q > 0.0f)) return 0.5f * __expf(b) * 0.69314718055994531f;
    return js_term(__logf(q), b);
}

constexpr int kJsThreads = 256;

__global__ __launch_bounds__(kJsThreads) void k_js(const Plan P, const float* __restrict__ logits,
                                                   const float* __restrict__ q_hat,
                                                   const RowStat* __restrict__ rowstat,
                                                   const RowStat* __restrict__ centstat,
                                                   float* __restrict__ jspart) {
    const int jp = blockIdx.x, c = blockIdx.y;
    const int b = select_of(P.js_bits, P.B, jp / P.G, true);
    const int t = jp % P.G;
    const int pidx = b * P.T1 + t;
    const int K = P.K;
    float logz[kMaxK];
#pragma unroll
    for (int i = 0; i < kMaxK; ++i) {
        logz[i] = 0.0f;
        if (i < K) logz[i] = rowstat[pidx * K + i].logz;
    }
    const float logz_c = centstat[pidx].logz;
    float acc[kMaxK + 1];
#pragma unroll
    for (int i = 0; i <= kMaxK; ++i) acc[i] = 0.0f;
    const int v0 = c * P.js_chunk;
    int v1 = v0 + P.js_chunk;
    v1 = v1 < P.V ? v1 : P.V;
    const float* lrow = logits + (size_t)pidx * K * P.V;
    const float* qrow = q_hat + (size_t)(b * P.G + t) * P.V;
    for (int v = v0 + threadIdx.x; v < v1; v += kJsThreads) {
        float l[kMaxK];
#pragma unroll
        for (int i = 0; i < kMaxK; ++i) {
            l[i] = 0.0f;
            if (i < K) l[i] = lrow[(size_t)i * P.V + v];
        }
        // same operations, in the same order, as centroid_logit()
        float lsum = l[0];
#pragma unroll
        for (int i = 1; i < kMaxK; ++i)
            if (i < K) lsum += l[i];
        const float lb = lsum / (float)K;
        const float bb = lb - logz_c;
#pragma unroll
        for (int i = 0; i < kMaxK; ++i)
            if (i < K) acc[i] += js_term(l[i] - logz[i], bb);
        acc[kMaxK] += js_term_q(qrow[v], bb);
    }
    // block reduction, fixed order
    __shared__ float red[kJsThreads / 64][kMaxK + 1];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i <= kMaxK; ++i) {
        if (i < K || i == kMaxK) {
            float x = acc[i];
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
            if (lane == 0) red[wave][i] = x;
        }
    }
    __syncthreads();
    if (threadIdx.x <= K) {
        const int i = threadIdx.x == K ? kMaxK : threadIdx.x;
        float x = 0.0f;
#pragma unroll
        for (int w = 0; w < kJsThreads / 64; ++w) x += red[w][i];
        jspart[((size_t)jp * P.js_chunks + c) * (K + 1) + threadIdx.x] = x;
    }
}

// =====================================================================
// k_decide: one wave per sequence.  Lane t < gamma decides drafted position
// t with the sequence's rule; a ballot gives the first rejection A
// ("Speculative Decoding: Draft, Then Verify", the draft-then-verify loop,
// step 3).  Lossy sequences emit the centroid argmax at A; lossless ones
// leave the emit to the residual race and reset its slots here.
// =====================================================================
__global__ __launch_bounds__(64) void k_decide(const Plan P, const int32_t* __restrict__ draft,
                                               const float* __restrict__ q_hat, const float* __restrict__ logits,
                                               const RowStat* __restrict__ rowstat,
                                               const RowStat* __restrict__ centstat,
                                               const float* __restrict__ jspart, int32_t* __restrict__ accept_len,
                                               int32_t* __restrict__ out_token,
                                               unsigned long long* __restrict__ race_best,
                                               uint8_t* __restrict__ dbg_flags, float* __restrict__ dbg_js_heads,
                                               float* __restrict__ dbg_js_draft) {
    const int b = blockIdx.x, t = threadIdx.x;
    const int K = P.K, G = P.G, T1 = P.T1;
    const bool lossless = bit_of(P.lossless_bits, b);
    const bool js = bit_of(P.js_bits, b);
    bool reject = false;
    if (t < G) {
        const int32_t x = draft[b * G + t];
        const bool valid = x >= 0 && x < P.V;
        const int pidx = b * T1 + t;
        bool accept = false;
        if (lossless) {
            if (valid) {
                const float lx = logits[(size_t)pidx * K * P.V + x];
                const float px = __expf(lx - rowstat[pidx * K].logz);
                const float qx = q_hat[(size_t)(b * G + t) * P.V + x];
                u32x4 r = philox10(u32x4{0u, (uint32_t)pidx, 0u, kStreamAccept}, P.key0, P.key1);
                const float u = (float)(r.x >> 8) * 5.9604644775390625e-08f;
                accept = u * qx < px;
            }
        } else {
            int count = 0;
            for (int i = 0; i < K; ++i) count += rowstat[pidx * K + i].idx == x;
            if (js) {
                const int jp = rank_of(P.js_bits, b, true) * G + t;
                float jmax = -INFINITY, jq = 0.0f;
                for (int i = 0; i <= K; ++i) {
                    float s = 0.0f;
                    for (int c = 0; c < P.js_chunks; ++c) s += jspart[((size_t)jp * P.js_chunks + c) * (K + 1) + i];
                    if (i < K) {
                        jmax = fmaxf(jmax, s);
                        if (dbg_js_heads) dbg_js_heads[(size_t)(b * G + t) * K + i] = s;
                    } else {
                        jq = s;
                    }
                }
                if (dbg_js_draft) dbg_js_draft[b * G + t] = jq;
                accept = valid && (jq <= jmax || 2 * count > K);
            } else {
                accept = valid && count > 0;
            }
        }
        reject = !accept;
        if (dbg_flags) dbg_flags[b * G + t] = accept ? 1 : 0;
    }
    const unsigned long long rej = __ballot(reject);
    const int A = rej ? __ffsll((long long)rej) - 1 : G;
    if (t == 0) {
        accept_len[b] = A;
        if (!lossless) {
            out_token[b] = centstat[b * T1 + A].idx;
        } else {
            race_best[2 * b] = 0ull;
            race_best[2 * b + 1] = 0ull;
        }
    }
}

// =====================================================================
// k_race: exponential race over the emit distribution of a lossless
// sequence ("Why speculative decoding preserves distributions...", Sec. 5:
// sample normalize((p_A - q_A)+) after a rejection, p_gamma otherwise).
// Entry v gets the clock E_v = -ln U_v (Philox stream 2); the winner
// maximises w_v / E_v, smaller v on ties.  A second race over p_A itself
// covers the zero-residual fallback.  Winners are packed as
// (key bits << 32) | (~v) and merged with a 64-bit atomic max.
// =====================================================================
constexpr int kRaceThreads = 256;

__device__ __forceinline__ unsigned long long race_pack(float key, int v) {
    return ((unsigned long long)__float_as_uint(key) << 32) | (unsigned long long)(0xffffffffu - (uint32_t)v);
}

__global__ __launch_bounds__(kRaceThreads) void k_race(const Plan P, const float* __restrict__ q_hat,
                                                       const float* __restrict__ logits,
                                                       const RowStat* __restrict__ rowstat,
                                                       const int32_t* __restrict__ accept_len,
                                                       unsigned long long* __restrict__ race_best) {
    const int b = select_of(P.lossless_bits, P.B, blockIdx.x, true);
    const int A = accept_len[b];
    const int pidx = b * P.T1 + A;
    const float logz = rowstat[pidx * P.K].logz;
    const float* lrow = logits + (size_t)pidx * P.K * P.V;
    const float* qrow = A < P.G ? q_hat + (size_t)(b * P.G + A) * P.V : nullptr;
    unsigned long long best_r = 0ull, best_p = 0ull;
    const int v0 = blockIdx.y * P.race_chunk;
    int v1 = v0 + P.race_chunk;
    v1 = v1 < P.V ? v1 : P.V;
    for (int vq = v0 + 4 * threadIdx.x; vq < v1; vq += 4 * kRaceThreads) {
        u32x4 r = philox10(u32x4{(uint32_t)(vq >> 2), (uint32_t)pidx, 0u, kStreamRace}, P.key0, P.key1);
        const uint32_t words[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int v = vq + k;
            if (v >= v1) break;
            const float p = __expf(lrow[v] - logz);
            const float w = qrow ? fmaxf(p - qrow[v], 0.0f) : p;
            const float U = ((float)(words[k] >> 9) + 0.5f) * 1.1920928955078125e-07f;
            const float E = -logf(U);
            if (w > 0.0f) {
                unsigned long long kr = race_pack(w / E, v);
                best_r = kr > best_r ? kr : best_r;
            }
            if (p > 0.0f) {
                unsigned long long kp = race_pack(p / E, v);
                best_p = kp > best_p ? kp : best_p;
            }
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        unsigned long long o = __shfl_xor(best_r, off, 64);
        best_r = o > best_r ? o : best_r;
        o = __shfl_xor(best_p, off, 64);
        best_p = o > best_p ? o : best_p;
    }
    if ((threadIdx.x & 63) == 0) {
        if (best_r) atomicMax(&race_best[2 * b], best_r);
        if (best_p) atomicMax(&race_best[2 * b + 1], best_p);
    }
}

__global__ __launch_bounds__(256) void k_emit(const Plan P, const unsigned long long* __restrict__ race_best,
                                              int32_t* __restrict__ out_token) {
    const int r = blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= P.n_lossless_seq) return;
    const int b = select_of(P.lossless_bits, P.B, r, true);
    unsigned long long best = race_best[2 * b];
    if (!best) best = race_best[2 * b + 1];
    out_token[b] = best ? (int32_t)(0xffffffffu - (uint32_t)(best & 0xffffffffull)) : 0;
}

__global__ void k_fill_i32(int32_t* __restrict__ p, int n, int32_t v) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

// =====================================================================
// launch wrappers
// =====================================================================
hipError_t launch_prep(const Plan& P, const void* h, void* Hm, uint32_t* dbg_mask, hipStream_t st) {
    if (P.dtype == 1)
        hipLaunchKernelGGL(k_prep<true>, dim3(P.R_phys), dim3(256), 0, st, P, h, Hm, dbg_mask);
    else
        hipLaunchKernelGGL(k_prep<false>, dim3(P.R_phys), dim3(256), 0, st, P, h, Hm, dbg_mask);
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

hipError_t launch_gemm(const Plan& P, const void* W, const void* Hm, float* logits, Stat* part, hipStream_t st) {
    return P.dtype == 1 ? launch_skinny_t<true>(P, W, Hm, logits, part, st)
                        : launch_skinny_t<false>(P, W, Hm, logits, part, st);
}

int skinny_strips_per_group() { return kSkinnyNS * kSkinnyWaves; }

hipError_t launch_combine(const Plan& P, const Stat* part, RowStat* rowstat, RowStat* centstat, int32_t* dbg_head_arg,
                          float* dbg_head_logz, int32_t* dbg_cent_arg, float* dbg_cent_logz, hipStream_t st) {
    const int n = P.R_phys + P.n_lossy_pos;
    hipLaunchKernelGGL(k_combine, dim3((n + 255) / 256), dim3(256), 0, st, P, part, rowstat, centstat, dbg_head_arg,
                       dbg_head_logz, dbg_cent_arg, dbg_cent_logz);
    return hipGetLastError();
}

hipError_t launch_js(const Plan& P, const float* logits, const float* q_hat, const RowStat* rowstat,
                     const RowStat* centstat, float* jspart, hipStream_t st) {
    hipLaunchKernelGGL(k_js, dim3(P.n_js_pos, P.js_chunks), dim3(kJsThreads), 0, st, P, logits, q_hat, rowstat,
                       centstat, jspart);
    return hipGetLastError();
}

hipError_t launch_decide(const Plan& P, const int32_t* draft, const float* q_hat, const float* logits,
                         const RowStat* rowstat, const RowStat* centstat, const float* jspart, int32_t* accept_len,
                         int32_t* out_token, unsigned long long* race_best, uint8_t* dbg_flags, float* dbg_js_heads,
                         float* dbg_js_draft, hipStream_t st) {
    hipLaunchKernelGGL(k_decide, dim3(P.B), dim3(64), 0, st, P, draft, q_hat, logits, rowstat, centstat, jspart,
                       accept_len, out_token, race_best, dbg_flags, dbg_js_heads, dbg_js_draft);
    return hipGetLastError();
}

hipError_t launch_race(const Plan& P, const float* q_hat, const float* logits, const RowStat* rowstat,
                       const int32_t* accept_len, unsigned long long* race_best, int32_t* out_token, hipStream_t st) {
    hipLaunchKernelGGL(k_race, dim3(P.n_lossless_seq, P.race_chunks), dim3(kRaceThreads), 0, st, P, q_hat, logits,
                       rowstat, accept_len, race_best);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_emit, dim3((P.n_lossless_seq + 255) / 256), dim3(256), 0, st, P, race_best, out_token);
    return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t* p, int n, int32_t v, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_fill_i32, dim3((n + 255) / 256), dim3(256), 0, st, p, n, v);
    return hipGetLastError();
}

}  // namespace dmv
