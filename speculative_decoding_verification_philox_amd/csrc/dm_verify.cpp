// dm_verify.cpp -- host side of libdmverify: argument checks, the per-call
// plan (row layout, work split), workspace, and the kernel sequence.
#include "../../include/dm_verify.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>

#include "dm_common.hpp"
#include "dm_launch.hpp"

using namespace dmv;

struct dm_verify {
    dm_verify_desc desc;
    int device;
    uint8_t* ws;
    size_t ws_bytes;
    void* Hm;
    float* logits;
    Stat* part;
    RowStat* rowstat;
    RowStat* centstat;
    RowMeta* meta;
    float* jspart;
    unsigned long long* race;
    FiltStat* filt;
    size_t cap_hm, cap_part, cap_jspart, cap_meta_rows;
    hipEvent_t prof_start, prof_stop;
};

namespace {

constexpr int kGroupsPerTile = 4;
// Planner weight of one tile of the matrix-core kernel, in rows: every tile
// streams the whole weight slice of its panel group and runs one epilogue.
// Fitted to GEMM times over every sub-tile count at the wide mixed shape
// (1728 rows, K = 8; the fit gives 24..51 rows per tile) and checked at the
// batched 70B and the 60-node tree, whose best counts it keeps.
constexpr double kTileFixedRows = 40.0;
// The vocabulary pass splits a position into at most 256 chunks of 2048.
constexpr int kMaxVocab = 256 * 2048;  // 16x16 MFMA output: four row groups per lane

int elem_size(int dtype) { return dtype == DM_DTYPE_BF16 ? 2 : 4; }

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int check_desc(const dm_verify_desc* D) {
    if (!D) return DM_ERR_INVALID_ARGUMENT;
    if (D->d <= 0 || D->vocab <= 0 || D->max_batch <= 0 || D->gamma < 0 || D->k_max <= 0)
        return DM_ERR_INVALID_ARGUMENT;
    if (D->max_batch > kMaxBatch || D->gamma > kMaxGamma || D->k_max > kMaxK || D->vocab > kMaxVocab)
        return DM_ERR_INVALID_ARGUMENT;
    if (D->dtype != DM_DTYPE_F32 && D->dtype != DM_DTYPE_BF16) return DM_ERR_UNSUPPORTED;
    if (D->d % 64 != 0 || D->d > 65536) return DM_ERR_UNSUPPORTED;
    return DM_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int check_args(const dm_verify_desc* D, const dm_verify_args* a) {
    if (!a) return DM_ERR_INVALID_ARGUMENT;
    if (a->w_layout != DM_W_ROW_MAJOR && a->w_layout != DM_W_PANELS) return DM_ERR_INVALID_ARGUMENT;
    if (a->batch < 1 || a->batch > D->max_batch) return DM_ERR_INVALID_ARGUMENT;
    if (a->K < 1 || a->K > D->k_max) return DM_ERR_INVALID_ARGUMENT;
    if (!(a->p_drop >= 0.0f && a->p_drop < 1.0f)) return DM_ERR_INVALID_ARGUMENT;
    if (!(a->temperature >= 0.0f) || !std::isfinite(a->temperature)) return DM_ERR_INVALID_ARGUMENT;
    if (a->top_k < 0 || !(a->top_p >= 0.0f) || !std::isfinite(a->top_p) || a->reserved != 0)
        return DM_ERR_INVALID_ARGUMENT;
    if (!a->W || !a->h || !a->modes || !a->accept_len || !a->out_token) return DM_ERR_INVALID_ARGUMENT;
    if (D->gamma > 0 && !a->draft) return DM_ERR_INVALID_ARGUMENT;
    bool need_q = false, need_tree = false;
    for (int b = 0; b < a->batch; ++b) {
        uint8_t m = a->modes[b];
        if (m > DM_MODE_TREE_NAIVE) return DM_ERR_INVALID_ARGUMENT;
        if (m == DM_MODE_LOSSLESS || m == DM_MODE_JS_MAJORITY) need_q = true;
        if (m == DM_MODE_TREE_NAIVE) need_tree = true;
        if (a->seq_gamma && (a->seq_gamma[b] < 0 || a->seq_gamma[b] > D->gamma)) return DM_ERR_INVALID_ARGUMENT;
        if (a->seq_heads && (a->seq_heads[b] < 1 || a->seq_heads[b] > a->K)) return DM_ERR_INVALID_ARGUMENT;
        if (a->seq_p_drop && !(a->seq_p_drop[b] >= 0.0f && a->seq_p_drop[b] < 1.0f)) return DM_ERR_INVALID_ARGUMENT;
    }
    if (a->seq_p_drop) {
        float seen[kMaxDropValues];
        int n = 0;
        for (int b = 0; b < a->batch; ++b) {
            int k = 0;
            while (k < n && seen[k] != a->seq_p_drop[b]) ++k;
            if (k == n) {
                if (n == kMaxDropValues) return DM_ERR_UNSUPPORTED;
                seen[n++] = a->seq_p_drop[b];
            }
        }
    }
    if (need_q && D->gamma > 0 && !a->q_hat) return DM_ERR_INVALID_ARGUMENT;
    if (need_tree && D->gamma > 0 && !a->tree_parent) return DM_ERR_INVALID_ARGUMENT;
    if (!aligned(a->W, 16) || !aligned(a->h, 16)) return DM_ERR_UNSUPPORTED;
    const void* four[] = {a->draft, a->q_hat, a->accept_len, a->out_token, a->head_argmax, a->centroid_argmax,
                          a->head_logz, a->centroid_logz, a->js_heads, a->js_draft, a->logits, a->mask_bits,
                          a->filter_count, a->filter_logz, a->tree_parent, a->accept_pos, a->data_status};
    for (const void* p : four)
        if (p && !aligned(p, 4)) return DM_ERR_UNSUPPORTED;
    return DM_OK;
}

uint32_t drop_threshold(float p_drop) {
    // keep iff a 32-bit Philox word is >= T, so P(drop) = T / 2^32
    double t = std::floor((double)p_drop * 4294967296.0 + 0.5);
    if (t > 4294967295.0) t = 4294967295.0;
    if (t < 0.0) t = 0.0;
    return (uint32_t)t;
}

int cdiv(long long a, long long b) { return (int)((a + b - 1) / b); }

// Row layout and work split of one call.  lossy_pos / lossless_pos are the
// live positions of each class (a ragged batch has fewer than gamma + 1 per
// sequence); -1 means gamma + 1 per sequence.
void make_plan(const dm_verify_desc& D, int B, int K, int n_lossless, int n_js, int w_packed, Plan& P,
               int lossy_pos = -1, int lossless_pos = -1) {
    // counts only; the sequence bit sets are filled in by the caller
    P.B = B;
    P.T1 = D.gamma + 1;
    P.G = D.gamma;
    P.K = K;
    P.V = D.vocab;
    P.d = D.d;
    P.dtype = D.dtype;
    P.n_lossless_seq = n_lossless;
    P.n_lossy_seq = B - n_lossless;
    P.n_js_seq = n_js;
    P.n_lossy_pos = lossy_pos >= 0 ? lossy_pos : P.n_lossy_seq * P.T1;
    P.n_lossless_pos = lossless_pos >= 0 ? lossless_pos : n_lossless * P.T1;

    // smallest number of tiles, then the fewest rows
    P.geom = 0;
    P.GR = kGroupsPerTile;
    int best_ms = 0, best_tiles = 0;
    for (int ms = 1; ms <= 4; ++ms) {
        const int S = 4 * ms;
        if (P.n_lossy_pos > 0 && S < K) continue;
        const int ppg = S / K;
        const int tl = P.n_lossy_pos > 0 ? cdiv(P.n_lossy_pos, (long long)P.GR * ppg) : 0;
        const int tn = P.n_lossless_pos > 0 ? cdiv(P.n_lossless_pos, (long long)P.GR * S) : 0;
        if (best_ms == 0 || tl + tn < best_tiles) {
            best_ms = ms;
            best_tiles = tl + tn;
        }
    }
    // Panel-ordered W with more rows than one small tile holds: the
    // matrix-core kernel, one row tile of 4..10 sub-tiles per workgroup of
    // four 64-column panels.  A sub-tile count costs its tiles times
    // (rows per tile + kTileFixedRows): the rows computed, padding included,
    // plus a fixed share per tile for the weight stream every tile reads;
    // the cheapest wins, ties going to the larger tile.
    P.tile_kernel = 0;
    if (w_packed && best_tiles > 1) {
        double best_cost = 0.0;
        best_ms = 0;
        for (int ms = 4; ms <= 10; ++ms) {
            const int S = 4 * ms;
            const int ppg = S / K;  // >= 1: S >= 16 >= K
            const int tl = P.n_lossy_pos > 0 ? cdiv(P.n_lossy_pos, (long long)P.GR * ppg) : 0;
            const int tn = P.n_lossless_pos > 0 ? cdiv(P.n_lossless_pos, (long long)P.GR * S) : 0;
            const double cost = (double)(tl + tn) * (16.0 * ms + kTileFixedRows);
            if (best_ms == 0 || cost <= best_cost) {
                best_ms = ms;
                best_tiles = tl + tn;
                best_cost = cost;
            }
        }
        P.tile_kernel = 1;
    }
    P.msub = best_ms;
    P.MT = 16 * best_ms;
    P.S = 4 * best_ms;
    P.ppg = P.n_lossy_pos > 0 ? P.S / K : 1;
    P.tiles_lossy = P.n_lossy_pos > 0 ? cdiv(P.n_lossy_pos, (long long)P.GR * P.ppg) : 0;
    P.n_tiles = best_tiles;
    P.R_phys = P.n_tiles * P.MT;

    P.w_packed = w_packed;
    P.nkb = (int)((size_t)D.d * elem_size(D.dtype) / 64);
    P.n_panels = cdiv(P.V, 64);
    if (w_packed) {
        // one wave per (panel, tile); statistic partials per group of four
        // panels (both panel-order kernels)
        P.n_vgroups = cdiv(P.n_panels, 4);
    } else {
        const int nstr = cdiv(P.V, 16);
        const int spg = skinny_strips_per_group();
        int ng = cdiv(nstr, spg);
        const int fill = nstr < 256 ? nstr : 256;
        P.n_vgroups = ng > fill ? ng : fill;
    }

    // vocabulary pass: JS positions split into chunks of 2048 entries (eight
    // per thread of a 256-thread block)
    P.n_js_pos = n_js * P.G;
    P.js_chunks = 0;
    P.js_chunk = 2048;
    if (P.n_js_pos > 0) P.js_chunks = cdiv(P.V, P.js_chunk);
    P.race_chunks = 0;
    P.race_chunk = P.V;
    if (n_lossless > 0) {
        int ch = cdiv(1024, n_lossless);
        const int chmax = cdiv(P.V, 1024);
        ch = ch < 1 ? 1 : (ch > chmax ? chmax : ch);
        P.race_chunk = cdiv(cdiv(P.V, ch), 1024) * 1024;
        if (P.race_chunk > kRaceChunkMax) P.race_chunk = kRaceChunkMax;  // a block holds at most this many
        P.race_chunks = cdiv(P.V, P.race_chunk);
    }
    P.blk_js = P.n_js_pos * P.js_chunks;
    P.blk_race = n_lossless * P.race_chunks;
}

struct Sizes {
    size_t hm, logits, part, rowstat, centstat, meta, jspart, race, filt;
};

Sizes workspace_sizes(const dm_verify_desc& D) {
    Sizes s{};
    const size_t T1 = (size_t)D.gamma + 1;
    size_t max_hm_rows = 0, max_part = 0, max_js = 0;
    for (int wp = 0; wp <= 1; ++wp)
        for (int K = 1; K <= D.k_max; ++K) {
            for (int nl = 0; nl <= D.max_batch; ++nl) {
                Plan P{};
                make_plan(D, D.max_batch, K, nl, D.max_batch - nl, wp, P);
                if ((size_t)P.R_phys > max_hm_rows) max_hm_rows = P.R_phys;
                size_t part = (size_t)P.n_vgroups * (P.R_phys + P.n_lossy_pos);
                if (part > max_part) max_part = part;
            }
        }
    // JS positions can be any count up to max_batch * gamma
    for (int nj = 1; nj <= D.max_batch; ++nj) {
        Plan P{};
        make_plan(D, D.max_batch, D.k_max, 0, nj, 0, P);
        size_t js = (size_t)P.n_js_pos * P.js_chunks * (D.k_max + 1);
        if (js > max_js) max_js = js;
    }
    s.hm = max_hm_rows * (size_t)D.d * elem_size(D.dtype);
    s.logits = (size_t)D.max_batch * T1 * D.k_max * D.vocab * sizeof(float);
    s.part = max_part * sizeof(Stat);
    s.rowstat = (size_t)D.max_batch * T1 * D.k_max * sizeof(RowStat);
    s.centstat = (size_t)D.max_batch * T1 * sizeof(RowStat);
    s.meta = max_hm_rows * sizeof(RowMeta);
    s.jspart = (max_js > 0 ? max_js : 1) * sizeof(float);
    s.race = (size_t)D.max_batch * kRaceSlotStride * sizeof(unsigned long long);
    s.filt = (size_t)D.max_batch * T1 * sizeof(FiltStat);
    return s;
}

size_t total_bytes(const Sizes& s) {
    const size_t a = 256;
    return align_up(s.hm, a) + align_up(s.logits, a) + align_up(s.part, a) + align_up(s.rowstat, a) +
           align_up(s.centstat, a) + align_up(s.meta, a) + align_up(s.jspart, a) + align_up(s.race, a) +
           align_up(s.filt, a);
}

// The workspace one planned call uses (the handle's is sized for the worst
// plan of its desc instead).
Sizes plan_sizes(const dm_verify_desc& D, const Plan& P) {
    Sizes s{};
    const size_t rows = (size_t)P.B * P.T1;
    s.hm = (size_t)P.R_phys * D.d * elem_size(D.dtype);
    s.logits = rows * P.K * D.vocab * sizeof(float);
    s.part = (size_t)P.n_vgroups * (P.R_phys + P.n_lossy_pos) * sizeof(Stat);
    s.rowstat = rows * P.K * sizeof(RowStat);
    s.centstat = rows * sizeof(RowStat);
    s.meta = (size_t)P.R_phys * sizeof(RowMeta);
    s.jspart = ((size_t)P.n_js_pos * P.js_chunks * (P.K + 1) + 1) * sizeof(float);
    s.race = (size_t)P.B * kRaceSlotStride * sizeof(unsigned long long);
    s.filt = rows * sizeof(FiltStat);
    return s;
}

// Device buffers of one call.
struct Workspace {
    void* Hm;
    float* logits;
    Stat* part;
    RowStat* rowstat;
    RowStat* centstat;
    RowMeta* meta;
    float* jspart;
    unsigned long long* race;
    FiltStat* filt;
};

// Carves the buffers of `s` out of `base` in a fixed order, each 256-byte aligned.
Workspace carve(uint8_t* base, const Sizes& s) {
    uint8_t* p = base;
    auto take = [&](size_t n) {
        uint8_t* r = p;
        p += align_up(n, 256);
        return r;
    };
    Workspace w;
    w.Hm = take(s.hm);
    w.logits = (float*)take(s.logits);
    w.part = (Stat*)take(s.part);
    w.rowstat = (RowStat*)take(s.rowstat);
    w.centstat = (RowStat*)take(s.centstat);
    w.meta = (RowMeta*)take(s.meta);
    w.jspart = (float*)take(s.jspart);
    w.race = (unsigned long long*)take(s.race);
    w.filt = (FiltStat*)take(s.filt);
    return w;
}

// The call's plan from its (checked) arguments: row layout, work split,
// sequence sets, scales, thresholds and the Philox key.
void plan_call(const dm_verify_desc& D, const dm_verify_args* a, Plan& P) {
    int n_lossless = 0, n_js = 0;
    // live positions of each class: a ragged sequence verifies gamma_b + 1
    int live[2] = {0, 0};
    for (int b = 0; b < a->batch; ++b) {
        n_lossless += a->modes[b] == DM_MODE_LOSSLESS;
        n_js += a->modes[b] == DM_MODE_JS_MAJORITY;
        live[a->modes[b] == DM_MODE_LOSSLESS] += (a->seq_gamma ? a->seq_gamma[b] : D.gamma) + 1;
    }
    make_plan(D, a->batch, a->K, n_lossless, n_js, (int)a->w_layout, P, live[0], live[1]);
    for (int b = 0; b < a->batch; ++b) {
        if (a->modes[b] == DM_MODE_LOSSLESS) P.lossless_bits[b >> 5] |= 1u << (b & 31);
        if (a->modes[b] == DM_MODE_JS_MAJORITY) P.js_bits[b >> 5] |= 1u << (b & 31);
        if (a->modes[b] == DM_MODE_TREE_NAIVE) P.tree_bits[b >> 5] |= 1u << (b & 31);
    }
    // temperature divides every row: folded into the row scales
    const double temp = a->temperature > 0.0f ? (double)a->temperature : 1.0;
    P.scale = (float)(1.0 / ((1.0 - (double)a->p_drop) * temp));
    P.scale_undropped = (float)(1.0 / temp);
    P.top_k = a->top_k;
    P.top_p = a->top_p;
    // ragged batches: per-sequence drafts and heads, dropout by palette index
    P.ragged = a->seq_gamma || a->seq_heads || a->seq_p_drop;
    if (P.ragged) {
        int n_p = 0;
        float pal[kMaxDropValues];
        for (int b = 0; b < a->batch; ++b) {
            P.seq_gamma[b] = (uint8_t)(a->seq_gamma ? a->seq_gamma[b] : D.gamma);
            P.seq_k[b] = (uint8_t)(a->seq_heads ? a->seq_heads[b] : a->K);
            const float pb = a->seq_p_drop ? a->seq_p_drop[b] : a->p_drop;
            int k = 0;
            while (k < n_p && pal[k] != pb) ++k;
            if (k == n_p) {  // at most kMaxDropValues: checked above
                pal[n_p++] = pb;
                P.p_thresh[k] = drop_threshold(pb);
                P.p_scale[k] = (float)(1.0 / ((1.0 - (double)pb) * temp));
            }
            P.seq_pi[b] = (uint8_t)k;
        }
        int rank[2] = {0, 0};
        for (int b = 0; b < a->batch; ++b) {
            const int c = a->modes[b] == DM_MODE_LOSSLESS;
            P.rk_seq[c][rank[c]] = (uint8_t)b;
            P.rk_start[c][rank[c] + 1] = (uint16_t)(P.rk_start[c][rank[c]] + P.seq_gamma[b] + 1);
            ++rank[c];
        }
    }
    P.filter = n_lossless > 0 && ((a->top_k > 0 && a->top_k < D.vocab) || (a->top_p > 0.0f && a->top_p < 1.0f));
    P.inv_k = 1.0f / (float)a->K;
    P.thresh = drop_threshold(a->p_drop);
    P.key0 = (uint32_t)(a->seed & 0xffffffffu);
    P.key1 = (uint32_t)(a->seed >> 32);
    P.store_all = a->logits != nullptr;
}

// Enqueues the kernels of one planned call on `st` over workspace `w`;
// `prof_start` / `prof_stop` (or null) bracket the GEMM launch.
int enqueue(const dm_verify_desc& D, Plan& P, const Workspace& w, const dm_verify_args* a, hipStream_t st,
            hipEvent_t prof_start, hipEvent_t prof_stop) {
    float* logits = a->logits ? a->logits : w.logits;
    P.vec4 = (D.vocab % 4 == 0) && aligned(a->q_hat, 16) && aligned(logits, 16);
    const int T1 = P.T1;
    hipError_t e = hipSuccess;
#define DM_TRY(x)                               \
    do {                                        \
        e = (x);                                \
        if (e != hipSuccess) return DM_ERR_HIP; \
    } while (0)
    if (a->head_argmax) DM_TRY(launch_fill_i32(a->head_argmax, a->batch * T1 * a->K, -1, st));
    if (a->centroid_argmax && P.ragged) DM_TRY(launch_fill_i32(a->centroid_argmax, a->batch * T1, -1, st));
    if (a->mask_bits) DM_TRY(launch_fill_i32((int32_t*)a->mask_bits, a->batch * T1 * a->K * (D.d / 32), 0, st));
    DM_TRY(launch_prep(P, a->h, w.Hm, w.meta, a->mask_bits, st));
    if (prof_start) DM_TRY(hipEventRecord(prof_start, st));
    DM_TRY(launch_gemm(P, a->W, w.Hm, w.meta, logits, w.part, st));
    if (prof_stop) DM_TRY(hipEventRecord(prof_stop, st));
    DM_TRY(launch_combine(P, w.part, w.rowstat, w.centstat, w.race, a->head_argmax, a->head_logz, a->centroid_argmax,
                          a->centroid_logz, st));
    DM_TRY(launch_filter(P, logits, w.rowstat, w.filt, a->filter_count, a->filter_logz, st));
    DM_TRY(launch_vocab(P, a->draft, a->q_hat, a->tree_parent, logits, w.rowstat, w.centstat, w.jspart, w.race,
                        w.filt, a->accept_len, a->out_token, a->accept_pos, a->data_status, a->accept_flags,
                        a->js_heads, a->js_draft, st));
#undef DM_TRY
    return DM_OK;
}

// ---------------------------------------------------- fixed scratch array
// dm_verify_run_static's workspace: a fixed device array, one per GPU, held
// until the process ends, so that entry point allocates nothing.  Host code
// never uses the array's name as an address (on the host it is only a
// stand-in for the symbol): the device address comes from
// hipGetSymbolAddress, once per device, with that device current.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch array, or null on a HIP error.
void* scratch_address(int dev) {
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
            (void)hipGetLastError();
            return nullptr;
        }
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

const char* dm_verify_status_string(int status) {
    switch (status) {
        case DM_OK: return "ok";
        case DM_ERR_INVALID_ARGUMENT: return "invalid argument";
        case DM_ERR_UNSUPPORTED: return "unsupported";
        case DM_ERR_HIP: return "HIP runtime error";
        case DM_ERR_OUT_OF_MEMORY: return "out of device memory";
        case DM_ERR_TOO_LARGE: return "the call's workspace exceeds the fixed scratch array";
        default: return "unknown status";
    }
}

int dm_verify_check(const dm_verify_desc* desc, const dm_verify_args* args) {
    int rc = check_desc(desc);
    if (rc != DM_OK || !args) return rc;
    return check_args(desc, args);
}

size_t dm_verify_workspace_bytes(const dm_verify_desc* desc) {
    if (check_desc(desc) != DM_OK) return 0;
    return total_bytes(workspace_sizes(*desc));
}

int dm_verify_create(const dm_verify_desc* desc, dm_verify_t** out) {
    if (!out) return DM_ERR_INVALID_ARGUMENT;
    *out = nullptr;
    int rc = check_desc(desc);
    if (rc != DM_OK) return rc;
    dm_verify* h = new (std::nothrow) dm_verify();
    if (!h) return DM_ERR_OUT_OF_MEMORY;
    h->desc = *desc;
    if (hipGetDevice(&h->device) != hipSuccess) {
        delete h;
        return DM_ERR_HIP;
    }
    const Sizes s = workspace_sizes(*desc);
    h->ws_bytes = total_bytes(s);
    hipError_t e = hipMalloc((void**)&h->ws, h->ws_bytes);
    if (e != hipSuccess) {
        delete h;
        (void)hipGetLastError();
        return e == hipErrorOutOfMemory ? DM_ERR_OUT_OF_MEMORY : DM_ERR_HIP;
    }
    const Workspace w = carve(h->ws, s);
    h->Hm = w.Hm;
    h->logits = w.logits;
    h->part = w.part;
    h->rowstat = w.rowstat;
    h->centstat = w.centstat;
    h->meta = w.meta;
    h->jspart = w.jspart;
    h->race = w.race;
    h->filt = w.filt;
    h->cap_hm = s.hm;
    h->cap_meta_rows = s.meta / sizeof(RowMeta);
    h->cap_part = s.part;
    h->cap_jspart = s.jspart;
    *out = h;
    return DM_OK;
}

size_t dm_verify_packed_w_bytes(const dm_verify_desc* desc) {
    if (check_desc(desc) != DM_OK) return 0;
    const size_t nkb = (size_t)desc->d * elem_size(desc->dtype) / 64;
    return (size_t)cdiv(desc->vocab, 64) * nkb * 4 * 1024;
}

int dm_verify_pack_w(const dm_verify_desc* desc, const void* W, void* W_packed, void* stream) {
    int rc = check_desc(desc);
    if (rc != DM_OK) return rc;
    if (!W || !W_packed) return DM_ERR_INVALID_ARGUMENT;
    if (!aligned(W, 16) || !aligned(W_packed, 16)) return DM_ERR_UNSUPPORTED;
    const int nkb = (int)((size_t)desc->d * elem_size(desc->dtype) / 64);
    const size_t n16 = dm_verify_packed_w_bytes(desc) / 16;
    if (launch_pack_w(W, W_packed, desc->vocab, nkb, n16, (hipStream_t)stream) != hipSuccess) return DM_ERR_HIP;
    return DM_OK;
}

int dm_verify_profile(dm_verify_t* h, void* start, void* stop) {
    if (!h) return DM_ERR_INVALID_ARGUMENT;
    h->prof_start = (start && stop) ? (hipEvent_t)start : nullptr;
    h->prof_stop = (start && stop) ? (hipEvent_t)stop : nullptr;
    return DM_OK;
}

int dm_verify_destroy(dm_verify_t* h) {
    if (!h) return DM_OK;
    int rc = DM_OK;
    if (h->ws && hipFree(h->ws) != hipSuccess) rc = DM_ERR_HIP;
    delete h;
    return rc;
}

int dm_verify_run(dm_verify_t* h, const dm_verify_args* a, void* stream) {
    if (!h) return DM_ERR_INVALID_ARGUMENT;
    int rc = check_args(&h->desc, a);
    if (rc != DM_OK) return rc;
    const dm_verify_desc& D = h->desc;
    Plan P{};
    plan_call(D, a, P);
    // The workspace was sized for the worst plan of the desc; refuse a plan
    // that would not fit rather than launch past the end of a buffer.
    if ((size_t)P.R_phys * D.d * elem_size(D.dtype) > h->cap_hm || (size_t)P.R_phys > h->cap_meta_rows ||
        (size_t)P.n_vgroups * (P.R_phys + P.n_lossy_pos) * sizeof(Stat) > h->cap_part ||
        (size_t)P.n_js_pos * P.js_chunks * (P.K + 1) * sizeof(float) > h->cap_jspart)
        return DM_ERR_UNSUPPORTED;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != h->device) return DM_ERR_HIP;
    const Workspace w{h->Hm, h->logits, h->part, h->rowstat, h->centstat, h->meta, h->jspart, h->race, h->filt};
    hipEvent_t ps = h->prof_start, pe = h->prof_stop;
    h->prof_start = h->prof_stop = nullptr;  // armed for one run
    return enqueue(D, P, w, a, (hipStream_t)stream, ps && pe ? ps : nullptr, ps && pe ? pe : nullptr);
}

size_t dm_verify_static_scratch_bytes(void) { return kScratchBytes; }

int dm_verify_run_static(const dm_verify_desc* desc, const dm_verify_args* a, void* stream) {
    int rc = check_desc(desc);
    if (rc != DM_OK) return rc;
    rc = check_args(desc, a);
    if (rc != DM_OK) return rc;
    Plan P{};
    plan_call(*desc, a, P);
    const Sizes s = plan_sizes(*desc, P);
    if (total_bytes(s) > kScratchBytes) return DM_ERR_TOO_LARGE;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return DM_ERR_HIP;
    uint8_t* base = (uint8_t*)scratch_address(dev);
    if (!base) return DM_ERR_HIP;
    return enqueue(*desc, P, carve(base, s), a, (hipStream_t)stream, nullptr, nullptr);
}

}  // extern "C"
