// Host-only check of the LM-head row layout (no HIP call is made): includes
// the library's host source with the kernel launches stubbed out, then for
// many shapes verifies that every (sequence, position, head) maps to exactly
// one physical GEMM row inside the workspace, that row_info inverts
// lossy_row / lossless_row, and that all workspace indices stay in bounds.
#include "../../speculative_decoding_verification_philox_amd/csrc/dm_verify.cpp"

#include <cstdio>
#include <vector>

namespace dmv {
hipError_t launch_prep(const Plan&, const void*, void*, RowMeta*, uint32_t*, hipStream_t) { return hipSuccess; }
hipError_t launch_pack_w(const void*, void*, int, int, size_t, hipStream_t) { return hipSuccess; }
hipError_t launch_gemm(const Plan&, const void*, const void*, const RowMeta*, float*, Stat*, hipStream_t) {
    return hipSuccess;
}
hipError_t launch_combine(const Plan&, const Stat*, RowStat*, RowStat*, unsigned long long*, int32_t*, float*,
                          int32_t*, float*, hipStream_t) {
    return hipSuccess;
}
hipError_t launch_filter(const Plan&, const float*, const RowStat*, FiltStat*, int32_t*, float*, hipStream_t) {
    return hipSuccess;
}
hipError_t launch_vocab(const Plan&, const int32_t*, const float*, const int32_t*, const float*, const RowStat*,
                        const RowStat*, float*, unsigned long long*, const FiltStat*, int32_t*, int32_t*, int32_t*,
                        uint32_t*, uint8_t*, float*, float*, hipStream_t) {
    return hipSuccess;
}
hipError_t launch_fill_i32(int32_t*, int, int32_t, hipStream_t) { return hipSuccess; }
int skinny_strips_per_group() { return 32; }
}  // namespace dmv

static int fails = 0;
#define CHECK(c, ...)                                  \
    do {                                               \
        if (!(c)) {                                    \
            if (fails < 20) std::printf(__VA_ARGS__);  \
            ++fails;                                   \
        }                                              \
    } while (0)

static void check_case(int d, int V, int maxB, int gamma, int kmax, int B, int K, unsigned seed, int wp) {
    dm_verify_desc D{d, V, maxB, gamma, kmax, DM_DTYPE_BF16};
    std::vector<uint8_t> modes(B);
    unsigned s = seed;
    int nl = 0, nj = 0;
    for (int b = 0; b < B; ++b) {
        s = s * 1103515245u + 12345u;
        modes[b] = (uint8_t)((s >> 16) % 4);
        if (seed == 0) modes[b] = DM_MODE_JS_MAJORITY;
        if (seed == 1) modes[b] = DM_MODE_LOSSLESS;
        nl += modes[b] == DM_MODE_LOSSLESS;
        nj += modes[b] == DM_MODE_JS_MAJORITY;
    }
    Plan P{};
    make_plan(D, B, K, nl, nj, wp, P);
    for (int b = 0; b < B; ++b) {
        if (modes[b] == DM_MODE_LOSSLESS) P.lossless_bits[b >> 5] |= 1u << (b & 31);
        if (modes[b] == DM_MODE_JS_MAJORITY) P.js_bits[b >> 5] |= 1u << (b & 31);
        if (modes[b] == DM_MODE_TREE_NAIVE) P.tree_bits[b >> 5] |= 1u << (b & 31);
    }
    Sizes sz = workspace_sizes(D);
    const int T1 = gamma + 1;
    CHECK((size_t)P.R_phys * d * 2 <= sz.hm, "Hm overflow\n");
    CHECK((size_t)P.R_phys * sizeof(RowMeta) <= sz.meta, "row metadata overflow\n");
    CHECK(!wp || (P.n_vgroups == (P.n_panels + 3) / 4 && (long long)P.n_panels * 64 >= V && P.nkb * 64 == d * 2),
          "panel split\n");
    // packed Hm: the last fragment of the last tile ends exactly at R_phys rows
    CHECK((size_t)P.n_tiles * P.nkb * P.msub * 1024 == (size_t)P.R_phys * d * 2, "packed Hm size\n");
    CHECK((size_t)P.n_vgroups * (P.R_phys + P.n_lossy_pos) * sizeof(Stat) <= sz.part, "part overflow\n");
    CHECK((size_t)P.n_js_pos * P.js_chunks * (K + 1) * sizeof(float) <= sz.jspart || P.n_js_pos == 0,
          "jspart overflow\n");
    CHECK(P.GR * P.ppg <= 2 * P.MT && P.ppg >= 1, "tile shape\n");
    CHECK(P.tile_kernel ? (wp && P.msub >= 4 && P.msub <= 10) : (P.MT <= 64 && P.msub >= 1 && P.msub <= 4),
          "kernel choice %d msub %d\n", P.tile_kernel, P.msub);
    CHECK(P.n_js_pos == 0 || ((long long)P.js_chunks * P.js_chunk >= V && (long long)(P.js_chunks - 1) * P.js_chunk < V),
          "js chunks\n");
    CHECK(nl == 0 || ((long long)P.race_chunks * P.race_chunk >= V && (long long)(P.race_chunks - 1) * P.race_chunk < V),
          "race chunks\n");
    // a race block covers at most kRaceChunkMax entries in whole 1024-entry steps
    CHECK(nl == 0 || (P.race_chunk <= kRaceChunkMax && P.race_chunk % 1024 == 0), "race chunk %d\n", P.race_chunk);
    CHECK(sz.race >= (size_t)B * kRaceSlotStride * sizeof(unsigned long long), "race slots\n");
    CHECK(P.blk_js == P.n_js_pos * P.js_chunks && P.blk_race == nl * P.race_chunks, "block count\n");
    CHECK(gamma <= kMaxGamma && T1 <= 64, "gamma beyond one wave of positions\n");
    std::vector<int> seen((size_t)B * T1 * K, 0);
    for (int rho = 0; rho < P.R_phys; ++rho) {
        RowInfo ri = row_info(P, rho);
        if (ri.b < 0) continue;
        CHECK(ri.b < B && ri.t >= 0 && ri.t < T1 && ri.i >= 0 && ri.i < K, "row %d out of range\n", rho);
        bool lossless = modes[ri.b] == DM_MODE_LOSSLESS;
        CHECK(lossless == !ri.lossy, "row %d mode\n", rho);
        CHECK(!lossless || ri.i == 0, "lossless head\n");
        seen[((size_t)ri.b * T1 + ri.t) * K + ri.i]++;
        if (ri.lossy) {
            CHECK(lossy_row(P, ri.lossy_pos, ri.i) == rho, "lossy_row inverse %d\n", rho);
            int rank = rank_of(P.lossless_bits, ri.b, false);
            CHECK(ri.lossy_pos == rank * T1 + ri.t, "lossy position numbering\n");
        } else {
            int q = rank_of(P.lossless_bits, ri.b, true) * T1 + ri.t;
            CHECK(lossless_row(P, q) == rho, "lossless_row inverse %d\n", rho);
        }
    }
    for (int b = 0; b < B; ++b)
        for (int t = 0; t < T1; ++t)
            for (int i = 0; i < K; ++i) {
                int want = (modes[b] != DM_MODE_LOSSLESS || i == 0) ? 1 : 0;
                CHECK(seen[((size_t)b * T1 + t) * K + i] == want, "coverage b=%d t=%d i=%d -> %d\n", b, t, i,
                      seen[((size_t)b * T1 + t) * K + i]);
            }
    // a lossy position's heads share one lane group of one tile
    for (int p = 0; p < P.n_lossy_pos; ++p) {
        int r0 = lossy_row(P, p, 0);
        for (int i = 1; i < K; ++i) {
            int r = lossy_row(P, p, i);
            int g0, l0, g1, l1;
            tile_slot(P.geom, r0 % P.MT, &g0, &l0);
            tile_slot(P.geom, r % P.MT, &g1, &l1);
            CHECK(r / P.MT == r0 / P.MT && g0 == g1 && l1 == l0 + i, "position %d heads split\n", p);
        }
    }
    // JS positions map to JS sequences
    for (int jp = 0; jp < P.n_js_pos; ++jp) {
        int b = select_of(P.js_bits, B, jp / P.G, true);
        CHECK(b >= 0 && modes[b] == DM_MODE_JS_MAJORITY, "js select\n");
        CHECK(rank_of(P.js_bits, b, true) == jp / P.G, "js rank\n");
    }
}

// Ragged batches (per-sequence drafts and heads) through plan_call: only
// live positions get rows, every live (b, t, i) exactly once, a position's
// heads in one lane group, and class_pos inverting the position numbering.
static void check_ragged_case(int d, int V, int maxB, int gamma, int kmax, int B, int K, unsigned seed, int wp) {
    dm_verify_desc D{d, V, maxB, gamma, kmax, DM_DTYPE_BF16};
    std::vector<uint8_t> modes(B);
    std::vector<int32_t> sg(B), sk(B);
    unsigned s = seed * 2654435761u + 1u;
    for (int b = 0; b < B; ++b) {
        s = s * 1103515245u + 12345u;
        modes[b] = (uint8_t)((s >> 16) % 4);
        s = s * 1103515245u + 12345u;
        sg[b] = (int)((s >> 16) % (unsigned)(gamma + 1));
        s = s * 1103515245u + 12345u;
        sk[b] = 1 + (int)((s >> 16) % (unsigned)K);
    }
    dm_verify_args a{};
    a.modes = modes.data();
    a.batch = B;
    a.K = K;
    a.p_drop = 0.2f;
    a.w_layout = (uint32_t)wp;
    a.seq_gamma = sg.data();
    a.seq_heads = sk.data();
    Plan P{};
    plan_call(D, &a, P);
    const int T1 = gamma + 1;
    int live[2] = {0, 0};
    for (int b = 0; b < B; ++b) live[modes[b] == DM_MODE_LOSSLESS] += sg[b] + 1;
    CHECK(P.ragged && P.n_lossy_pos == live[0] && P.n_lossless_pos == live[1], "ragged position counts\n");
    Sizes sz = workspace_sizes(D);
    CHECK((size_t)P.R_phys * d * 2 <= sz.hm && (size_t)P.R_phys * sizeof(RowMeta) <= sz.meta, "ragged Hm\n");
    CHECK((size_t)P.n_vgroups * (P.R_phys + P.n_lossy_pos) * sizeof(Stat) <= sz.part, "ragged part\n");
    std::vector<int> seen((size_t)B * T1 * K, 0);
    int rows_live = 0;
    for (int rho = 0; rho < P.R_phys; ++rho) {
        RowInfo ri = row_info(P, rho);
        if (ri.b < 0) continue;
        ++rows_live;
        CHECK(ri.b < B && ri.t >= 0 && ri.t <= sg[ri.b] && ri.i >= 0, "ragged row %d out of range\n", rho);
        const bool lossless = modes[ri.b] == DM_MODE_LOSSLESS;
        CHECK(lossless ? ri.i == 0 : ri.i < sk[ri.b], "ragged row %d head\n", rho);
        if (ri.b < B && ri.t >= 0 && ri.t < T1 && ri.i >= 0 && ri.i < K) seen[((size_t)ri.b * T1 + ri.t) * K + ri.i]++;
    }
    int want_rows = 0;
    for (int b = 0; b < B; ++b)
        for (int t = 0; t <= sg[b]; ++t) {
            const int heads = modes[b] == DM_MODE_LOSSLESS ? 1 : sk[b];
            want_rows += heads;
            for (int i = 0; i < heads; ++i)
                CHECK(seen[((size_t)b * T1 + t) * K + i] == 1, "ragged coverage b=%d t=%d i=%d\n", b, t, i);
        }
    CHECK(rows_live == want_rows, "ragged live rows %d, want %d\n", rows_live, want_rows);
    // rows computed: the tiles the live positions need, no more
    const int tiles = (live[0] ? (live[0] + P.GR * P.ppg - 1) / (P.GR * P.ppg) : 0) +
                      (live[1] ? (live[1] + P.GR * P.S - 1) / (P.GR * P.S) : 0);
    CHECK(P.n_tiles == tiles && P.R_phys == tiles * P.MT, "ragged tiles %d, want %d\n", P.n_tiles, tiles);
    for (int c = 0; c < 2; ++c) {
        const int n = c ? P.n_lossless_pos : P.n_lossy_pos;
        int pb = -1, pt = -1;
        for (int p = 0; p < n; ++p) {
            int b, t;
            class_pos(P, c, p, &b, &t);
            CHECK(b >= 0 && b < B && (modes[b] == DM_MODE_LOSSLESS) == (c == 1) && t >= 0 && t <= sg[b],
                  "class_pos %d %d\n", c, p);
            CHECK(b > pb || (b == pb && t == pt + 1), "class_pos order %d %d\n", c, p);
            pb = b;
            pt = t;
        }
    }
    for (int p = 0; p < P.n_lossy_pos; ++p) {
        int r0 = lossy_row(P, p, 0);
        for (int i = 1; i < K; ++i) {
            int r = lossy_row(P, p, i);
            int g0, l0, g1, l1;
            tile_slot(P.geom, r0 % P.MT, &g0, &l0);
            tile_slot(P.geom, r % P.MT, &g1, &l1);
            CHECK(r / P.MT == r0 / P.MT && g0 == g1 && l1 == l0 + i, "ragged position %d heads split\n", p);
        }
    }
}

// select_of against a plain scan, for random sets and every rank.
static void check_select() {
    unsigned s = 12345u;
    for (int trial = 0; trial < 2000; ++trial) {
        uint32_t bits[kMaskWords];
        for (int w = 0; w < kMaskWords; ++w) {
            s = s * 1103515245u + 12345u;
            uint32_t x = s;
            s = s * 1103515245u + 12345u;
            x ^= s << 7;
            if (trial % 5 == 0) x = 0u;
            if (trial % 7 == 0) x = 0xffffffffu;
            bits[w] = x;
        }
        const int B = 1 + (int)(s % 256u);
        for (int set = 0; set <= 1; ++set) {
            int rank = 0;
            for (int b = 0; b < B; ++b) {
                if ((int)bit_of(bits, b) == set) {
                    CHECK(select_of(bits, B, rank, set) == b, "select_of rank %d -> %d, want %d\n", rank,
                          select_of(bits, B, rank, set), b);
                    ++rank;
                }
            }
            CHECK(select_of(bits, B, rank, set) == -1, "select_of past the end\n");
        }
    }
}

int main() {
    check_select();
    int cases = 0;
    const int Ks[] = {1, 2, 3, 4, 5, 7, 8, 13, 16};
    for (int kmax : {5, 8, 16})
        for (int K : Ks) {
            if (K > kmax) continue;
            for (int B : {1, 2, 7, 32, 64, 200, 256})
                for (int gamma : {0, 4, 7, 31, 63})
                    for (unsigned seed : {0u, 1u, 2u, 3u}) {
                        for (int wp = 0; wp <= 1; ++wp) {
                            check_case(512, 5003, 256, gamma, kmax, B, K, seed, wp);
                            ++cases;
                        }
                    }
        }
    for (int wp = 0; wp <= 1; ++wp) {
        check_case(8192, 128256, 32, 7, 5, 32, 5, 0, wp);
        check_case(5120, 151936, 64, 5, 8, 64, 8, 2, wp);
        check_case(4096, 128256, 1, 7, 5, 1, 5, 0, wp);
        check_case(64, 20000, 256, 1, 1, 256, 1, 1, wp);  // many races: chunks cut to kRaceChunkMax
        cases += 4;
    }
    for (int wp = 0; wp <= 1; ++wp)
        for (int K : {1, 3, 5, 8, 16})
            for (int B : {1, 5, 32, 64, 256})
                for (int gamma : {0, 3, 7, 63})
                    for (unsigned seed : {0u, 1u, 2u}) {
                        check_ragged_case(512, 5003, 256, gamma, 16, B, K, seed, wp);
                        ++cases;
                    }
    std::printf("%d cases, %d failures\n", cases, fails);
    return fails ? 1 : 0;
}
