/*
 * dm_oracle.c -- TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.
 *
 * A plain, slow, obviously-correct fp64 CPU reference of the DropMatch verify
 * step.  Only the test suite, the smoke check and the benchmark's CPU-baseline
 * leg load this library; the HIP library never links it and shares no code,
 * header, table or helper with it.  Every step below follows the passage it
 * cites, in the order the pages give; where the pages leave a step open the
 * reading taken is named in the comment.
 *
 * Sources (page title, then section / equation):
 *   [DM]  "Training-free Dropout Sampling for Semantic Token Acceptance in
 *         Speculative Decoding" (arXiv 2603.03333): Sec. 3.1 Eq. (1)-(3),
 *         Sec. 3.2 Eq. (4)-(7) and Algorithm 1.
 *   [SD]  "Speculative Decoding: Draft, Then Verify" (abhik.ai): "The
 *         draft-then-verify loop", "The acceptance rule", "Greedy decoding".
 *   [PB]  "Why speculative decoding preserves distributions but may not be
 *         faster" (youchengli.com, probability budget): Sec. 1, Sec. 2, Sec. 5
 *         (verify-round pseudocode).
 *   [TR]  "Speculative Decoding: Draft, Then Verify", "Variants": one
 *         target pass verifies a tree of candidate continuations under a
 *         tree-shaped attention mask (Medusa, EAGLE); [DM] Sec. 4.4: on
 *         EAGLE3's trees the naive rule, Eq. (4), is the one applied.
 *   [PX]  Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as
 *         1, 2, 3" (SC'11): the Philox4x32-10 counter-based generator.
 *
 * Precision: every floating-point quantity is fp64.  bf16 / fp32 inputs are
 * decoded exactly; q_hat is used as stored (fp32 -> fp64, not renormalised).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define DMO_LOSSLESS 0
#define DMO_NAIVE 1
#define DMO_JS 2
#define DMO_TREE_NAIVE 3

/* ------------------------------------------------------------------------ */
/* Philox4x32-10 [PX]: ten rounds of the Philox S-box on a 128-bit counter,  */
/* key bumped by the Weyl constants between rounds.                          */
/* ------------------------------------------------------------------------ */
void dmo_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    const uint32_t MUL0 = 0xD2511F53u, MUL1 = 0xCD9E8D57u;
    const uint32_t WEYL0 = 0x9E3779B9u, WEYL1 = 0xBB67AE85u;
    uint32_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += WEYL0;
            k1 += WEYL1;
        }
        uint64_t prod0 = (uint64_t)MUL0 * (uint64_t)x0;
        uint64_t prod1 = (uint64_t)MUL1 * (uint64_t)x2;
        uint32_t hi0 = (uint32_t)(prod0 >> 32), lo0 = (uint32_t)prod0;
        uint32_t hi1 = (uint32_t)(prod1 >> 32), lo1 = (uint32_t)prod1;
        uint32_t y0 = hi1 ^ x1 ^ k0;
        uint32_t y1 = lo1;
        uint32_t y2 = hi0 ^ x3 ^ k1;
        uint32_t y3 = lo0;
        x0 = y0; x1 = y1; x2 = y2; x3 = y3;
    }
    out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
}

/* One 32-bit word of the stream: counter (c0, c1, c2, c3), word index w. */
static uint32_t philox_word(uint64_t seed, uint32_t c0, uint32_t c1, uint32_t c2,
                            uint32_t c3, int w)
{
    uint32_t ctr[4] = {c0, c1, c2, c3};
    uint32_t key[2] = {(uint32_t)(seed & 0xffffffffu), (uint32_t)(seed >> 32)};
    uint32_t out[4];
    dmo_philox4x32_10(ctr, key, out);
    return out[w];
}

/* Dropout threshold: a 32-bit word r drops its element iff r < T, so the
 * drop probability is T / 2^32 (the Bernoulli(1 - p_drop) keep of [DM]
 * Eq. (1) taken on 32 random bits; reading: integer compare). */
uint32_t dmo_threshold(float p_drop)
{
    double t = floor((double)p_drop * 4294967296.0 + 0.5);
    if (t < 0.0) t = 0.0;
    if (t > 4294967295.0) t = 4294967295.0;
    return (uint32_t)t;
}

/* keep bit of element j for head i at position index pidx = b*(gamma+1)+t.
 * Stream 0: counter (j/4, pidx, i, 0), word j%4. */
static int keep_bit(uint64_t seed, uint32_t pidx, uint32_t head, uint32_t j, uint32_t T)
{
    uint32_t r = philox_word(seed, j >> 2, pidx, head, 0u, (int)(j & 3u));
    return r >= T;
}

/* Acceptance uniform for the lossless test at position index pidx.
 * Stream 1: counter (0, pidx, 0, 1), word 0; 24 bits -> [0, 1). */
double dmo_accept_uniform(uint64_t seed, uint32_t pidx)
{
    uint32_t r = philox_word(seed, 0u, pidx, 0u, 1u, 0);
    return (double)(r >> 8) * (1.0 / 16777216.0);
}

/* Race uniform for vocabulary entry v at position index pidx.
 * Stream 2: counter (v/4, pidx, 0, 2), word v%4; the top 23 bits plus one
 * half, times 2^-23, give a value in (0, 1) that fp32 holds exactly. */
double dmo_race_uniform(uint64_t seed, uint32_t pidx, uint32_t v)
{
    uint32_t r = philox_word(seed, v >> 2, pidx, 0u, 2u, (int)(v & 3u));
    return ((double)(r >> 9) + 0.5) * (1.0 / 8388608.0);
}

static double decode(const void* base, int dtype, size_t idx)
{
    if (dtype == 0) return (double)((const float*)base)[idx];
    uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* ------------------------------------------------------------------------ */
/* Softmax statistics of one logit row ([DM] Eq. (3)): max, log-partition,   */
/* argmax (smallest index attaining the max: the fixed tie rule greedy       */
/* decoding needs, [PB] Sec. 1) and the gap between the two largest values.  */
/* ------------------------------------------------------------------------ */
void dmo_row_stats(const double* l, int n, double* out_max, double* out_logz,
                   int32_t* out_arg, double* out_gap)
{
    double m = -INFINITY, second = -INFINITY;
    int arg = -1;
    for (int v = 0; v < n; ++v) {
        if (l[v] > m) {
            second = m;
            m = l[v];
            arg = v;
        } else if (l[v] > second) {
            second = l[v];
        }
    }
    double z = 0.0;
    for (int v = 0; v < n; ++v) z += exp(l[v] - m);
    if (out_max) *out_max = m;
    if (out_logz) *out_logz = m + log(z);
    if (out_arg) *out_arg = arg;
    if (out_gap) *out_gap = m - second;
}

/* Jensen-Shannon divergence, natural log ([DM] Eq. (6); the paper does not
 * define JS, the reading is the standard divergence with M = (P + Q) / 2 and
 * 0 ln 0 = 0).  P and Q are used as given (not renormalised).  ln M is taken
 * as ln(P + Q) - ln 2, which never forms a halved subnormal that could round
 * to zero. */
double dmo_js(const double* P, const double* Q, int n)
{
    double acc = 0.0;
    for (int v = 0; v < n; ++v) {
        double p = P[v], q = Q[v];
        if (!(p + q > 0.0)) continue;
        double log_mix = log(p + q) - log(2.0);
        double term = 0.0;
        if (p > 0.0) term += p * (log(p) - log_mix);
        if (q > 0.0) term += q * (log(q) - log_mix);
        acc += term;
    }
    return 0.5 * acc;
}

/* Draws one index with probability w_v / sum(w) ([PB] Sec. 5: sample from the
 * normalised weights).  Exact sampler chosen so both sides can be compared
 * bit for bit: each v with w_v > 0 gets an exponential clock E_v = -ln U_v
 * (U_v from stream 2) and the winner maximises w_v / E_v; ties go to the
 * smallest v.  Returns -1 when no weight is positive.  gap_out receives the
 * relative gap between the best and second-best key. */
int32_t dmo_race(const double* w, int n, uint64_t seed, uint32_t pidx, double* gap_out)
{
    int32_t best = -1;
    double best_key = -1.0, second_key = -1.0;
    for (int v = 0; v < n; ++v) {
        if (!(w[v] > 0.0)) continue;
        double u = dmo_race_uniform(seed, pidx, (uint32_t)v);
        double key = w[v] / (-log(u));
        if (key > best_key) {
            second_key = best_key;
            best_key = key;
            best = v;
        } else if (key > second_key) {
            second_key = key;
        }
    }
    if (gap_out) *gap_out = (best >= 0 && second_key > 0.0) ? (best_key - second_key) / best_key : INFINITY;
    return best;
}

/* ------------------------------------------------------------------------ */
/* The processed target distribution.  [PB] Sec. 1: p and q must already     */
/* include temperature, top-k, top-p and the renormalisation; [SD]           */
/* "Production gotchas", "The same sampling settings": the test and the      */
/* residual use the processed p.  Temperature divides the logits before      */
/* this step (see dmo_run).  The pages name top-k and top-p without defining */
/* ties; the readings taken here:                                            */
/*   top-k (0 < k < n): keep every v whose logit is >= the k-th largest      */
/*     logit (ties at the boundary are all kept);                            */
/*   then renormalise over that set S_k;                                     */
/*   top-p (0 < top_p < 1): keep v in S_k iff the renormalised mass of the   */
/*     tokens of S_k with a strictly larger logit is below top_p (the        */
/*     nucleus: the smallest prefix, by probability, whose mass reaches      */
/*     top_p, with the boundary's ties kept);                                */
/*   then renormalise over the kept set S.                                   */
/* k = 0 or >= n, and top_p = 0 or >= 1, switch the filter off.              */
/* Writes p_out (0 off S), returns |S|; *logz_out = log sum_{v in S} e^l_v,  */
/* *margin_out = distance of the decisions from flipping: the smallest of    */
/* the logit gap at the k-th value and the mass gap (relative to S_k's mass) */
/* at the top_p boundary.                                                    */
/* ------------------------------------------------------------------------ */
static const double* g_sort_key;
static int cmp_desc(const void* a, const void* b)
{
    double x = g_sort_key[*(const int32_t*)a], y = g_sort_key[*(const int32_t*)b];
    if (x > y) return -1;
    if (x < y) return 1;
    return (*(const int32_t*)a > *(const int32_t*)b) - (*(const int32_t*)a < *(const int32_t*)b);
}

int dmo_processed(const double* l, int n, int top_k, double top_p, double* p_out, double* logz_out,
                  double* margin_out)
{
    int32_t* ord = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
    if (!ord) return -1;
    for (int v = 0; v < n; ++v) ord[v] = v;
    g_sort_key = l; /* the oracle is single-threaded here */
    qsort(ord, (size_t)n, sizeof(int32_t), cmp_desc);
    const double m = l[ord[0]];
    double margin = INFINITY;

    /* top-k: S_k = the first n_k entries of the order, ties at the k-th kept */
    int n_k = n;
    if (top_k > 0 && top_k < n) {
        const double lk = l[ord[top_k - 1]];
        n_k = top_k;
        while (n_k < n && l[ord[n_k]] == lk) ++n_k;
        if (n_k < n) margin = lk - l[ord[n_k]];
    }
    double z_k = 0.0;
    for (int r = 0; r < n_k; ++r) z_k += exp(l[ord[r]] - m);

    /* top-p over the renormalised S_k, walking groups of equal logits */
    int n_s = n_k;
    if (top_p > 0.0 && top_p < 1.0) {
        const double target = top_p * z_k;
        double above = 0.0; /* mass of S_k strictly above the current group */
        int r = 0;
        n_s = 0;
        while (r < n_k) {
            int e = r;
            double group = 0.0;
            while (e < n_k && l[ord[e]] == l[ord[r]]) group += exp(l[ord[e++]] - m);
            if (!(above < target)) {
                margin = fmin(margin, (above - target) / z_k);
                break;
            }
            margin = fmin(margin, (target - above) / z_k);
            n_s = e;
            above += group;
            r = e;
        }
    }
    double z = 0.0;
    for (int r = 0; r < n_s; ++r) z += exp(l[ord[r]] - m);
    for (int v = 0; v < n; ++v) p_out[v] = 0.0;
    for (int r = 0; r < n_s; ++r) p_out[ord[r]] = exp(l[ord[r]] - m) / z;
    if (logz_out) *logz_out = m + log(z);
    if (margin_out) *margin_out = margin;
    free(ord);
    return n_s;
}

/* ------------------------------------------------------------------------ */
/* The three acceptance rules, each on already-reduced quantities.           */
/* ------------------------------------------------------------------------ */

/* [DM] Eq. (4): keep the draft token x iff it equals one of the K head tokens. */
int dmo_rule_naive(const int32_t* head_tokens, int K, int32_t x)
{
    for (int i = 0; i < K; ++i)
        if (head_tokens[i] == x) return 1;
    return 0;
}

/* [DM] Algorithm 1: accept when the draft's divergence to the centroid is no
 * larger than the largest head divergence (Eq. (6), equality accepts), else
 * when x is the majority head token (Eq. (7); reading: strict majority, more
 * than K/2 of the heads), else reject. */
int dmo_rule_js(double js_draft, double js_max, const int32_t* head_tokens, int K, int32_t x)
{
    if (js_draft <= js_max) return 1;
    int count = 0;
    for (int i = 0; i < K; ++i)
        if (head_tokens[i] == x) ++count;
    return 2 * count > K;
}

/* [PB] Sec. 2 and the verify-round pseudocode of Sec. 5: keep x with
 * probability min(1, p(x)/q(x)), decided as u < p(x)/q(x) for a uniform u in
 * [0, 1), evaluated without division as u * q(x) < p(x) (so q(x) = 0 keeps x
 * iff p(x) > 0). */
int dmo_rule_lossless(double u, double px, double qx)
{
    return u * qx < px;
}

/* [TR] with [DM] Sec. 4.4: the round on a token tree.  Node t+1 holds draft
 * t and hangs below position parent[t] (0 = the root); flags[t] is the rule's
 * decision for draft t at its parent.  A node is on an accepted path iff it
 * passed and so did every node between it and the root; the round commits
 * the deepest such path (reading: on equal depths the node that comes first,
 * the smallest index), then the target's token at its last node.  A parent
 * outside [0, t] puts the node off every path.  Returns the depth (drafts
 * committed) and writes the last node's position (0 = the root) to *pos. */
int dmo_tree_walk(const int32_t* parent, const uint8_t* flags, int G, int32_t* pos)
{
    int32_t* depth = (int32_t*)malloc(sizeof(int32_t) * (size_t)(G + 1));
    uint8_t* on_path = (uint8_t*)malloc((size_t)(G + 1));
    if (!depth || !on_path) {
        free(depth);
        free(on_path);
        return -1;
    }
    depth[0] = 0;
    on_path[0] = 1; /* the root is committed already */
    int best = 0, best_pos = 0;
    for (int t = 0; t < G; ++t) {
        const int node = t + 1, up = parent[t];
        if (up < 0 || up > t) {
            depth[node] = 0;
            on_path[node] = 0;
            continue;
        }
        depth[node] = depth[up] + 1;
        on_path[node] = flags[t] && on_path[up];
        if (on_path[node] && depth[node] > best) {
            best = depth[node];
            best_pos = node;
        }
    }
    free(depth);
    free(on_path);
    *pos = best_pos;
    return best;
}

/* ------------------------------------------------------------------------ */
/* Problem / result records (this library's own layout).                     */
/* ------------------------------------------------------------------------ */
typedef struct dmo_problem {
    int32_t d, vocab, batch, gamma, K;
    int32_t dtype; /* 0: float32, 1: bfloat16 bits */
    float p_drop;
    uint32_t pad0;
    uint64_t seed;
    const void* W;         /* [vocab, d] */
    const void* h;         /* [batch, gamma+1, d] */
    const int32_t* draft;  /* [batch, gamma] */
    const float* q_hat;    /* [batch, gamma, vocab] or NULL */
    const uint8_t* modes;  /* [batch] */
    int32_t n_seq;         /* number of sequences evaluated */
    int32_t n_threads;
    const int32_t* seq;    /* [n_seq] batch indices evaluated */
    float temperature;     /* > 0 divides every logit row; 0 is read as 1 */
    int32_t top_k;         /* lossless rows; 0 = off */
    float top_p;           /* lossless rows; 0 or >= 1 = off */
    uint32_t pad1;
    /* Ragged batches (NULL = every sequence uses gamma, K, p_drop): sequence
     * b drafts seq_gamma[b] <= gamma tokens (positions 0..seq_gamma[b]),
     * lossy sequences use seq_K[b] <= K heads and dropout seq_p_drop[b]. */
    const int32_t* seq_gamma;
    const int32_t* seq_K;
    const float* seq_p_drop;
    /* Token trees (NULL = every sequence is a chain): for a DMO_TREE_NAIVE
     * sequence, draft t is node t+1 and tree_parent[b, t] in [0, t] is the
     * position whose hidden state predicts it (0 = the root, the last
     * committed token); h[b, t+1] is the state after the root-to-node path.
     * A chain is tree_parent[b, t] = t. */
    const int32_t* tree_parent;
} dmo_problem;

typedef struct dmo_result { /* leading dimension n_seq everywhere; NULL = not wanted */
    int32_t* accept_len;      /* [n] */
    int32_t* out_token;       /* [n] */
    uint8_t* accept_flags;    /* [n, gamma] */
    double* margin;           /* [n, gamma] */
    double* uniforms;         /* [n, gamma] lossless acceptance uniforms */
    int32_t* head_argmax;     /* [n, gamma+1, K] (-1 for unused heads) */
    double* head_gap;         /* [n, gamma+1, K] */
    double* head_max;         /* [n, gamma+1, K] */
    double* head_logz;        /* [n, gamma+1, K] */
    int32_t* centroid_argmax; /* [n, gamma+1] */
    double* centroid_gap;     /* [n, gamma+1] */
    double* centroid_logz;    /* [n, gamma+1] */
    double* js_heads;         /* [n, gamma, K] */
    double* js_draft;         /* [n, gamma] */
    double* logits;           /* [n, gamma+1, K, vocab] */
    uint32_t* mask_bits;      /* [n, gamma+1, K, d/32] */
    double* race_gap;         /* [n] */
    int32_t* filter_count;    /* [n, gamma+1] lossless sequences: |S| of the processed target */
    double* filter_logz;      /* [n, gamma+1] lossless sequences: log sum over S of e^l */
    double* filter_margin;    /* [n, gamma+1] lossless sequences: see dmo_processed */
    int32_t* accept_pos;      /* [n] position of the last kept node (chains: accept_len) */
    uint32_t* data_status;    /* [n] bit 0: a draft id outside [0, vocab); bit 1: a tree parent
                                 outside [0, t] (each such draft counts as rejected) */
} dmo_result;

/* ------------------------------------------------------------------------ */
/* One verify step for the listed sequences.                                 */
/* ------------------------------------------------------------------------ */
int dmo_run(const dmo_problem* P, const dmo_result* R)
{
    const int d = P->d, V = P->vocab, G = P->gamma, K = P->K, T1 = G + 1;
    if (d <= 0 || V <= 0 || G < 0 || K <= 0 || P->batch <= 0) return 1;
    if (!(P->p_drop >= 0.0f && P->p_drop < 1.0f)) return 1;
    if (!(P->temperature >= 0.0f) || !(P->top_p >= 0.0f) || P->top_k < 0) return 1;
    /* temperature: the sampled distribution is softmax(l / T) ([PB] Sec. 1) */
    const double temp = P->temperature > 0.0f ? (double)P->temperature : 1.0;
    const int nthreads = P->n_threads > 0 ? P->n_threads : 1;

    double* hm = (double*)malloc(sizeof(double) * (size_t)T1 * K * d);
    double* L = (double*)malloc(sizeof(double) * (size_t)T1 * K * V);
    double* Lbar = (double*)malloc(sizeof(double) * (size_t)T1 * V);
    double* prob = (double*)malloc(sizeof(double) * (size_t)(K + 2) * V);
    double* pproc = (double*)malloc(sizeof(double) * (size_t)T1 * V); /* lossless: processed p per position */
    if (!hm || !L || !Lbar || !prob || !pproc) {
        free(hm); free(L); free(Lbar); free(prob); free(pproc);
        return 4;
    }
    double* rmax = (double*)malloc(sizeof(double) * (size_t)T1 * K);
    double* rlogz = (double*)malloc(sizeof(double) * (size_t)T1 * K);
    double* rgap = (double*)malloc(sizeof(double) * (size_t)T1 * K);
    int32_t* rarg = (int32_t*)malloc(sizeof(int32_t) * (size_t)T1 * K);
    double* clogz = (double*)malloc(sizeof(double) * (size_t)T1);
    double* cgap = (double*)malloc(sizeof(double) * (size_t)T1);
    int32_t* carg = (int32_t*)malloc(sizeof(int32_t) * (size_t)T1);
    uint8_t* acc = (uint8_t*)malloc((size_t)(G > 0 ? G : 1));

    for (int n = 0; n < P->n_seq; ++n) {
        const int b = P->seq ? P->seq[n] : n;
        const int mode = P->modes[b];
        const int lossy = mode != DMO_LOSSLESS;
        if (mode > DMO_TREE_NAIVE || (mode == DMO_TREE_NAIVE && G > 0 && !P->tree_parent)) {
            free(hm); free(L); free(Lbar); free(prob); free(pproc);
            free(rmax); free(rlogz); free(rgap); free(rarg); free(clogz); free(cgap); free(carg); free(acc);
            return 1;
        }
        /* This sequence's drafts, heads and dropout (a ragged batch, [SD]
         * "Production gotchas", "Batching": sequences keep different numbers
         * of drafts).  Layout strides stay the batch's gamma and K; the Philox
         * counters keep pidx = b * (gamma + 1) + t. */
        const int Gb = P->seq_gamma ? P->seq_gamma[b] : G, Tb = Gb + 1;
        const int Kb = P->seq_K ? P->seq_K[b] : K;
        const float pb = P->seq_p_drop ? P->seq_p_drop[b] : P->p_drop;
        if (Gb < 0 || Gb > G || Kb < 1 || Kb > K || !(pb >= 0.0f && pb < 1.0f)) {
            free(hm); free(L); free(Lbar); free(prob); free(pproc);
            free(rmax); free(rlogz); free(rgap); free(rarg); free(clogz); free(cgap); free(carg); free(acc);
            return 1;
        }
        const uint32_t thresh = dmo_threshold(pb);
        /* Lossless sequences verify with the undropped target head, one row
         * per position (reading: the classical test of [SD] / [PB] Sec. 2 is
         * defined for the target's own p). */
        const int rows = lossy ? Kb : 1;
        /* Inverted-dropout scale 1 / (1 - p_drop), [DM] Eq. (2). */
        const double scale = lossy ? 1.0 / (1.0 - (double)pb) : 1.0;

        /* [DM] Eq. (1)-(2): masked hidden state per (position, head). */
        for (int t = 0; t < Tb; ++t) {
            const uint32_t pidx = (uint32_t)(b * T1 + t);
            for (int i = 0; i < rows; ++i) {
                double* dst = hm + ((size_t)t * K + i) * d;
                for (int j = 0; j < d; ++j) {
                    double hv = decode(P->h, P->dtype, ((size_t)b * T1 + t) * d + j);
                    int keep = lossy ? keep_bit(P->seed, pidx, (uint32_t)i, (uint32_t)j, thresh) : 1;
                    dst[j] = keep ? hv : 0.0;
                    if (R->mask_bits && keep) {
                        size_t w = (((size_t)n * T1 + t) * K + i) * (size_t)(d / 32) + (size_t)(j / 32);
                        R->mask_bits[w] |= 1u << (j & 31);
                    }
                }
            }
        }

        /* [DM] Eq. (3): l^(i) = W h^(i) with the shared W, scaled. */
#pragma omp parallel num_threads(nthreads)
        {
            double* wrow = (double*)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(static)
            for (int v = 0; v < V; ++v) {
                for (int j = 0; j < d; ++j) wrow[j] = decode(P->W, P->dtype, (size_t)v * d + j);
                for (int t = 0; t < Tb; ++t) {
                    for (int i = 0; i < rows; ++i) {
                        const double* x = hm + ((size_t)t * K + i) * d;
                        double s = 0.0;
                        for (int j = 0; j < d; ++j) s += wrow[j] * x[j];
                        L[((size_t)t * K + i) * V + v] = scale * s / temp;
                    }
                }
            }
            free(wrow);
        }

        /* Per-head statistics; centroid l-bar = mean of head logits, [DM] Eq. (5). */
        for (int t = 0; t < Tb; ++t) {
            for (int i = 0; i < rows; ++i) {
                const double* l = L + ((size_t)t * K + i) * V;
                dmo_row_stats(l, V, &rmax[t * K + i], &rlogz[t * K + i], &rarg[t * K + i], &rgap[t * K + i]);
            }
            double* lb = Lbar + (size_t)t * V;
            for (int v = 0; v < V; ++v) {
                double s = 0.0;
                for (int i = 0; i < rows; ++i) s += L[((size_t)t * K + i) * V + v];
                lb[v] = s / rows;
            }
            dmo_row_stats(lb, V, NULL, &clogz[t], &carg[t], &cgap[t]);
        }

        /* Lossless sequences: the processed target at every position. */
        if (!lossy) {
            for (int t = 0; t < Tb; ++t) {
                double lz, mg;
                int cnt = dmo_processed(L + ((size_t)t * K) * V, V, P->top_k, (double)P->top_p,
                                        pproc + (size_t)t * V, &lz, &mg);
                if (cnt < 0) {
                    free(hm); free(L); free(Lbar); free(prob); free(pproc);
                    free(rmax); free(rlogz); free(rgap); free(rarg); free(clogz); free(cgap); free(carg); free(acc);
                    return 4;
                }
                if (R->filter_count) R->filter_count[(size_t)n * T1 + t] = cnt;
                if (R->filter_logz) R->filter_logz[(size_t)n * T1 + t] = lz;
                if (R->filter_margin) R->filter_margin[(size_t)n * T1 + t] = mg;
            }
        }

        /* Decisions for every drafted position t < gamma_b. */
        uint32_t status = 0;
        for (int t = 0; t < Gb; ++t) {
            const int32_t x = P->draft[(size_t)b * G + t];
            const uint32_t pidx = (uint32_t)(b * T1 + t);
            const int valid = x >= 0 && x < V;
            if (!valid) status |= 1u;
            int accept = 0;
            double margin = INFINITY;
            double min_gap = INFINITY;
            for (int i = 0; i < rows; ++i)
                if (rgap[t * K + i] < min_gap) min_gap = rgap[t * K + i];
            if (mode == DMO_NAIVE) {
                accept = valid && dmo_rule_naive(rarg + t * K, rows, x);
                margin = min_gap;
            } else if (mode == DMO_TREE_NAIVE) {
                /* [TR]: draft t is judged by the heads at its parent position */
                const int32_t up = P->tree_parent[(size_t)b * G + t];
                if (!(up >= 0 && up <= t)) status |= 2u;
                if (up >= 0 && up <= t) {
                    accept = valid && dmo_rule_naive(rarg + up * K, rows, x);
                    margin = INFINITY;
                    for (int i = 0; i < rows; ++i)
                        if (rgap[up * K + i] < margin) margin = rgap[up * K + i];
                }
            } else if (mode == DMO_JS) {
                /* [DM] Algorithm 1: centroid p-bar, head and draft divergences. */
                double* pc = prob;                 /* centroid p-bar */
                double* ph = prob + V;             /* one head at a time */
                double* pq = prob + 2 * (size_t)V; /* draft q-hat */
                for (int v = 0; v < V; ++v) pc[v] = exp(Lbar[(size_t)t * V + v] - clogz[t]);
                double jmax = -INFINITY;
                for (int i = 0; i < rows; ++i) {
                    const double* l = L + ((size_t)t * K + i) * V;
                    for (int v = 0; v < V; ++v) ph[v] = exp(l[v] - rlogz[t * K + i]);
                    double ji = dmo_js(ph, pc, V);
                    if (R->js_heads) R->js_heads[((size_t)n * G + t) * K + i] = ji;
                    if (ji > jmax) jmax = ji;
                }
                const float* q = P->q_hat + ((size_t)b * G + t) * V;
                for (int v = 0; v < V; ++v) pq[v] = (double)q[v];
                double jq = dmo_js(pq, pc, V);
                if (R->js_draft) R->js_draft[(size_t)n * G + t] = jq;
                accept = valid && dmo_rule_js(jq, jmax, rarg + t * K, rows, x);
                /* margins of the two branches, for the near-tie accounting */
                int acc_js = valid && (jq <= jmax);
                int acc_maj = valid && dmo_rule_js(1.0, 0.0, rarg + t * K, rows, x);
                double m_js = fabs(jq - jmax);
                if (accept)
                    margin = fmax(acc_js ? m_js : 0.0, acc_maj ? min_gap : 0.0);
                else
                    margin = fmin(m_js, min_gap);
            } else {
                /* [PB] Sec. 2: the classical test on the undropped, processed
                 * target p. */
                double u = dmo_accept_uniform(P->seed, pidx);
                if (R->uniforms) R->uniforms[(size_t)n * G + t] = u;
                if (valid) {
                    double px = pproc[(size_t)t * V + x];
                    double qx = (double)P->q_hat[((size_t)b * G + t) * V + x];
                    accept = dmo_rule_lossless(u, px, qx);
                    margin = qx > 0.0 ? fabs(u - px / qx) : px;
                }
            }
            if (!valid) margin = INFINITY;
            acc[t] = (uint8_t)accept;
            if (R->accept_flags) R->accept_flags[(size_t)n * G + t] = (uint8_t)accept;
            if (R->margin) R->margin[(size_t)n * G + t] = margin;
        }

        /* [SD] "The draft-then-verify loop" step 3 / [PB] Sec. 5: scan left to
         * right, the first rejection ends the round.  A tree keeps its
         * deepest accepted path instead, and emits at that path's end. */
        int A = Gb;
        int32_t pos = Gb;
        if (mode == DMO_TREE_NAIVE) {
            A = dmo_tree_walk(P->tree_parent + (size_t)b * G, acc, Gb, &pos);
            if (A < 0) {
                free(hm); free(L); free(Lbar); free(prob); free(pproc);
                free(rmax); free(rlogz); free(rgap); free(rarg); free(clogz); free(cgap); free(carg); free(acc);
                return 4;
            }
        } else {
            for (int t = 0; t < Gb; ++t)
                if (!acc[t]) {
                    A = t;
                    break;
                }
            pos = A;
        }

        /* Emit one target token. */
        int32_t y;
        double race_gap = INFINITY;
        if (lossy) {
            /* Reading: the lossy rules are greedy, so the target's own token
             * is the centroid argmax at row A ([SD] "Greedy decoding"); on a
             * tree, at the last node of the kept path. */
            y = carg[pos];
        } else {
            /* [PB] Sec. 5: residual normalize((p_A - q_A)+) after a rejection,
             * the bonus p_gamma when every draft survived; a zero residual
             * (only possible by rounding) falls back to p_A ([PB] Sec. 2). */
            double* w = prob;
            const double* pa = pproc + (size_t)A * V;
            double total = 0.0;
            for (int v = 0; v < V; ++v) {
                double p = pa[v];
                if (A < Gb) {
                    double q = (double)P->q_hat[((size_t)b * G + A) * V + v];
                    w[v] = p - q > 0.0 ? p - q : 0.0;
                } else {
                    w[v] = p;
                }
                total += w[v];
            }
            if (!(total > 0.0))
                for (int v = 0; v < V; ++v) w[v] = pa[v];
            y = dmo_race(w, V, P->seed, (uint32_t)(b * T1 + A), &race_gap);
        }

        if (R->accept_len) R->accept_len[n] = A;
        if (R->accept_pos) R->accept_pos[n] = pos;
        if (R->data_status) R->data_status[n] = status;
        if (R->out_token) R->out_token[n] = y;
        if (R->race_gap) R->race_gap[n] = race_gap;
        for (int t = 0; t < T1; ++t) {
            for (int i = 0; i < K; ++i) {
                size_t o = ((size_t)n * T1 + t) * K + i;
                int used = i < rows && t < Tb;
                if (R->head_argmax) R->head_argmax[o] = used ? rarg[t * K + i] : -1;
                if (R->head_gap) R->head_gap[o] = used ? rgap[t * K + i] : NAN;
                if (R->head_max) R->head_max[o] = used ? rmax[t * K + i] : NAN;
                if (R->head_logz) R->head_logz[o] = used ? rlogz[t * K + i] : NAN;
                if (R->logits && used)
                    memcpy(R->logits + o * V, L + ((size_t)t * K + i) * V, sizeof(double) * V);
            }
            if (R->centroid_argmax) R->centroid_argmax[(size_t)n * T1 + t] = t < Tb ? carg[t] : -1;
            if (R->centroid_gap) R->centroid_gap[(size_t)n * T1 + t] = t < Tb ? cgap[t] : NAN;
            if (R->centroid_logz) R->centroid_logz[(size_t)n * T1 + t] = t < Tb ? clogz[t] : NAN;
        }
    }

    free(hm); free(L); free(Lbar); free(prob); free(pproc);
    free(rmax); free(rlogz); free(rgap); free(rarg);
    free(clogz); free(cgap); free(carg); free(acc);
    return 0;
}
