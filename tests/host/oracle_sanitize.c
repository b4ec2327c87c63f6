/* The fp64 oracle under AddressSanitizer and UndefinedBehaviorSanitizer (a
 * CPU test): one verify step per setting with every output requested, each
 * buffer allocated at exactly the size the oracle's interface gives, so an
 * access past one is reported.  Settings cover every rule, fp32 and bf16,
 * a vocabulary that is no multiple of 4 or 16, out-of-range drafts, an
 * invalid tree parent, ragged sequences, temperature, top-k and top-p. */
#include "../../oracle/dm_oracle.c"

#include <stdio.h>
#include <string.h>

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double urand(void) { /* splitmix64, then the top 53 bits */
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return (double)(z >> 11) * (1.0 / 9007199254740992.0);
}
static uint16_t to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

static int run_case(int dtype, int d, int V, int B, int G, int K, float p, float temp, int top_k, float top_p,
                    int ragged) {
    const int T1 = G + 1;
    const size_t esz = dtype ? 2 : 4;
    void* W = malloc((size_t)V * d * esz);
    void* h = malloc((size_t)B * T1 * d * esz);
    for (size_t i = 0; i < (size_t)V * d; ++i) {
        const float x = (float)((urand() - 0.5) * 0.2);
        if (dtype) ((uint16_t*)W)[i] = to_bf16(x); else ((float*)W)[i] = x;
    }
    for (size_t i = 0; i < (size_t)B * T1 * d; ++i) {
        const float x = (float)(urand() * 2.0 - 1.0);
        if (dtype) ((uint16_t*)h)[i] = to_bf16(x); else ((float*)h)[i] = x;
    }
    int32_t* draft = malloc(sizeof(int32_t) * B * G);
    float* q = malloc(sizeof(float) * (size_t)B * G * V);
    uint8_t* modes = malloc(B);
    int32_t* seq = malloc(sizeof(int32_t) * B);
    int32_t* parent = malloc(sizeof(int32_t) * B * G);
    int32_t* sg = malloc(sizeof(int32_t) * B);
    int32_t* sk = malloc(sizeof(int32_t) * B);
    float* sp = malloc(sizeof(float) * B);
    for (int b = 0; b < B; ++b) {
        modes[b] = (uint8_t)(b % 4); /* lossless, naive, JS+majority, tree */
        seq[b] = b;
        sg[b] = G - (b % (G + 1));
        sk[b] = 1 + b % K;
        sp[b] = (float)(0.1 * (b % 3));
        for (int t = 0; t < G; ++t) {
            draft[b * G + t] = (int32_t)(urand() * V);
            parent[b * G + t] = (int32_t)(urand() * (t + 1));
            double s = 0.0;
            for (int v = 0; v < V; ++v) s += (q[((size_t)b * G + t) * V + v] = (float)urand());
            for (int v = 0; v < V; ++v) q[((size_t)b * G + t) * V + v] = (float)(q[((size_t)b * G + t) * V + v] / s);
        }
    }
    if (G > 0) draft[0] = -1; /* out of range: rejected, status bit 0 */
    if (B > 1 && G > 1) draft[G + 1] = V + 3;
    if (B > 3 && G > 2) parent[3 * G + 2] = 3; /* a parent past its node: rejected, status bit 1 */

    dmo_problem P;
    memset(&P, 0, sizeof(P));
    P.d = d; P.vocab = V; P.batch = B; P.gamma = G; P.K = K; P.dtype = dtype; P.p_drop = p;
    P.seed = 0x1234567890ull; P.W = W; P.h = h; P.draft = draft; P.q_hat = q; P.modes = modes;
    P.n_seq = B; P.n_threads = 2; P.seq = seq; P.temperature = temp; P.top_k = top_k; P.top_p = top_p;
    P.tree_parent = parent;
    if (ragged) { P.seq_gamma = sg; P.seq_K = sk; P.seq_p_drop = sp; }

    const size_t n = B;
    dmo_result R;
    R.accept_len = malloc(sizeof(int32_t) * n);
    R.out_token = malloc(sizeof(int32_t) * n);
    R.accept_flags = malloc(n * G);
    R.margin = malloc(sizeof(double) * n * G);
    R.uniforms = malloc(sizeof(double) * n * G);
    R.head_argmax = malloc(sizeof(int32_t) * n * T1 * K);
    R.head_gap = malloc(sizeof(double) * n * T1 * K);
    R.head_max = malloc(sizeof(double) * n * T1 * K);
    R.head_logz = malloc(sizeof(double) * n * T1 * K);
    R.centroid_argmax = malloc(sizeof(int32_t) * n * T1);
    R.centroid_gap = malloc(sizeof(double) * n * T1);
    R.centroid_logz = malloc(sizeof(double) * n * T1);
    R.js_heads = malloc(sizeof(double) * n * G * K);
    R.js_draft = malloc(sizeof(double) * n * G);
    R.logits = malloc(sizeof(double) * n * T1 * K * V);
    R.mask_bits = d % 32 == 0 ? malloc(sizeof(uint32_t) * n * T1 * K * (d / 32)) : NULL;
    R.race_gap = malloc(sizeof(double) * n);
    R.filter_count = malloc(sizeof(int32_t) * n * T1);
    R.filter_logz = malloc(sizeof(double) * n * T1);
    R.filter_margin = malloc(sizeof(double) * n * T1);
    R.accept_pos = malloc(sizeof(int32_t) * n);
    R.data_status = malloc(sizeof(uint32_t) * n);

    const int rc = dmo_run(&P, &R);
    int bad = rc != 0;
    for (int b = 0; b < B; ++b) {
        const int gb = ragged ? sg[b] : G;
        if (R.accept_len[b] < 0 || R.accept_len[b] > gb) bad = 1;
        if (R.out_token[b] < 0 || R.out_token[b] >= V) bad = 1;
    }
    if (G > 0 && !(R.data_status[0] & 1u)) bad = 1;

    void* ptrs[] = {W, h, draft, q, modes, seq, parent, sg, sk, sp, R.accept_len, R.out_token, R.accept_flags,
                    R.margin, R.uniforms, R.head_argmax, R.head_gap, R.head_max, R.head_logz, R.centroid_argmax,
                    R.centroid_gap, R.centroid_logz, R.js_heads, R.js_draft, R.logits, R.mask_bits, R.race_gap,
                    R.filter_count, R.filter_logz, R.filter_margin, R.accept_pos, R.data_status};
    for (size_t i = 0; i < sizeof(ptrs) / sizeof(ptrs[0]); ++i) free(ptrs[i]);
    return bad;
}

int main(void) {
    int runs = 0, failures = 0;
    /* dtype, d, V, B, gamma, K, p, temperature, top_k, top_p, ragged */
    failures += run_case(0, 64, 70, 8, 4, 3, 0.2f, 1.0f, 0, 1.0f, 0); ++runs;
    failures += run_case(1, 96, 37, 8, 5, 5, 0.3f, 0.7f, 5, 0.9f, 0); ++runs;
    failures += run_case(1, 64, 131, 9, 6, 4, 0.25f, 1.3f, 0, 0.8f, 1); ++runs;
    failures += run_case(0, 40, 9, 5, 0, 2, 0.0f, 1.0f, 1, 1.0f, 0); ++runs;
    failures += run_case(0, 32, 1, 4, 3, 1, 0.5f, 1.0f, 0, 1.0f, 1); ++runs;
    printf("%d runs, %d failures\n", runs, failures);
    return failures != 0;
}
