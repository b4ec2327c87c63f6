/*
 * dm_verify.h -- C ABI of the DropMatch verify-step library (libdmverify.so),
 * hand-written HIP kernels for MI355X (gfx950).
 *
 * One call verifies the gamma drafted tokens of each of B sequences.  For each
 * of the gamma+1 positions t of sequence b it runs the LM head on the target's
 * last hidden state h[b, t, :], then applies that sequence's acceptance rule,
 * scans the drafts left to right and emits one target token.
 *
 * What the call computes (sources: "Training-free Dropout Sampling for
 * Semantic Token Acceptance in Speculative Decoding" (DropMatch), Sec. 3.1
 * Eq. (1)-(3) and Sec. 3.2 Eq. (4)-(7), Algorithm 1; "Speculative Decoding:
 * Draft, Then Verify", sections "The draft-then-verify loop", "The acceptance
 * rule", "Greedy decoding"; "Why speculative decoding preserves distributions
 * but may not be faster", Sec. 2 and the verify-round pseudocode of Sec. 5):
 *
 *   Lossy sequences (DM_MODE_NAIVE, DM_MODE_JS_MAJORITY, DM_MODE_TREE_NAIVE),
 *   each position t:
 *     keep[i, j] = Philox word (j/4, b*(gamma+1)+t, i, 0)[j%4] >= T,
 *                  T = min(floor(p_drop * 2^32 + 1/2), 2^32 - 1)  (Eq. (1))
 *     l^(i)[v]  = s * sum_j W[v, j] * h[b, t, j] * keep[i, j],
 *                 s = 1 / (1 - p_drop), i = 0..K-1             (Eq. (2)-(3))
 *     y^(i)     = argmax_v l^(i)[v] (smallest v on ties)
 *     l-bar     = (1/K) sum_i l^(i); p-bar = softmax(l-bar)      (Eq. (5))
 *   NAIVE:   accept draft x_t iff x_t is one of the y^(i)          (Eq. (4))
 *   JS:      accept iff JS(q_hat_t || p-bar) <= max_i JS(p^(i) || p-bar)
 *            (natural log, Eq. (6)), else iff more than K/2 heads give x_t
 *            (Eq. (7)), else reject                         (Algorithm 1)
 *   Emitted token: argmax of p-bar at the first rejected position A
 *            (A = gamma when all drafts pass).
 *
 *   Token trees (DM_MODE_TREE_NAIVE; "Speculative Decoding: Draft, Then
 *     Verify", "Variants": one target pass verifies a tree of candidate
 *     continuations under a tree-shaped attention mask; DropMatch Sec. 4.4:
 *     on EAGLE3's trees the naive rule is the one applied).  Draft t is node
 *     t+1 of the tree and hangs below position tree_parent[b, t] in [0, t]
 *     (0 = the root); h[b, t+1] is the target's state after the path from
 *     the root to that node, so a chain is tree_parent[b, t] = t.  Every
 *     position runs the K dropout heads as above.  Draft t passes iff it is
 *     one of the y^(i) at its parent position (Eq. (4)); a node is on a kept
 *     path iff it and every node above it pass.  The round keeps the deepest
 *     such path (on equal depths the node with the smallest index): A is its
 *     depth, the emitted token the argmax of p-bar at its last node.  A
 *     parent outside [0, t] rejects the draft and so every node below it.
 *
 *   Lossless sequences (DM_MODE_LOSSLESS): one undropped row per position,
 *     p_t = softmax(W h[b, t]).  With u_t = (Philox word (0, b*(gamma+1)+t,
 *     0, 1)[0] >> 8) * 2^-24, accept x_t iff u_t * q_hat_t(x_t) < p_t(x_t)
 *     (the min(1, p/q) test).  After a rejection at A the emitted token is
 *     drawn from (p_A - q_hat_A)+ (p_A if that is zero everywhere); when all
 *     pass, from p_gamma.  The draw is an exponential race: the winner
 *     maximises w_v / (-ln U_v), U_v = ((Philox word (v/4, b*(gamma+1)+A, 0,
 *     2)[v%4] >> 9) + 1/2) * 2^-23, ties to the smallest v.
 *
 *   Philox is Philox4x32-10 (Salmon et al., SC'11) keyed by the 64-bit seed
 *   (low word first).  A draft id outside [0, vocab) is rejected, and so is
 *   a draft whose tree parent is out of range; data_status reports both.
 *
 * Precision: bf16 (or fp32) inputs, fp32 accumulation and statistics.
 *
 * Memory: every pointer in dm_verify_args is DEVICE memory owned by the
 * caller, except `modes`, which is HOST memory (the host needs the mode mix to
 * lay out the LM-head rows).  The handle owns only its device workspace.
 *
 * Streams: dm_verify_run only enqueues work on `stream` (a hipStream_t; NULL
 * means the null stream) and returns; outputs are valid once the stream has
 * been synchronised.  One run may be in flight per handle at a time.
 *
 * Errors: every function returns a dm_status.  Argument checks happen on the
 * host before any HIP call; a HIP failure maps to DM_ERR_HIP.
 */
#ifndef DM_VERIFY_H
#define DM_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dm_status {
    DM_OK = 0,
    DM_ERR_INVALID_ARGUMENT = 1, /* NULL where required, value out of range */
    DM_ERR_UNSUPPORTED = 2,      /* valid but not handled: dtype, d % 64, alignment */
    DM_ERR_HIP = 3,              /* a HIP runtime call or a launch failed */
    DM_ERR_OUT_OF_MEMORY = 4,    /* workspace allocation failed */
    DM_ERR_TOO_LARGE = 5         /* dm_verify_run_static: the call needs more than the scratch array */
} dm_status;

typedef enum dm_dtype { DM_DTYPE_F32 = 0, DM_DTYPE_BF16 = 1 } dm_dtype;

/* Storage order of the LM-head weight W passed to dm_verify_run. */
typedef enum dm_w_layout {
    DM_W_ROW_MAJOR = 0, /* [vocab, d] row-major */
    DM_W_PANELS = 1     /* the panel order written by dm_verify_pack_w (below) */
} dm_w_layout;

typedef enum dm_mode {
    DM_MODE_LOSSLESS = 0,    /* classical min(1, p/q) test, (p - q)+ residual */
    DM_MODE_NAIVE = 1,       /* DropMatch naive token matching, Eq. (4) */
    DM_MODE_JS_MAJORITY = 2, /* DropMatch Algorithm 1, Eq. (6) then Eq. (7) */
    DM_MODE_TREE_NAIVE = 3   /* Eq. (4) on a token tree (tree_parent below) */
} dm_mode;

/* Problem limits fixed at handle creation. */
typedef struct dm_verify_desc {
    int32_t d;         /* hidden size; multiple of 64, 64..65536 */
    int32_t vocab;     /* |V|, 1..524288 */
    int32_t max_batch; /* largest B a run may pass, 1..256 */
    int32_t gamma;     /* drafted tokens (tree nodes) per sequence, 0..63 (gamma+1 positions) */
    int32_t k_max;     /* largest K a run may pass, 1..16 */
    int32_t dtype;     /* dm_dtype of W and h */
} dm_verify_desc;

/* One verify step.  Shapes use the desc's d, vocab, gamma and this B, K. */
typedef struct dm_verify_args {
    const void* W;          /* device LM-head weight, dtype, stored as w_layout says; 16-byte aligned */
    const void* h;          /* device [B, gamma+1, d] row-major, dtype; 16-byte aligned */
    const int32_t* draft;   /* device [B, gamma] drafted token ids (may be NULL iff gamma == 0) */
    const float* q_hat;     /* device [B, gamma, vocab] draft distributions, used as given;
                               required iff a sequence is LOSSLESS or JS_MAJORITY */
    const uint8_t* modes;   /* HOST [B] dm_mode per sequence */
    int32_t batch;          /* B, 1..max_batch */
    int32_t K;              /* dropout heads for lossy sequences, 1..k_max */
    float p_drop;           /* dropout probability, 0 <= p_drop < 1 */
    uint32_t w_layout;      /* dm_w_layout of W */
    uint64_t seed;          /* Philox key */
    /* Sampling settings of the target.  The lossless test and its residual
     * must use the distribution the sampler actually draws from: temperature,
     * top-k, top-p and the renormalisation ("Why speculative decoding
     * preserves distributions but may not be faster", Sec. 1; "Speculative
     * Decoding: Draft, Then Verify", "The same sampling settings").  q_hat is
     * the draft's processed distribution, used as given.  All three zero =
     * the plain softmax. */
    float temperature;      /* > 0 divides every logit row, all rules; 0 is read as 1 */
    int32_t top_k;          /* LOSSLESS: keep the tokens whose logit is >= the top_k-th largest
                               (ties kept); 0 or >= vocab = off */
    float top_p;            /* LOSSLESS: of those, keep the tokens whose strictly larger
                               renormalised mass is < top_p; 0 or >= 1 = off */
    uint32_t reserved;      /* 0 */
    /* Ragged batches ("Speculative Decoding: Draft, Then Verify", "Production
     * gotchas", "Batching": sequences keep different numbers of drafts).  HOST
     * arrays of B entries, each NULL = every sequence uses gamma, K, p_drop.
     * Sequence b verifies positions 0..seq_gamma[b] (its drafts are
     * draft[b, 0..seq_gamma[b]-1], the rest of its rows unread); a lossy
     * sequence uses seq_heads[b] of the K heads and dropout seq_p_drop[b].
     * The layout strides stay gamma and K, and the Philox counters keep
     * pidx = b * (gamma + 1) + t.  At most 8 distinct seq_p_drop values per
     * call (else DM_ERR_UNSUPPORTED).  Outputs past a sequence's drafts or
     * heads are not written (accept_len[b] <= seq_gamma[b]). */
    const int32_t* seq_gamma;  /* 0 <= seq_gamma[b] <= gamma */
    const int32_t* seq_heads;  /* 1 <= seq_heads[b] <= K */
    const float* seq_p_drop;   /* 0 <= seq_p_drop[b] < 1 */
    /* Token trees: device [B, gamma], the parent position of every draft of
     * the TREE_NAIVE sequences (rows of other sequences are not read).
     * Required iff a sequence is TREE_NAIVE and gamma > 0; with seq_gamma,
     * only the first seq_gamma[b] entries of row b are read. */
    const int32_t* tree_parent;
    int32_t* accept_len;    /* device out [B]: A, drafts accepted (on a tree: depth of the kept path) */
    int32_t* out_token;     /* device out [B]: correction (A < gamma) or bonus (A == gamma) token */
    int32_t* accept_pos;    /* device out [B] or NULL: position of the last kept node, whose p-bar
                               (or p) gave out_token; A for chains */
    uint32_t* data_status;  /* device out [B] or NULL: what the device found in the sequence's own
                               inputs (each such draft was rejected): bit 0 a draft id outside
                               [0, vocab), bit 1 a tree parent outside [0, t]; 0 = none */
    /* Optional device outputs for inspection; NULL = not written. */
    uint8_t* accept_flags;     /* [B, gamma] decision at every drafted position */
    int32_t* head_argmax;      /* [B, gamma+1, K]; -1 in heads 1.. of lossless sequences */
    int32_t* centroid_argmax;  /* [B, gamma+1]; the undropped argmax for lossless sequences */
    float* head_logz;          /* [B, gamma+1, K] log partition of each head row */
    float* centroid_logz;      /* [B, gamma+1] */
    float* js_heads;           /* [B, gamma, K] JS(p^(i) || p-bar), JS_MAJORITY sequences only */
    float* js_draft;           /* [B, gamma] JS(q_hat || p-bar), JS_MAJORITY sequences only */
    float* logits;             /* [B, gamma+1, K, vocab] every row, fp32 (lossless: head 0) */
    uint32_t* mask_bits;       /* [B, gamma+1, K, d/32] keep bits, bit j%32 of word j/32
                                  (lossless: all ones in head 0) */
    int32_t* filter_count;     /* [B, gamma+1] LOSSLESS sequences, when top_k or top_p is on:
                                  size of the kept set */
    float* filter_logz;        /* [B, gamma+1] same: log of the sum of e^l over the kept set */
} dm_verify_args;

typedef struct dm_verify dm_verify_t; /* opaque */

/* Validates `desc`, allocates the device workspace on the current device.
 * *out receives the handle (NULL on failure). */
int dm_verify_create(const dm_verify_desc* desc, dm_verify_t** out);

/* Enqueues one verify step on `stream` (hipStream_t, NULL = null stream).
 * Validates every argument first; returns without enqueuing on error. */
int dm_verify_run(dm_verify_t* handle, const dm_verify_args* args, void* stream);

/* The same verify step for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  It needs no handle and calls no allocating routine: the
 * workspace is a fixed device array of dm_verify_static_scratch_bytes()
 * bytes (64 MiB) inside the library, one per GPU, held until the process
 * ends.  `desc` gives the limits the handle's desc would (checked the same
 * way); the arguments, outputs, stream behaviour and results are those of
 * dm_verify_run with a handle created from `desc`.  The call's own
 * workspace (masked rows, the fp32 logits of B * (gamma+1) * K rows, the
 * statistics) must fit the array, else it returns DM_ERR_TOO_LARGE before
 * any HIP call: the Llama-3.1-70B-shaped head at B = 1, gamma = 7, K = 5
 * needs about 22 MB.  Every call on a GPU uses that GPU's one array: calls
 * that overlap on one GPU (on different streams, or from several host
 * threads) race and must be serialised by the caller.  Nothing has to be
 * cleared between calls: each call zeroes what it accumulates. */
int dm_verify_run_static(const dm_verify_desc* desc, const dm_verify_args* args, void* stream);

/* Size in bytes of the fixed scratch array of dm_verify_run_static. */
size_t dm_verify_static_scratch_bytes(void);

/* Frees the workspace and the handle.  NULL is a no-op returning DM_OK. */
int dm_verify_destroy(dm_verify_t* handle);

/* For measurement tools: arms `handle` so that its next dm_verify_run records
 * `start` (a hipEvent_t) on the run's stream right before the LM-head GEMM
 * kernel and `stop` right after it; the run then disarms it.  Either event
 * may be NULL to disarm.  The events stay owned by the caller. */
int dm_verify_profile(dm_verify_t* handle, void* start, void* stop);

/* Host-only checks, no HIP call: the validation dm_verify_create and
 * dm_verify_run perform, usable without a GPU.  `args` may be NULL to check
 * only `desc`. */
int dm_verify_check(const dm_verify_desc* desc, const dm_verify_args* args);

/* Device bytes the workspace of `desc` occupies (0 when desc is invalid). */
size_t dm_verify_workspace_bytes(const dm_verify_desc* desc);

/* Panel order of W (DM_W_PANELS).  The LM head is a fixed weight, so it can
 * be reordered once, when the model is loaded, into the order in which the
 * LM-head kernel streams it: each wave then reads one contiguous run of
 * memory in 1 KiB pieces that are already in matrix-core operand order.
 *
 * With E = element size (2 for bf16, 4 for f32), row_bytes = d * E,
 * nkb = row_bytes / 64 and n_panels = ceil(vocab / 64), the packed buffer
 * holds n_panels * nkb * 4 * 1024 bytes.  For panel p, fragment kb, strip g
 * (0..3), lane l (0..63) and byte e (0..15):
 *   packed[((p * nkb + kb) * 4 + g) * 1024 + l * 16 + e]
 *     = byte (kb * 64 + (l / 16) * 16 + e) of row (64 p + 16 g + l % 16) of
 *       row-major W, or 0 when that row is >= vocab.
 * dm_verify_packed_w_bytes returns the size (0 for an invalid desc).
 * dm_verify_pack_w enqueues the reordering of row-major device `W` into
 * device `W_packed` (caller-owned, 16-byte aligned, that many bytes) on
 * `stream`; it checks its arguments on the host first. */
size_t dm_verify_packed_w_bytes(const dm_verify_desc* desc);
int dm_verify_pack_w(const dm_verify_desc* desc, const void* W, void* W_packed, void* stream);

/* Static description of a status code. */
const char* dm_verify_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* DM_VERIFY_H */
