/*
 * eagle3.h -- C ABI of libeagle3.so: one verify step of an EAGLE-3 draft
 * token tree on an AMD Instinct MI355X (gfx950), plus the EAGLE-3 draft head.
 *
 * Sources, by page and section:
 *   [lesson] "EAGLE-3 speculative decoding: the tree-verifier method" (course
 *            lesson): "Verify-accept semantics" (a draft token is accepted when
 *            it equals the target's highest-probability token given the tokens
 *            before it; scan stops at the first miss and the target's token
 *            there is appended), "Tree draft vs chain draft" (the target checks
 *            the whole tree in one forward pass under a mask that lets each
 *            token see only its ancestors).
 *   [blog]   Spec-Bench blog post on EAGLE-3, section 4.2 (inference table:
 *            top-k 10, 60 draft tokens); used for workload parameters only.
 *   [news]   News write-up of "EAGLE-3: Scaling up Inference Acceleration of
 *            Large Language Models via Training-Time Test": the draft-stage
 *            paragraphs (low/mid/high features l, m, h fused by an FC from 3k to
 *            k; concatenation with the embedding of the token one step ahead;
 *            an FC to k; a single-layer transformer; the target's LM head), and
 *            the note that each forward of the target reads all its parameters.
 *
 * Conventions for every entry point:
 *   - All tensor arguments are DEVICE pointers owned by the caller, dense
 *     row-major with the shapes given below. Floating-point tensors are bf16
 *     (raw 16-bit patterns) or fp32 as selected by the `dtype` argument; they
 *     must be 16-byte aligned. Index tensors are int32, masks uint64.
 *   - The library never allocates or frees device memory. Scratch comes from
 *     the caller through a `ws` pointer sized by the matching *_workspace()
 *     query (same arguments). It keeps no state between calls.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     the call returns without synchronising.
 *   - Errors found on the host are returned before anything is launched:
 *       EAGLE3_ERR_ARG          null pointer, negative size, misalignment
 *       EAGLE3_ERR_UNSUPPORTED  a shape or option this library does not handle
 *       EAGLE3_ERR_WORKSPACE    ws smaller than the *_workspace() query
 *     A launch failure returns EAGLE3_ERR_HIP. Data errors (a parent[] that is
 *     not a tree in topological order, an id out of range) are reported
 *     through the optional device status arrays; without them the outputs of
 *     bad data are unspecified but every memory access stays in bounds.
 *   - No call throws; every call is safe to make from several host threads on
 *     different streams.
 *
 * Tree conventions (reading of [lesson]): node 0 of every tree is the root,
 * the last committed token; parent[0] = -1 and 0 <= parent[n] < n for n > 0.
 * T = number of nodes including the root; T <= 64 * W where W is the number
 * of 64-bit mask words per node (W = 1 or 2).
 */
#ifndef EAGLE3_H
#define EAGLE3_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum eagle3_status {
    EAGLE3_OK = 0,
    EAGLE3_ERR_ARG = -1,
    EAGLE3_ERR_UNSUPPORTED = -2,
    EAGLE3_ERR_TREE = -3,
    EAGLE3_ERR_RANGE = -4,
    EAGLE3_ERR_HIP = -5,
    EAGLE3_ERR_WORKSPACE = -6
};

enum eagle3_dtype { EAGLE3_F32 = 0, EAGLE3_BF16 = 1 };

/* Human-readable name of a status code (static storage; never NULL). */
const char *eagle3_status_string(int status);

/* ABI version: bumped whenever a signature or layout below changes. */
int eagle3_abi_version(void);

/*
 * Ancestor bitmask of every node ([lesson] "Tree draft vs chain draft": a node
 * sees only its ancestors; reading: and itself).
 *   parent  [B, T] int32
 *   mask    [B, T, W] uint64 out: bit (t % 64) of word t / 64 of node n is set
 *           iff t is n or an ancestor of n
 *   depth   [B, T] int32 out (nullable): number of ancestors excluding n
 *   status  [B] int32 out (nullable): EAGLE3_OK, or EAGLE3_ERR_TREE when the
 *           sequence's parent[] breaks the tree conventions (its mask is then
 *           unspecified)
 * Needs 1 <= T <= 64 * W, W in {1, 2}.
 */
int eagle3_tree_mask(const int32_t *parent, int B, int T, int W,
                     uint64_t *mask, int32_t *depth, int32_t *status, void *stream);

/*
 * Tree attention ([lesson] "Tree draft vs chain draft"; GQA reading: query
 * head h reads KV head h / (Hq / Hkv)). For sequence b, query node i, head h:
 *   keys = the b-th prefix (prefix_len[b] positions, paged) followed by the
 *          tree keys t = 0..Tk-1 whose bit is set in mask[b][i];
 *   out  = softmax(scale * q . k) . v over those keys; lse = ln sum exp.
 * Layouts:
 *   q        [B, Tq, Hq, D]            k_tree, v_tree [B, Tk, Hkv, D]
 *   k_cache  [num_blocks, Hkv, block_size, D]   (key rows, D contiguous)
 *   v_cache  [num_blocks, Hkv, D, block_size]   (value columns, slot contiguous)
 *   block_table [B, max_blocks] int32: physical block of logical block j of
 *            sequence b; entries past ceil(prefix_len[b] / block_size) are
 *            never read
 *   prefix_len [B] int32, each in [0, max_blocks * block_size]
 *   mask     [B, Tq, W] uint64 over the Tk tree keys (from eagle3_tree_mask
 *            when the queries are the tree nodes themselves, Tq == Tk), or
 *            NULL together with parent [B, Tq] (Tq == Tk) to build it on the fly
 *   out      [B, Tq, Hq, D]; lse [B, Tq, Hq] fp32 (nullable), natural log
 * Supported: bf16 with D = 128; fp32 with D = 64 or 128; block_size 16;
 * Tk <= 64 * W, W in {1, 2}; Hq % Hkv == 0. A query row that sees no key gets
 * out = 0 and lse = -inf. Slots of the cache past prefix_len are never read.
 * split_keys: prefixes are cut into splits of split_keys keys (a positive
 * multiple of 64; EAGLE3_ERR_UNSUPPORTED otherwise), each attended by its own
 * work-groups, and the partial results merged in split order. 0 = automatic:
 * no split when the call has at least one (sequence, KV head, block of 256
 * query rows) work-group per CU, else enough splits of at least 256 keys to
 * cover the CUs, cut from max_blocks * block_size. Splits need the workspace
 * eagle3_tree_attn_workspace() reports (0 without splits; the fp32 path never
 * splits). For a given split_keys, results do not depend on the call's batch
 * composition.
 * norm_out (nullable): the RMSNorm (gamma = 1, eps = norm_eps) of each output
 * row [Hq * D], as eagle3_rmsnorm on out would give (a second launch).
 * Validate mode: with status [B] int32 non-NULL, each sequence's status is
 * written before the attention runs: EAGLE3_ERR_RANGE when prefix_len[b] lies
 * outside [0, max_blocks * block_size] or a block id the prefix uses
 * (block_table[b][j], j < ceil(prefix_len[b] / block_size)) lies outside
 * [0, num_blocks); else EAGLE3_ERR_TREE when parent[] is given and is not a
 * tree in topological order; else EAGLE3_OK. Without it, bad ids are clamped
 * (wrong values, never an out-of-bounds access).
 */
typedef struct eagle3_tree_attn_args {
    int dtype;
    int B, Tq, Tk, Hq, Hkv, D, W;
    float scale;
    const void *q;
    const void *k_tree;
    const void *v_tree;
    const void *k_cache;
    const void *v_cache;
    int num_blocks, block_size;
    const int32_t *block_table;
    int max_blocks;
    const int32_t *prefix_len;
    const uint64_t *mask;
    const int32_t *parent;
    void *out;
    float *lse;
    int split_keys;
    void *norm_out;  /* nullable: [B, Tq, Hq * D], RMSNorm (gamma = 1, norm_eps) of each output row */
    float norm_eps;
    int32_t *status; /* nullable: [B] validate mode (see above) */
} eagle3_tree_attn_args;

size_t eagle3_tree_attn_workspace(const eagle3_tree_attn_args *a);
int eagle3_tree_attn(const eagle3_tree_attn_args *a, void *ws, size_t ws_bytes, void *stream);

/*
 * RMSNorm over the last dimension (reading: the hidden state is normalised
 * before the LM head, as in Llama): y = x / sqrt(mean(x^2) + eps) * gamma.
 *   x, y [M, K]; gamma [K] (nullable: 1). In-place (x == y) is allowed.
 * Supported: K % 8 == 0.
 */
int eagle3_rmsnorm(const void *x, const void *gamma, int M, int K, float eps,
                   int dtype, void *y, void *stream);

/*
 * LM head with a fused per-row selection; the [M, N] logits are never stored
 * ([lesson] "Verify-accept semantics": the target's argmax at each node;
 * [news]: the draft also uses the target's LM head).
 *   hidden [M, K]; w [N, K] (vocabulary-major)
 *   idx [M, topk] int32, val [M, topk] fp32: the topk largest logits of each
 *        row in the order (logit descending, id ascending), so idx[m][0] is
 *        the lowest id attaining the maximum
 *   gap [M] fp32 (nullable): top1 - top2, top2 the largest logit over the
 *        other ids (0 on an exact tie)
 *   lse [M] fp32 (nullable): ln sum_v exp(logit_v)
 * Supported: 1 <= topk <= 16; K % 64 == 0 (bf16), K % 4 == 0 (fp32); N >= 2.
 * Logits are accumulated in fp32 (bf16 products are exact in fp32) in a k
 * order that is fixed per 128-row vocabulary tile, so a row's result never
 * depends on the other rows; bitwise-equal logits resolve to the lowest id
 * (duplicate weight rows in different tiles may differ in the last bits).
 */
size_t eagle3_lmhead_workspace(int M, int N, int K, int topk, int dtype);
int eagle3_lmhead_argmax(const void *hidden, const void *w, int M, int N, int K, int topk, int dtype,
                         int32_t *idx, float *val, float *gap, float *lse,
                         void *ws, size_t ws_bytes, void *stream);

/*
 * eagle3_lmhead_argmax for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid it):
 * same arguments and results, no workspace argument. The per-tile records go
 * to a device array inside the library, EAGLE3_LMHEAD_NOALLOC_MAX_BYTES long,
 * one copy per GPU, held until the process ends. A call whose records need
 * more (eagle3_lmhead_workspace() of the same arguments) returns
 * EAGLE3_ERR_WORKSPACE before any launch; the limit covers a 64-sequence
 * verify batch of 61-node trees over a 128256-row head (3904 rows, top-2) and
 * the draft head's 640-row top-10 calls. The call allocates nothing (the
 * array's address is looked up once per device, on the first call with that
 * device current). All calls on one GPU share the array: calls that overlap
 * in time on one GPU (other streams, other host threads) race.
 */
#define EAGLE3_LMHEAD_NOALLOC_MAX_BYTES ((size_t)96 << 20)
int eagle3_lmhead_argmax_noalloc(const void *hidden, const void *w, int M, int N, int K, int topk, int dtype,
                                 int32_t *idx, float *val, float *gap, float *lse, void *stream);

/*
 * Greedy acceptance on a tree ([lesson] "Verify-accept semantics", applied to
 * every root-to-leaf path). A non-root node is accepted when its parent is
 * accepted and tokens[n] == target_idx[parent[n]]; the root always is.
 * accept_len = depth of the deepest accepted node; among equally deep ones the
 * lowest index is the end node (reading). Outputs:
 *   accept_len [B] int32
 *   path       [B, T] int32: root, ..., end node; -1 after
 *   out_tokens [B, T] int32: tokens of path[1..accept_len], then
 *              target_idx[end] (the target's own token); -1 after
 * Inputs: tokens, target_idx [B, T] int32; exactly one of parent [B, T] or
 * mask [B, T, W] (from eagle3_tree_mask) non-NULL. T <= 64 * W, W in {1, 2}.
 * Validate mode: with status [B] int32 non-NULL, each sequence's status is
 * written: EAGLE3_ERR_TREE when a given parent[] is not a tree in topological
 * order (parent[0] != -1 or parent[n] outside [0, n)), else EAGLE3_ERR_RANGE
 * when a token or target id lies outside [0, V), else EAGLE3_OK. V >= 1 is
 * required with status (EAGLE3_ERR_ARG otherwise) and ignored without it. The
 * outputs are written either way; for a flagged sequence they are unspecified.
 */
int eagle3_accept_path(const int32_t *tokens, const int32_t *parent, const uint64_t *mask, int W,
                       const int32_t *target_idx, int B, int T,
                       int32_t *accept_len, int32_t *path, int32_t *out_tokens,
                       int V, int32_t *status, void *stream);


/*
 * Node positions for the target's pass over a tree ([lesson] "Verify-accept
 * semantics": the drafts continue the committed sequence; reading: a node at
 * depth d sits d places after the root, and the root takes the first free
 * position): pos[b][t] = prefix_len[b] + depth[b][t]. prefix_len [B], depth
 * and pos [B, T] int32 device (depth from eagle3_tree_mask); B * T < 2^31.
 */
int eagle3_node_positions(const int32_t *prefix_len, const int32_t *depth, int B, int T, int32_t *pos,
                          void *stream);

/*
 * Bookkeeping after acceptance for a decoding loop that stays on the device
 * ([lesson] "Verify-accept semantics": the accepted drafts and the target's
 * own token at the end node extend the sequence; [news] draft stage: a
 * context row of the draft pairs the target's features of a token with the
 * embedding of the token after it). For sequence b with a = accept_len[b]
 * (from eagle3_accept_path; a < min(T, R) is required, larger values are
 * clamped) and P = prefix_len[b] on entry:
 *   start[b] = P;  prefix_len[b] = P + a + 1     (in place)
 *   path_rows[b][j] = b * T + path[b][j] for j <= a, else -1   [B, R]: the
 *       accepted rows of the [B * T] tree rows, in path order (for a row gather)
 *   tok_ahead[b][j] = out_tokens[b][j] for j <= a, else 0      [B, R]: the
 *       token after row j (the next accepted draft, then the target's token)
 *   last_rows[b] = b * R + a;   root[b] = out_tokens[b][a]   (the next root)
 *   out_seq [B, cap] (nullable; needs out_len [B]): out_tokens[b][0..a] are
 *       written at out_seq[b][out_len[b]..] (entries past cap dropped), then
 *       out_len[b] += a + 1.
 * All int32 device arrays; accept_len, path, out_tokens as written by
 * eagle3_accept_path ([B], [B, T], [B, T]). No output may alias an input.
 */
int eagle3_spec_advance(const int32_t *accept_len, const int32_t *path, const int32_t *out_tokens, int B, int T,
                        int R, int32_t *prefix_len, int32_t *start, int32_t *path_rows, int32_t *tok_ahead,
                        int32_t *last_rows, int32_t *root, int32_t *out_seq, int32_t *out_len, int cap,
                        void *stream);

/*
 * Trimmed draft vocabulary ([blog] sections 1, 3.2 and 5.1: VocabTrim, FR-Spec
 * and SpecVocab shrink the draft's search space by 40-60%). The draft LM head
 * runs over V_sub kept rows, row i being full-vocabulary id vmap[i] (gather
 * them once, e.g. with eagle3_copy_rows), so eagle3_lmhead_argmax returns row
 * numbers of the trimmed head; this maps them back before they enter the tree:
 *   out[i] = vmap[ids[i]]  for i < n;  an id outside [0, V_sub) gives -1.
 * ids, out [n] int32 device (out may be ids: in place); vmap [V_sub] int32
 * device, strictly ascending (caller's duty), so that the lowest-row rule of
 * eagle3_lmhead_argmax on ties is the lowest-full-id rule. With status [1]
 * int32 non-NULL, status[0] = EAGLE3_ERR_RANGE if any id was out of range,
 * else EAGLE3_OK (written also for n == 0). One work-group of 1024 threads:
 * sized for the few thousand ids of a draft step.
 */
int eagle3_vocab_map(const int32_t *ids, int n, const int32_t *vmap, int V_sub, int32_t *out, int32_t *status,
                     void *stream);

/*
 * Dense layers for the EAGLE-3 draft head and small decoders.
 *
 * [news] draft stage: an FC reduces the concatenated low/mid/high features
 * (3k) to k; the result (from step 2 on, the draft's own output) is
 * concatenated with the embedding of the token one step ahead and an FC takes
 * 2k to k; a single transformer layer and the target's LM head follow.
 * reading: the layer is a Llama decoder layer (RMSNorm, GQA with rotate-half
 * RoPE, SwiGLU MLP, residual adds).
 *
 * eagle3_gemm: C[M, N] = A[M, K] . B[N, K]^T (+ residual), where A is the
 * concatenation along K of nseg (1..3) segments: segment s has k[s] columns
 * and its row for output row m is a[s][a_rows[s][m]] (a_rows[s] nullable:
 * row m itself; gathered rows are clamped to [0, a_nrows[s])). So the fusion
 * FCs read [l; m; h] and [g; E[token]] without building the concatenation.
 *   a[s]       [rows_s, k[s]] row-major          b  [N, sum k] row-major
 *   residual   [M, ldc] (nullable; may alias c)   c  [M, ldc] (ldc 0 = N)
 * bf16: fp32 accumulation, each k[s] % 64 == 0, pointers 16-byte aligned;
 * fp32: any sizes. Without a workspace the summation order is fixed per
 * output column block, so a row's result does not depend on the other rows
 * of the call.
 * ws / ws_bytes (optional, device, caller-owned, 16-byte aligned): when the
 * output tiles would leave more than half of the CUs idle, a bf16 call given
 * at least eagle3_gemm_workspace(args) bytes splits K over up to 8
 * work-groups per tile and adds the fp32 partials in split order (plus the
 * residual) before the one rounding to bf16. The split count depends on M,
 * so with a workspace a row's rounding can depend on the batch (results stay
 * within the same accuracy). NULL or too small: no split, same results as
 * without. A large bf16 call (one A segment without a row gather, 256 x 256
 * output tiles at least four times the CU count or as many as the CUs, N and
 * ldc multiples of 8, c and residual 16-byte aligned, K >= 128) given at least
 * EAGLE3_PERSIST_WS_BYTES runs one work-group per CU that takes output tiles
 * from counters kept in the workspace (the caller must not use it for
 * anything else while the call runs); its results are the same as without.
 */
typedef struct eagle3_gemm_args {
    int dtype;
    int M, N;
    int nseg;
    const void *a[3];
    const int32_t *a_rows[3];
    int a_nrows[3];
    int k[3];
    const void *b;
    const void *residual;
    void *c;
    int ldc;
    void *ws;
    size_t ws_bytes;
} eagle3_gemm_args;

/* bf16: each A segment (M rows, or a_nrows rows when gathered) must be under
 * 4 GiB (EAGLE3_ERR_UNSUPPORTED otherwise); the same holds for the hidden
 * state of eagle3_lmhead_argmax. */
/* bytes of workspace the call would use: S * M * N * 4 to split K S ways
 * (S >= 2), or EAGLE3_PERSIST_WS_BYTES for the tile counters of its
 * persistent form (a call takes one or neither); 0: it would use none */
size_t eagle3_gemm_workspace(const eagle3_gemm_args *args);

int eagle3_gemm(const eagle3_gemm_args *args, void *stream);

/* SwiGLU gating (reading: Llama's MLP): y[m][f] = silu(gu[m][f]) * gu[m][F + f]
 * with silu(g) = g / (1 + exp(-g)); gu [M, 2F] (gate columns first), y [M, F]. */
int eagle3_silu_mul(const void *gu, int M, int F, int dtype, void *y, void *stream);

/* The gate/up projection and the SwiGLU gating in one call (reading: Llama's
 * MLP), y[m][f] = silu(g[m][f]) * u[m][f] with g = A . Wg^T and u = A . Wu^T
 * rounded to bf16 first, so y equals eagle3_gemm followed by eagle3_silu_mul
 * bit for bit. bf16 only. args as for eagle3_gemm except: b is the gate/up
 * weight [N = 2F, K] in paired layout (rows 256 j .. 256 j + 127 are gate rows
 * 128 j .. 128 j + 127, the next 128 rows the up rows of the same outputs;
 * eagle3_copy_rows with a row table builds it from [Wg; Wu]); N % 256 == 0;
 * c is y [M, F] with row stride ldc (0: F; a multiple of 8; 16-byte aligned);
 * no residual. ws / ws_bytes (optional, device, caller-owned, 16-byte
 * aligned, at least EAGLE3_PERSIST_WS_BYTES): for large calls with one A
 * segment and no row gather, the call then runs one work-group per CU that
 * takes output tiles from counters kept there (the caller must not use the
 * workspace for anything else while the call runs); results are the same
 * with or without it. */
#define EAGLE3_PERSIST_WS_BYTES ((size_t)1024)
int eagle3_gemm_swiglu(const eagle3_gemm_args *args, void *stream);

/* Rotary embedding, rotate-half convention (reading): in place on x viewed as
 * [M][H][D] with row stride ld (elements, >= H * D); row m sits at position
 * p = pos_offset + pos[m] (e.g. the committed length plus the node's depth)
 * and pair (i, i + D/2) turns by p * theta^(-2i/D) (angle in double). */
int eagle3_rope(void *x, int M, int H, int D, int ld, const int32_t *pos, int pos_offset, float theta, int dtype,
                void *stream);

/* Embedding gather: out[m] = E[ids[m]] (ids clamped to [0, V)); E [V, K],
 * out [M, K]; K * element size must be a multiple of 16 bytes. */
int eagle3_embed(const void *E, const int32_t *ids, int M, int K, int V, int dtype, void *out, void *stream);

/* Row copy: dst[dst_rows[i]] = src[src_rows[i]] for i < n (device int32
 * tables; NULL = identity); a row index outside [0, src_nrows) or
 * [0, dst_nrows) skips that row. Rows are row_bytes long (a multiple of 16;
 * both bases 16-byte aligned). Used to gather the parents' draft outputs and
 * to place a draft step's K/V rows among the tree keys. Repeated destination
 * rows race. */
int eagle3_copy_rows(const void *src, const int32_t *src_rows, int src_nrows, void *dst, const int32_t *dst_rows,
                     int dst_nrows, int n, size_t row_bytes, void *stream);

/*
 * Append K/V rows to the paged cache after acceptance ([lesson] "Verify-accept
 * semantics": the accepted tokens become part of the sequence). For sequence
 * b, rows src[b][0..] of k_rows / v_rows [B, rows_per_seq, Hkv, D] go to
 * positions start[b] + j of the cache (layouts as in eagle3_tree_attn); the
 * list ends at the first negative entry or after max_n entries, so the `path`
 * output of eagle3_accept_path can be passed as is; a NULL src means rows
 * 0..max_n-1 of every sequence (bulk ingest of a context). src [B, max_n] and
 * start [B] are device int32 arrays; positions past max_blocks * 16 are
 * skipped; B <= 65535. Entries listing the same cache position race.
 */
int eagle3_commit_kv(const void *k_rows, const void *v_rows, int rows_per_seq, const int32_t *src, int max_n,
                     int B, int Hkv, int D, int dtype, void *k_cache, void *v_cache, const int32_t *block_table,
                     int max_blocks, int num_blocks, const int32_t *start, void *stream);

/*
 * EAGLE-3 draft input fusion ([news] draft stage):
 *   context mode (a_prev == NULL): g = w_fuse . [l; m; h]; x = w_in . [g; E[tok]]
 *   step mode    (l = m = h = NULL): x = w_in . [a_prev; E[tok]]
 * l, m, h, a_prev, g_out, x_out [M, k]; tok [M] int32 (the token one step
 * ahead of each row); E [V, k]; w_fuse [k, 3k]; w_in [k, 2k] (output-major).
 * g is stored (g_out, or the workspace when g_out is NULL) in the storage type
 * before the second FC. bf16 needs k % 64 == 0. The workspace query also
 * covers the GEMM workspace of the two FCs (K splits or the tile counters of
 * the persistent form, see eagle3_gemm): it follows g when g lives in the
 * workspace; with g_out (or in step mode) the whole workspace is the GEMMs'.
 * The query's size covers both cases. A smaller workspace runs the plain
 * form: the same results except for the rounding of a K split.
 */
size_t eagle3_draft_fuse_workspace(int M, int k, int dtype);
int eagle3_draft_fuse(const void *l, const void *m, const void *h, const void *a_prev, const int32_t *tok,
                      const void *E, const void *w_fuse, const void *w_in, int M, int k, int V, int dtype,
                      void *g_out, void *x_out, void *ws, size_t ws_bytes, void *stream);

/*
 * Draft-tree growth, EAGLE-2 style ([news]: the draft's confidence stands in
 * for the acceptance rate and shapes the tree; [blog] section 4.2: top-k 10,
 * 60 draft tokens). reading: score(child) = fp32(score(parent) + logp(child)),
 * every selection ranks by (score desc, creation index asc), and the pool keeps
 * every candidate ever drafted.
 *
 * eagle3_tree_expand: one step for B sequences. The F current frontier nodes
 * (fr_score, fr_pool = their pool index or -1 for the root, fr_mask = the draft
 * rows each may attend to, 2 words) each bring C children: child_ids,
 * child_val [B, F, C] (the LM head's top-C ids and logits) and child_lse
 * [B, F] (the row's log-sum-exp; nullable when child_val already holds
 * log-probabilities), logp = fp32(val - lse). The F*C candidates are appended to the pool at
 * pool_len.. (pool_* [B, pool_cap], creation order frontier-slot major) and the
 * top NF become the next frontier: next_pool/next_score/next_token [B, NF];
 * next_mask [B, NF, 2] = parent's mask plus the node's own draft row
 * row_base + rank; next_arow [B, NF] = b * arow_stride + fr_arow_base + f, the
 * row (in a per-sequence buffer of draft outputs) holding the parent's output.
 * Needs F * C <= 256, NF <= F * C, row_base + NF <= 128.
 *
 * eagle3_tree_rerank: pool (pool_len entries) -> top N -> creation order ->
 * parent [B, N + 1] and tokens [B, N + 1] with node 0 = the root
 * (root_token [B]); parents are remapped (the selection is closed under
 * parents because a child never outscores its parent). pool_len <= 4096.
 */
int eagle3_tree_expand(const float *fr_score, const int32_t *fr_pool, const uint64_t *fr_mask, int fr_arow_base,
                       int arow_stride, const int32_t *child_ids, const float *child_val, const float *child_lse,
                       int B, int F, int C, int NF, int pool_len, int pool_cap, int row_base, float *pool_score,
                       int32_t *pool_token,
                       int32_t *pool_parent, int32_t *next_pool, float *next_score, int32_t *next_token,
                       uint64_t *next_mask, int32_t *next_arow, void *stream);
int eagle3_tree_rerank(const float *pool_score, const int32_t *pool_token, const int32_t *pool_parent, int B,
                       int pool_len, int pool_cap, int N, const int32_t *root_token, int32_t *parent,
                       int32_t *tokens, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* EAGLE3_H */
