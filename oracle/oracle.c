/*
 * oracle.c -- plain CPU oracle for one EAGLE-3 draft-tree verify step and
 * the EAGLE-3 draft head.
 *
 * TEST INFRASTRUCTURE. Only the tests, the package's smoke check and the
 * benchmark's CPU-baseline leg load this library. It shares no code, header,
 * table or constant with the GPU path, and it never touches a device.
 *
 * Rules this file keeps, so that a reader can check it against the pages:
 *   - every reduction runs in double precision, in one documented order
 *     (ascending index: dimension k, key j, vocabulary id v);
 *   - results are rounded once, to the storage type of the output tensor
 *     (fp32: C cast; bf16: round-to-nearest-even from the double value);
 *   - every row is computed on its own: a row's result never depends on which
 *     other rows are in the call. OpenMP only splits independent rows.
 *
 * Sources (cited by page title and section; the pages are web pages):
 *   [lesson]  "EAGLE-3 speculative decoding: the tree-verifier method" (course
 *             lesson): "Verify-accept semantics", "Tree draft vs chain draft".
 *   [news]    News write-up of "EAGLE-3: Scaling up Inference Acceleration of
 *             Large Language Models via Training-Time Test": the draft stage
 *             paragraphs (features l, m, h; the fusion FC; the embedding of the
 *             token one step ahead; the single-layer transformer; steps 1-3).
 * Where the pages are silent the plainest reading is taken and marked
 * "reading:" in the comment.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1
#define ORC_OK 0
#define ORC_ERR_TREE (-3)

/* ------------------------------------------------------------ storage */

static double ld(const void *p, int dtype, size_t i) {
    if (dtype == ORC_F32) return (double)((const float *)p)[i];
    uint32_t u = (uint32_t)((const uint16_t *)p)[i] << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static void ld_row(const void *p, int dtype, size_t off, int n, double *dst) {
    for (int i = 0; i < n; ++i) dst[i] = ld(p, dtype, off + (size_t)i);
}

/* double -> bf16 bit pattern, rounded to nearest even directly from the
 * double (no intermediate fp32 rounding). bf16 keeps 8 significant bits and
 * the fp32 exponent range (smallest subnormal step 2^-133). */
static uint16_t to_bf16(double x) {
    if (isnan(x)) return 0x7FC0;
    if (x == 0.0) return signbit(x) ? 0x8000 : 0x0000;
    int e;
    frexp(x, &e);                       /* |x| = m * 2^e, m in [0.5, 1) */
    int step_exp = e - 8;
    if (step_exp < -133) step_exp = -133;
    double step = ldexp(1.0, step_exp);
    double r = nearbyint(x / step) * step; /* default mode: ties to even */
    float f = (float)r;                 /* exact unless it overflows */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

static void st(void *p, int dtype, size_t i, double x) {
    if (dtype == ORC_F32) ((float *)p)[i] = (float)x;
    else ((uint16_t *)p)[i] = to_bf16(x);
}

/* exported for the oracle's own rounding pins */
uint16_t orc_round_bf16(double x) { return to_bf16(x); }

/* ------------------------------------------------------------ O1: tree
 * The draft tree is parent[]: node 0 is the root (the last committed token,
 * reading: it belongs to the tree), every other node's parent has a smaller
 * index. anc(n) = {n} + anc(parent[n]): a node sees itself and its ancestors
 * and nothing else ([lesson] "Tree draft vs chain draft": the target checks
 * the whole tree in one pass, with a mask so that each token sees only its
 * ancestors).
 */
int orc_tree_check(const int32_t *parent, int T) {
    if (T < 1 || parent[0] != -1) return ORC_ERR_TREE;
    for (int n = 1; n < T; ++n)
        if (parent[n] < 0 || parent[n] >= n) return ORC_ERR_TREE;
    return ORC_OK;
}

/* mask[b][n][w]: bit (t mod 64) of word t/64 set iff t in anc(n); depth[b][n] = |anc(n)| - 1. */
int orc_tree_mask(const int32_t *parent, int B, int T, int W, uint64_t *mask, int32_t *depth) {
    for (int b = 0; b < B; ++b) {
        const int32_t *par = parent + (size_t)b * T;
        if (orc_tree_check(par, T) != ORC_OK) return ORC_ERR_TREE;
        uint64_t *mk = mask + (size_t)b * T * W;
        int32_t *dp = depth + (size_t)b * T;
        for (int n = 0; n < T; ++n) {
            uint64_t *row = mk + (size_t)n * W;
            for (int w = 0; w < W; ++w) row[w] = 0;
            if (n > 0) {
                const uint64_t *prow = mk + (size_t)par[n] * W;
                for (int w = 0; w < W; ++w) row[w] = prow[w];
                dp[n] = dp[par[n]] + 1;
            } else {
                dp[n] = 0;
            }
            row[n / 64] |= (uint64_t)1 << (n % 64);
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------ O2: tree attention
 * Dense attention with an explicit mask. For sequence b, query node i, query
 * head h (kv head = h / (Hq/Hkv), reading: contiguous GQA groups):
 *   keys, in this order: prefix positions j = 0..L_b-1, read through the
 *   block table (block = table[b][j / bs], slot = j % bs), then the tree keys
 *   t = 0..Tk-1 with t visible iff bit t of mask[b][i] is set. Invisible keys
 *   are skipped, not weighted by zero.
 *   s_j = scale * sum_d q[d] k_j[d]          (d ascending)
 *   m = max s_j; p_j = exp(s_j - m); l = sum p_j (key order)
 *   out[d] = (sum_j p_j v_j[d]) / l;  lse = m + ln l.
 * A row with no visible key gives out = 0 and lse = -inf.
 * Layouts: q [B,Tq,Hq,D]; k_tree, v_tree [B,Tk,Hkv,D];
 *   k_cache [nblk,Hkv,bs,D]; v_cache [nblk,Hkv,D,bs] (slot index fastest).
 */
void orc_tree_attn(int dtype, int B, int Tq, int Tk, int Hq, int Hkv, int D, double scale,
                   const void *q, const void *k_tree, const void *v_tree,
                   const void *k_cache, const void *v_cache, int bs,
                   const int32_t *block_table, int max_blocks, const int32_t *prefix_len,
                   const uint64_t *mask, int W, void *out, float *lse) {
    const int G = Hq / Hkv;
    int Lmax = 0;
    for (int b = 0; b < B; ++b) if (prefix_len[b] > Lmax) Lmax = prefix_len[b];
    const long total = (long)B * Tq * Hq;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(Lmax + Tk));
        char *vis = (char *)malloc((size_t)(Lmax + Tk) + 1);
        double *qv = (double *)malloc(sizeof(double) * (size_t)D);
        double *acc = (double *)malloc(sizeof(double) * (size_t)D);
#pragma omp for schedule(dynamic, 4)
        for (long r = 0; r < total; ++r) {
            const int h = (int)(r % Hq);
            const int i = (int)((r / Hq) % Tq);
            const int b = (int)(r / ((long)Hq * Tq));
            const int kvh = h / G;
            const int L = prefix_len[b];
            ld_row(q, dtype, (((size_t)b * Tq + i) * Hq + h) * D, D, qv);
            const uint64_t *mrow = mask + ((size_t)b * Tq + i) * W;
            int nvis = 0;
            double m = -INFINITY;
            for (int j = 0; j < L + Tk; ++j) {
                double dot = 0.0;
                if (j < L) {
                    const int blk = block_table[(size_t)b * max_blocks + j / bs];
                    const size_t base = (((size_t)blk * Hkv + kvh) * bs + (j % bs)) * D;
                    for (int d = 0; d < D; ++d) dot += qv[d] * ld(k_cache, dtype, base + d);
                    vis[j] = 1;
                } else {
                    const int t = j - L;
                    vis[j] = (char)((mrow[t / 64] >> (t % 64)) & 1u);
                    if (!vis[j]) continue;
                    const size_t base = (((size_t)b * Tk + t) * Hkv + kvh) * D;
                    for (int d = 0; d < D; ++d) dot += qv[d] * ld(k_tree, dtype, base + d);
                }
                s[j] = dot * scale;
                if (s[j] > m) m = s[j];
                ++nvis;
            }
            const size_t obase = (((size_t)b * Tq + i) * Hq + h) * D;
            if (nvis == 0) {
                for (int d = 0; d < D; ++d) st(out, dtype, obase + d, 0.0);
                if (lse) lse[((size_t)b * Tq + i) * Hq + h] = -INFINITY;
                continue;
            }
            double l = 0.0;
            for (int d = 0; d < D; ++d) acc[d] = 0.0;
            for (int j = 0; j < L + Tk; ++j) {
                if (!vis[j]) continue;
                const double p = exp(s[j] - m);
                l += p;
                if (j < L) {
                    const int blk = block_table[(size_t)b * max_blocks + j / bs];
                    const size_t base = ((size_t)blk * Hkv + kvh) * (size_t)D * bs + (j % bs);
                    for (int d = 0; d < D; ++d) acc[d] += p * ld(v_cache, dtype, base + (size_t)d * bs);
                } else {
                    const int t = j - L;
                    const size_t base = (((size_t)b * Tk + t) * Hkv + kvh) * D;
                    for (int d = 0; d < D; ++d) acc[d] += p * ld(v_tree, dtype, base + d);
                }
            }
            for (int d = 0; d < D; ++d) st(out, dtype, obase + d, acc[d] / l);
            if (lse) lse[((size_t)b * Tq + i) * Hq + h] = (float)(m + log(l));
        }
        free(s); free(vis); free(qv); free(acc);
    }
}

/* ------------------------------------------------------------ O3: RMSNorm
 * reading: the hidden state is RMS-normalised before the LM head, as in Llama:
 *   y = x / sqrt(mean_k x_k^2 + eps) * gamma   (gamma = 1 when NULL).
 */
void orc_rmsnorm(int dtype, const void *x, const void *gamma, int M, int K, double eps, void *y) {
#pragma omp parallel for schedule(static)
    for (int m = 0; m < M; ++m) {
        double ss = 0.0;
        for (int k = 0; k < K; ++k) { const double v = ld(x, dtype, (size_t)m * K + k); ss += v * v; }
        const double r = 1.0 / sqrt(ss / K + eps);
        for (int k = 0; k < K; ++k) {
            const double g = gamma ? ld(gamma, dtype, (size_t)k) : 1.0;
            st(y, dtype, (size_t)m * K + k, ld(x, dtype, (size_t)m * K + k) * r * g);
        }
    }
}

/* ------------------------------------------------------------ O4: LM head
 * logits[m][v] = sum_k h[m][k] * W[v][k] (k ascending) over the whole
 * vocabulary; nothing is pruned. Outputs per row, in the order
 * (logit descending, id ascending):
 *   idx[m][0..topk-1], val[m][0..topk-1]  -- so idx[m][0] is the lowest id
 *                                            attaining the maximum;
 *   gap[m] = top1 - (largest logit over v != idx[m][0])  (0 on an exact tie);
 *   lse[m] = log sum_v exp(logit_v)  (max-shifted; sum in id order).
 * The target's argmax at a node is what the draft token is checked against
 * ([lesson] "Verify-accept semantics"); the top-k feeds the draft tree.
 * Rows are processed in groups of 32 to bound the logit buffer; each row's
 * arithmetic is the same whatever the group.
 */
void orc_lmhead(int dtype, const void *h, const void *w, int M, int N, int K, int topk,
                int32_t *idx, double *val, double *gap, double *lse) {
    const int GR = 32;
    double *logit = (double *)malloc(sizeof(double) * (size_t)GR * N);
    double *hrow = (double *)malloc(sizeof(double) * (size_t)GR * K);
    for (int m0 = 0; m0 < M; m0 += GR) {
        const int gm = (M - m0 < GR) ? (M - m0) : GR;
        for (int r = 0; r < gm; ++r) ld_row(h, dtype, (size_t)(m0 + r) * K, K, hrow + (size_t)r * K);
#pragma omp parallel
        {
            double *wrow = (double *)malloc(sizeof(double) * (size_t)K);
#pragma omp for schedule(static)
            for (int v = 0; v < N; ++v) {
                ld_row(w, dtype, (size_t)v * K, K, wrow);
                for (int r = 0; r < gm; ++r) {
                    const double *hr = hrow + (size_t)r * K;
                    double acc = 0.0;
                    for (int k = 0; k < K; ++k) acc += hr[k] * wrow[k];
                    logit[(size_t)r * N + v] = acc;
                }
            }
            free(wrow);
        }
#pragma omp parallel for schedule(static)
        for (int r = 0; r < gm; ++r) {
            const double *lg = logit + (size_t)r * N;
            const int m = m0 + r;
            /* top-k by insertion into a sorted list: (value desc, id asc) */
            int32_t *ti = idx + (size_t)m * topk;
            double *tv = (double *)malloc(sizeof(double) * (size_t)topk);
            int cnt = 0;
            double best = -INFINITY, second = -INFINITY;
            int besti = -1;
            for (int v = 0; v < N; ++v) {
                const double x = lg[v];
                if (x > best) { second = best; best = x; besti = v; }
                else if (x > second) { second = x; }
                /* ids arrive ascending, so an equal value never displaces */
                int pos = cnt;
                while (pos > 0 && x > tv[pos - 1]) --pos;
                if (pos < topk) {
                    const int last = (cnt < topk) ? cnt : topk - 1;
                    for (int s2 = last; s2 > pos; --s2) { tv[s2] = tv[s2 - 1]; ti[s2] = ti[s2 - 1]; }
                    tv[pos] = x; ti[pos] = v;
                    if (cnt < topk) ++cnt;
                }
            }
            (void)besti;
            if (val) for (int s2 = 0; s2 < topk; ++s2) val[(size_t)m * topk + s2] = tv[s2];
            if (gap) gap[m] = (N > 1) ? best - second : INFINITY;
            if (lse) {
                double sum = 0.0;
                for (int v = 0; v < N; ++v) sum += exp(lg[v] - best);
                lse[m] = best + log(sum);
            }
            free(tv);
        }
    }
    free(logit);
    free(hrow);
}

/* ------------------------------------------------------------ O5: acceptance
 * Greedy acceptance ([lesson] "Verify-accept semantics"): along a draft
 * sequence, a draft token is accepted when it equals the target's argmax
 * given the tokens before it; scanning stops at the first miss and the
 * target's own token at that point is appended. On a tree this is applied to
 * every root-to-leaf path, brute force:
 *   for each leaf (ascending), path n_0 = root, n_1, ..., n_d:
 *     a = largest i with tok[n_j] == idx[n_{j-1}] for all 1 <= j <= i;
 *     candidate (a, n_a).
 *   a* = max a; end = lowest node index among candidates with a == a*
 *   (reading: equal-length accepted paths emit the same tokens; the lowest
 *   index fixes which node is reported).
 *   accept_len = a*; path = n_0..n_a* (-1 padded to T);
 *   out_tokens = tok[n_1..n_a*] then idx[end]  (a* + 1 tokens, -1 padded).
 * The root's own token is the last committed one and is never emitted.
 */
int orc_accept(const int32_t *tokens, const int32_t *parent, const int32_t *target_idx, int B, int T,
               int32_t *accept_len, int32_t *path, int32_t *out_tokens, int32_t *end_node) {
    int32_t *chain = (int32_t *)malloc(sizeof(int32_t) * (size_t)T);
    char *has_child = (char *)malloc((size_t)T);
    for (int b = 0; b < B; ++b) {
        const int32_t *par = parent + (size_t)b * T;
        const int32_t *tok = tokens + (size_t)b * T;
        const int32_t *tgt = target_idx + (size_t)b * T;
        if (orc_tree_check(par, T) != ORC_OK) { free(chain); free(has_child); return ORC_ERR_TREE; }
        memset(has_child, 0, (size_t)T);
        for (int n = 1; n < T; ++n) has_child[par[n]] = 1;
        int best_a = -1, best_end = 0;
        for (int leaf = 0; leaf < T; ++leaf) {
            if (has_child[leaf]) continue;
            int len = 0;
            for (int n = leaf; n >= 0; n = par[n]) chain[len++] = n;
            /* chain[len-1] = root ... chain[0] = leaf; n_i = chain[len-1-i] */
            int a = 0;
            while (a + 1 < len) {
                const int child = chain[len - 2 - a], prev = chain[len - 1 - a];
                if (tok[child] != tgt[prev]) break;
                ++a;
            }
            const int na = chain[len - 1 - a];
            if (a > best_a || (a == best_a && na < best_end)) { best_a = a; best_end = na; }
        }
        int32_t *pth = path + (size_t)b * T;
        int32_t *out = out_tokens + (size_t)b * T;
        for (int t = 0; t < T; ++t) { pth[t] = -1; out[t] = -1; }
        int len = 0;
        for (int n = best_end; n >= 0; n = par[n]) chain[len++] = n;
        for (int i = 0; i < len; ++i) pth[i] = chain[len - 1 - i];
        for (int i = 1; i < len; ++i) out[i - 1] = tok[pth[i]];
        out[len - 1] = tgt[best_end];
        accept_len[b] = best_a;
        if (end_node) end_node[b] = best_end;
    }
    free(chain); free(has_child);
    return ORC_OK;
}

/* ------------------------------------------------------------ dense layers
 * C[m][n] = sum_k A[m][k] * Bm[n][k] (k ascending) (+ R[m][n]), rounded once.
 * A row-major [M,K], Bm output-major [N,K] (the layout of every weight here).
 */
void orc_gemm(int dtype, const void *A, const void *Bm, const void *R, int M, int N, int K, void *C) {
#pragma omp parallel
    {
        double *arow = (double *)malloc(sizeof(double) * (size_t)K);
        double *brow = (double *)malloc(sizeof(double) * (size_t)K);
#pragma omp for schedule(static)
        for (long r = 0; r < (long)M * N; ++r) {
            const int m = (int)(r / N), n = (int)(r % N);
            ld_row(A, dtype, (size_t)m * K, K, arow);
            ld_row(Bm, dtype, (size_t)n * K, K, brow);
            double acc = 0.0;
            for (int k = 0; k < K; ++k) acc += arow[k] * brow[k];
            if (R) acc += ld(R, dtype, (size_t)m * N + n);
            st(C, dtype, (size_t)m * N + n, acc);
        }
        free(arow); free(brow);
    }
}

/* SwiGLU feed-forward input: with Wgu = [Wg; Wu] ([2F,K]),
 * y[m][f] = silu(g) * u, g = x.Wg[f], u = x.Wu[f] (each k ascending, not
 * rounded), silu(g) = g / (1 + exp(-g)). reading: Llama's MLP. */
void orc_swiglu(int dtype, const void *X, const void *Wgu, int M, int F, int K, void *Y) {
#pragma omp parallel
    {
        double *xr = (double *)malloc(sizeof(double) * (size_t)K);
        double *wr = (double *)malloc(sizeof(double) * (size_t)K);
#pragma omp for schedule(static)
        for (long r = 0; r < (long)M * F; ++r) {
            const int m = (int)(r / F), f = (int)(r % F);
            ld_row(X, dtype, (size_t)m * K, K, xr);
            double g = 0.0, u = 0.0;
            ld_row(Wgu, dtype, (size_t)f * K, K, wr);
            for (int k = 0; k < K; ++k) g += xr[k] * wr[k];
            ld_row(Wgu, dtype, (size_t)(F + f) * K, K, wr);
            for (int k = 0; k < K; ++k) u += xr[k] * wr[k];
            st(Y, dtype, (size_t)m * F + f, g / (1.0 + exp(-g)) * u);
        }
        free(xr); free(wr);
    }
}

/* SwiGLU gating on a stored gate/up product: gu is [M, 2F] (gate columns
 * first); y[m][f] = silu(g) * u with silu(g) = g / (1 + exp(-g)). */
void orc_silu_mul(int dtype, const void *GU, int M, int F, void *Y) {
#pragma omp parallel for schedule(static)
    for (long r = 0; r < (long)M * F; ++r) {
        const int m = (int)(r / F), f = (int)(r % F);
        const double g = ld(GU, dtype, (size_t)m * 2 * F + f), u = ld(GU, dtype, (size_t)m * 2 * F + F + f);
        st(Y, dtype, (size_t)r, g / (1.0 + exp(-g)) * u);
    }
}

/* Rotary embedding, rotate-half convention (reading: Llama's): for head
 * vector x[0..D) at position p, pair i with i + D/2, angle = p * theta^(-2i/D):
 *   x'[i] = x[i] cos - x[i+D/2] sin;  x'[i+D/2] = x[i+D/2] cos + x[i] sin.
 * x is [M, H, D] in place, pos[m] the position of row m. */
void orc_rope(int dtype, void *x, const int32_t *pos, int M, int H, int D, double theta) {
    const int half = D / 2;
#pragma omp parallel for schedule(static)
    for (long r = 0; r < (long)M * H; ++r) {
        const int m = (int)(r / H);
        const size_t base = (size_t)r * D;
        for (int i = 0; i < half; ++i) {
            const double ang = (double)pos[m] * pow(theta, -2.0 * i / D);
            const double c = cos(ang), s = sin(ang);
            const double a = ld(x, dtype, base + i), bb = ld(x, dtype, base + i + half);
            st(x, dtype, base + i, a * c - bb * s);
            st(x, dtype, base + i + half, bb * c + a * s);
        }
    }
}

/* rows of a table: out[m] = E[ids[m]] (copied, same type) */
void orc_embed(int dtype, const void *E, const int32_t *ids, int M, int K, void *out) {
    for (int m = 0; m < M; ++m)
        for (int k = 0; k < K; ++k)
            st(out, dtype, (size_t)m * K + k, ld(E, dtype, (size_t)ids[m] * K + k));
}

/* ------------------------------------------------------------ draft fusion
 * [news] draft stage: the low, mid and high features l, m, h (k each) are
 * concatenated to 3k and reduced to k by one FC, giving g; g (or, from step 2
 * on, the draft's own output a of the parent) is concatenated with the
 * embedding of the token one step ahead and reduced to k by a second FC.
 *   context mode (a_prev == NULL): g = Wf . [l; m; h];  x = Wi . [g; E[tok]]
 *   step mode    (l = m = h = NULL): x = Wi . [a_prev; E[tok]]
 * Wf is [k, 3k], Wi is [k, 2k] (output-major). g is rounded to the storage
 * type before the second FC (it is an FC output); dots run k ascending over
 * the concatenation. g_out may be NULL.
 */
void orc_draft_fuse(int dtype, const void *l, const void *mf, const void *hf, const void *a_prev,
                    const int32_t *tok, const void *E, const void *Wf, const void *Wi,
                    int M, int k, void *g_out, void *x_out) {
#pragma omp parallel
    {
        double *cat = (double *)malloc(sizeof(double) * (size_t)3 * k);
        double *wr = (double *)malloc(sizeof(double) * (size_t)3 * k);
        double *g = (double *)malloc(sizeof(double) * (size_t)k);
#pragma omp for schedule(static)
        for (int r = 0; r < M; ++r) {
            if (a_prev == NULL) {
                ld_row(l, dtype, (size_t)r * k, k, cat);
                ld_row(mf, dtype, (size_t)r * k, k, cat + k);
                ld_row(hf, dtype, (size_t)r * k, k, cat + 2 * k);
                for (int n = 0; n < k; ++n) {
                    ld_row(Wf, dtype, (size_t)n * 3 * k, 3 * k, wr);
                    double acc = 0.0;
                    for (int j = 0; j < 3 * k; ++j) acc += cat[j] * wr[j];
                    /* round to storage, as the stored g would be */
                    if (dtype == ORC_F32) g[n] = (double)(float)acc;
                    else { uint32_t u = (uint32_t)to_bf16(acc) << 16; float f; memcpy(&f, &u, 4); g[n] = f; }
                    if (g_out) st(g_out, dtype, (size_t)r * k + n, acc);
                }
                for (int n = 0; n < k; ++n) cat[n] = g[n];
            } else {
                ld_row(a_prev, dtype, (size_t)r * k, k, cat);
            }
            ld_row(E, dtype, (size_t)tok[r] * k, k, cat + k);
            for (int n = 0; n < k; ++n) {
                ld_row(Wi, dtype, (size_t)n * 2 * k, 2 * k, wr);
                double acc = 0.0;
                for (int j = 0; j < 2 * k; ++j) acc += cat[j] * wr[j];
                st(x_out, dtype, (size_t)r * k + n, acc);
            }
        }
        free(cat); free(wr); free(g);
    }
}

/* ------------------------------------------------------------ tree selection
 * Draft-tree growth (EAGLE-2 style, the news write-up: the draft's confidence
 * stands in for acceptance and shapes the tree). reading: candidates are
 * ranked by (score descending, creation index ascending); score(child) =
 * fp32(score(parent) + logp(child)) where logp is the draft's fp32 log-prob.
 *
 * orc_select_topk: for each of B independent lists of n entries (score, id),
 * return the positions of the top `k` entries under that order, in that order.
 */
void orc_select_topk(const float *score, const int32_t *order_id, int B, int n, int k, int32_t *sel) {
    for (int b = 0; b < B; ++b) {
        const float *s = score + (size_t)b * n;
        const int32_t *id = order_id + (size_t)b * n;
        int32_t *o = sel + (size_t)b * k;
        char *used = (char *)calloc((size_t)n, 1);
        for (int r = 0; r < k; ++r) {
            int best = -1;
            for (int i = 0; i < n; ++i) {
                if (used[i]) continue;
                if (best < 0 || s[i] > s[best] || (s[i] == s[best] && id[i] < id[best])) best = i;
            }
            o[r] = best;
            if (best >= 0) used[best] = 1;
        }
        free(used);
    }
}
