// Draft-tree growth (EAGLE-2 style, news write-up of the EAGLE-3 paper: the
// draft's confidence stands in for the acceptance rate and shapes the tree;
// parameters from the Spec-Bench blog post's inference table: top-k 10,
// 60 draft tokens). reading: a candidate's score is fp32(score(parent) +
// logp(candidate)); selections rank by (score descending, creation index
// ascending); every candidate ever drafted stays in the pool.
//
// Both kernels give one work-group to one sequence and rank by counting, so
// the result does not depend on thread timing.
#include "common.h"

namespace {

__device__ __forceinline__ bool ahead(float sa, int ca, float sb, int cb) {
    return sa > sb || (sa == sb && ca < cb);
}

// One expansion: F frontier nodes x C children -> F*C new pool entries
// (creation order: frontier slot major, child minor) and the next frontier
// (top NF of the new candidates).
__global__ __launch_bounds__(256) void tree_expand_kernel(
    const float *__restrict__ fr_score, const int32_t *__restrict__ fr_pool, const uint64_t *__restrict__ fr_mask,
    int fr_arow_base, int arow_stride, const int32_t *__restrict__ child_ids, const float *__restrict__ child_val,
    const float *__restrict__ child_lse, int F, int C, int NF, int pool_len, int pool_cap, int row_base,
    float *__restrict__ pool_score,
    int32_t *__restrict__ pool_token, int32_t *__restrict__ pool_parent, int32_t *__restrict__ next_pool,
    float *__restrict__ next_score, int32_t *__restrict__ next_token, uint64_t *__restrict__ next_mask,
    int32_t *__restrict__ next_arow) {
    __shared__ float sc[256];
    const int b = blockIdx.x, t = threadIdx.x;
    const int n = F * C;
    float s = 0.f;
    if (t < n) {
        const int f = t / C;
        // log-probability of the child under its parent's draft distribution
        float lp = child_val[((size_t)b * F + f) * C + (t % C)];
        if (child_lse) lp -= child_lse[b * F + f];
        s = fr_score[b * F + f] + lp;  // fp32 add
        sc[t] = s;
        const int slot = pool_len + t;
        if (slot < pool_cap) {
            pool_score[(size_t)b * pool_cap + slot] = s;
            pool_token[(size_t)b * pool_cap + slot] = child_ids[((size_t)b * F + f) * C + (t % C)];
            pool_parent[(size_t)b * pool_cap + slot] = fr_pool[b * F + f];
        }
    }
    __syncthreads();
    if (t < n) {
        int rank = 0;
        for (int u = 0; u < n; ++u) rank += ahead(sc[u], u, s, t);
        if (rank < NF) {
            const int f = t / C;
            const int out = b * NF + rank;
            next_pool[out] = pool_len + t;
            next_score[out] = s;
            next_token[out] = child_ids[((size_t)b * F + f) * C + (t % C)];
            // draft rows visible to this node: its ancestors' rows and its own
            const int row = row_base + rank;
            const uint64_t *pm = fr_mask + ((size_t)b * F + f) * 2;
            next_mask[(size_t)out * 2] = pm[0] | (row < 64 ? (uint64_t)1 << row : 0);
            next_mask[(size_t)out * 2 + 1] = pm[1] | (row >= 64 && row < 128 ? (uint64_t)1 << (row - 64) : 0);
            // the draft row holding this node's parent's output (the parent is frontier slot f)
            next_arow[out] = b * arow_stride + fr_arow_base + f;
        }
    }
}

// Pool -> top N by (score desc, creation asc) -> creation order -> parent[N+1],
// tokens[N+1] with the root (the last committed token) as node 0.
__global__ __launch_bounds__(256) void tree_rerank_kernel(const float *__restrict__ pool_score,
                                                          const int32_t *__restrict__ pool_token,
                                                          const int32_t *__restrict__ pool_parent, int pool_len,
                                                          int pool_cap, int N, const int32_t *__restrict__ root_token,
                                                          int32_t *__restrict__ parent, int32_t *__restrict__ tokens) {
    extern __shared__ unsigned char smem[];
    float *sc = reinterpret_cast<float *>(smem);
    int *sel = reinterpret_cast<int *>(sc + pool_len);  // 1 if among the top N
    int *nid = sel + pool_len;                           // new node index of a selected entry, else -1
    const int b = blockIdx.x;
    const float *ps = pool_score + (size_t)b * pool_cap;
    for (int i = threadIdx.x; i < pool_len; i += blockDim.x) sc[i] = ps[i];
    __syncthreads();
    for (int i = threadIdx.x; i < pool_len; i += blockDim.x) {
        int rank = 0;
        for (int u = 0; u < pool_len; ++u) rank += ahead(sc[u], u, sc[i], i);
        sel[i] = rank < N ? 1 : 0;
    }
    __syncthreads();
    // new index = 1 + number of selected entries created earlier
    for (int i = threadIdx.x; i < pool_len; i += blockDim.x) {
        int idx = -1;
        if (sel[i]) {
            idx = 1;
            for (int u = 0; u < i; ++u) idx += sel[u];
        }
        nid[i] = idx;
    }
    __syncthreads();
    int32_t *par = parent + (size_t)b * (N + 1);
    int32_t *tok = tokens + (size_t)b * (N + 1);
    if (threadIdx.x == 0) { par[0] = -1; tok[0] = root_token[b]; }
    for (int i = threadIdx.x; i < pool_len; i += blockDim.x) {
        const int ni = nid[i];
        if (ni > 0 && ni <= N) {
            const int pp = pool_parent[(size_t)b * pool_cap + i];
            const int np = pp < 0 ? 0 : nid[min(max(pp, 0), pool_len - 1)];
            par[ni] = np < 0 ? 0 : np;
            tok[ni] = pool_token[(size_t)b * pool_cap + i];
        }
    }
}

}  // namespace

extern "C" int eagle3_tree_expand(const float *fr_score, const int32_t *fr_pool, const uint64_t *fr_mask,
                                  int fr_arow_base, int arow_stride, const int32_t *child_ids, const float *child_val,
                                  const float *child_lse, int B, int F, int C, int NF, int pool_len, int pool_cap,
                                  int row_base,
                                  float *pool_score, int32_t *pool_token, int32_t *pool_parent, int32_t *next_pool,
                                  float *next_score, int32_t *next_token, uint64_t *next_mask, int32_t *next_arow,
                                  void *stream) {
    if (B < 0 || F < 1 || C < 1 || NF < 1 || pool_len < 0 || pool_cap < 1 || row_base < 0 || fr_arow_base < 0 ||
        arow_stride < 1)
        return EAGLE3_ERR_ARG;
    if (F * C > 256 || NF > F * C || row_base + NF > 128) return EAGLE3_ERR_UNSUPPORTED;
    if (pool_len + F * C > pool_cap) return EAGLE3_ERR_ARG;
    if (B == 0) return EAGLE3_OK;
    if (!fr_score || !fr_pool || !fr_mask || !child_ids || !child_val || !pool_score || !pool_token ||
        !pool_parent || !next_pool || !next_score || !next_token || !next_mask || !next_arow)
        return EAGLE3_ERR_ARG;
    tree_expand_kernel<<<B, 256, 0, e3_stream(stream)>>>(fr_score, fr_pool, fr_mask, fr_arow_base, arow_stride,
                                                        child_ids, child_val, child_lse, F, C, NF, pool_len, pool_cap,
                                                        row_base,
                                                        pool_score, pool_token, pool_parent, next_pool, next_score,
                                                        next_token, next_mask, next_arow);
    E3_LAUNCH_CHECK();
    return EAGLE3_OK;
}

extern "C" int eagle3_tree_rerank(const float *pool_score, const int32_t *pool_token, const int32_t *pool_parent,
                                  int B, int pool_len, int pool_cap, int N, const int32_t *root_token,
                                  int32_t *parent, int32_t *tokens, void *stream) {
    if (B < 0 || pool_len < 1 || pool_cap < pool_len || N < 1) return EAGLE3_ERR_ARG;
    if (N > pool_len || pool_len > 4096) return EAGLE3_ERR_UNSUPPORTED;
    if (B == 0) return EAGLE3_OK;
    if (!pool_score || !pool_token || !pool_parent || !root_token || !parent || !tokens) return EAGLE3_ERR_ARG;
    const size_t shm = (size_t)pool_len * (sizeof(float) + 2 * sizeof(int));
    tree_rerank_kernel<<<B, 256, shm, e3_stream(stream)>>>(pool_score, pool_token, pool_parent, pool_len, pool_cap, N,
                                                          root_token, parent, tokens);
    E3_LAUNCH_CHECK();
    return EAGLE3_OK;
}
