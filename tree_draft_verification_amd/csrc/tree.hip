// Tree bookkeeping on the GPU: ancestor masks and greedy acceptance.
//
// Both kernels give one 64-lane wavefront to one sequence; a lane owns nodes
// lane and lane + 64 (T <= 128). The ancestor relation follows the course
// lesson "EAGLE-3 speculative decoding: the tree-verifier method", section
// "Tree draft vs chain draft" (a node sees only its ancestors; reading: and
// itself). Acceptance follows its section "Verify-accept semantics" applied to
// every root-to-leaf path at once.
#include "common.h"

namespace {

constexpr int kMaxT = 128;

// bit test / set on a W-word mask held in registers
template <int W>
__device__ __forceinline__ void set_bit(uint64_t (&m)[W], int t) {
#pragma unroll
    for (int w = 0; w < W; ++w)
        if (t / 64 == w) m[w] |= (uint64_t)1 << (t % 64);
}

// Walk n's parent chain (bounded by T steps; stops on an out-of-range parent).
template <int W>
__device__ __forceinline__ int walk_ancestors(const int32_t *par, int T, int n, uint64_t (&m)[W]) {
#pragma unroll
    for (int w = 0; w < W; ++w) m[w] = 0;
    int d = -1, cur = n;
    for (int steps = 0; steps < T && cur >= 0 && cur < T; ++steps) {
        set_bit<W>(m, cur);
        ++d;
        cur = par[cur];
    }
    return d;
}

template <int W>
__global__ __launch_bounds__(64) void tree_mask_kernel(const int32_t *__restrict__ parent, int T,
                                                       uint64_t *__restrict__ mask, int32_t *__restrict__ depth,
                                                       int32_t *__restrict__ status) {
    __shared__ int32_t par[kMaxT];
    const int b = blockIdx.x, lane = threadIdx.x;
    bool bad = false;
    for (int n = lane; n < T; n += 64) {
        const int p = parent[(size_t)b * T + n];
        par[n] = p;
        bad |= (n == 0) ? (p != -1) : (p < 0 || p >= n);
    }
    __syncthreads();
    bad = __any(bad);
    for (int n = lane; n < T; n += 64) {
        uint64_t m[W];
        const int d = walk_ancestors<W>(par, T, n, m);
#pragma unroll
        for (int w = 0; w < W; ++w) mask[((size_t)b * T + n) * W + w] = m[w];
        if (depth) depth[(size_t)b * T + n] = d;
    }
    if (status && lane == 0) status[b] = bad ? EAGLE3_ERR_TREE : EAGLE3_OK;
}

// Greedy acceptance. ok(n) = tokens[n] == target[parent(n)] (root: true);
// accepted(n) = ok on every node of n's ancestor set (one AND-NOT against the
// wave's ballot of ok bits); end = deepest accepted node, lowest index on ties.
template <int W>
__global__ __launch_bounds__(64) void accept_kernel(const int32_t *__restrict__ tokens,
                                                    const int32_t *__restrict__ parent,
                                                    const uint64_t *__restrict__ mask,
                                                    const int32_t *__restrict__ target, int T,
                                                    int32_t *__restrict__ accept_len, int32_t *__restrict__ path,
                                                    int32_t *__restrict__ out_tokens, int V,
                                                    int32_t *__restrict__ status) {
    __shared__ int32_t par[kMaxT];
    __shared__ int32_t tgt[kMaxT];
    __shared__ int32_t tok[kMaxT];
    __shared__ int32_t slot[kMaxT];
    const int b = blockIdx.x, lane = threadIdx.x;
    const size_t row = (size_t)b * T;
    bool range_bad = false, tree_bad = false;
    for (int n = lane; n < T; n += 64) {
        tgt[n] = target[row + n];
        tok[n] = tokens[row + n];
        if (parent) par[n] = parent[row + n];
        slot[n] = -1;
        if (status) {
            // validate mode: every token and target id a vocabulary id; a
            // parent[] given in topological order with the root first
            range_bad |= tok[n] < 0 || tok[n] >= V || tgt[n] < 0 || tgt[n] >= V;
            if (parent) tree_bad |= n == 0 ? par[n] != -1 : (par[n] < 0 || par[n] >= n);
        }
    }
    if (status) {
        const bool rb = __ballot(range_bad) != 0, tb = __ballot(tree_bad) != 0;
        if (lane == 0) status[b] = tb ? EAGLE3_ERR_TREE : rb ? EAGLE3_ERR_RANGE : EAGLE3_OK;
    }
    __syncthreads();

    constexpr int NPL = W;  // nodes per lane (W words cover 64 * W nodes)
    uint64_t anc[NPL][W];
    int pidx[NPL];
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
        const int n = lane + 64 * j;
#pragma unroll
        for (int w = 0; w < W; ++w) anc[j][w] = 0;
        pidx[j] = -1;
        if (n < T) {
            if (mask) {
#pragma unroll
                for (int w = 0; w < W; ++w) anc[j][w] = mask[(row + n) * W + w];
                // parent = highest ancestor index below n
                uint64_t m2[W];
#pragma unroll
                for (int w = 0; w < W; ++w) m2[w] = anc[j][w];
#pragma unroll
                for (int w = 0; w < W; ++w)
                    if (w == n / 64) m2[w] &= ~((uint64_t)1 << (n % 64));
#pragma unroll
                for (int w = W - 1; w >= 0; --w)
                    if (pidx[j] < 0 && m2[w]) pidx[j] = 64 * w + 63 - __clzll(m2[w]);
            } else {
                walk_ancestors<W>(par, T, n, anc[j]);
                pidx[j] = par[n];
            }
        }
    }
    // ok bits, one ballot per mask word
    uint64_t okw[W];
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
        const int n = lane + 64 * j;
        bool ok = false;
        if (n < T) ok = (n == 0) || (pidx[j] >= 0 && pidx[j] < T && tok[n] == tgt[pidx[j]]);
        okw[j] = __ballot(ok);
    }
    // best = max over accepted nodes of (depth, -index)
    int best = -1;
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
        const int n = lane + 64 * j;
        if (n >= T) continue;
        bool accepted = true;
        int depth = -1;
#pragma unroll
        for (int w = 0; w < W; ++w) {
            accepted &= (anc[j][w] & ~okw[w]) == 0;
            depth += __popcll(anc[j][w]);
        }
        if (accepted) best = max(best, (depth << 8) | (255 - n));
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) best = max(best, __shfl_xor(best, off));
    const int a = best >> 8;
    const int end = 255 - (best & 255);
    // path = ancestors of end, ascending index (= root first: parent < child),
    // taken from the lane that holds node end (end is wave-uniform)
    uint64_t aend[W];
#pragma unroll
    for (int w = 0; w < W; ++w) {
        aend[w] = 0;
#pragma unroll
        for (int j = 0; j < NPL; ++j)
            if (j == (end >> 6)) {
                const uint32_t lo = __shfl((uint32_t)anc[j][w], end & 63);
                const uint32_t hi = __shfl((uint32_t)(anc[j][w] >> 32), end & 63);
                aend[w] = ((uint64_t)hi << 32) | lo;
            }
    }
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
        const int n = lane + 64 * j;
        if (n >= T) continue;
        bool on_path = false;
#pragma unroll
        for (int w = 0; w < W; ++w)
            if (w == n / 64) on_path = (aend[w] >> (n % 64)) & 1u;
        if (on_path) {
            int rank = 0;
#pragma unroll
            for (int w = 0; w < W; ++w) {
                if (w < n / 64) rank += __popcll(aend[w]);
                else if (w == n / 64) rank += __popcll(aend[w] & (((uint64_t)1 << (n % 64)) - 1));
            }
            if (rank < T) slot[rank] = n;
        }
    }
    __syncthreads();
    for (int i = lane; i < T; i += 64) {
        const int n = (i <= a) ? slot[i] : -1;
        path[row + i] = n;
        int o = -1;
        if (i < a) {
            const int nn = slot[i + 1];
            o = (nn >= 0) ? tok[nn] : -1;
        } else if (i == a) {
            o = tgt[end];
        }
        out_tokens[row + i] = o;
    }
    if (lane == 0) accept_len[b] = a;
}

// Trimmed draft vocabulary: row i of the trimmed LM head is full-vocabulary id
// vmap[i]. One work-group walks the list (a draft step maps a few thousand
// ids); an id outside [0, V_sub) becomes -1 and sets the flag.
__global__ __launch_bounds__(1024) void vocab_map_kernel(const int32_t *__restrict__ ids, int n,
                                                         const int32_t *__restrict__ vmap, int V_sub,
                                                         int32_t *__restrict__ out, int32_t *__restrict__ status) {
    __shared__ int bad_any;
    if (threadIdx.x == 0) bad_any = 0;
    __syncthreads();
    bool bad = false;
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
        const int r = ids[i];
        const bool ok = r >= 0 && r < V_sub;
        out[i] = ok ? vmap[r] : -1;
        bad |= !ok;
    }
    if (__ballot(bad) != 0 && (threadIdx.x & 63) == 0) bad_any = 1;
    __syncthreads();
    if (status && threadIdx.x == 0) status[0] = bad_any ? EAGLE3_ERR_RANGE : EAGLE3_OK;
}

// Position of every tree node: the sequence's cached length plus the node's
// depth (the root, the last emitted token, is not cached yet and takes the
// first free position).
__global__ __launch_bounds__(256) void node_positions_kernel(const int32_t *__restrict__ prefix_len,
                                                             const int32_t *__restrict__ depth, int B, int T,
                                                             int32_t *__restrict__ pos) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= B * T) return;
    pos[i] = prefix_len[i / T] + depth[i];
}

// Bookkeeping after acceptance, one wave per sequence: the accepted rows
// (root, accepted drafts) become the next context rows, the sequence length
// grows by accept_len + 1, the target's token at the end node is the next
// root, and the emitted tokens are appended.
__global__ __launch_bounds__(64) void spec_advance_kernel(
    const int32_t *__restrict__ accept_len, const int32_t *__restrict__ path, const int32_t *__restrict__ out_tokens,
    int T, int R, int32_t *__restrict__ prefix_len, int32_t *__restrict__ start, int32_t *__restrict__ path_rows,
    int32_t *__restrict__ tok_ahead, int32_t *__restrict__ last_rows, int32_t *__restrict__ root,
    int32_t *__restrict__ out_seq, int32_t *__restrict__ out_len, int cap) {
    const int b = blockIdx.x, lane = threadIdx.x;
    const size_t row = (size_t)b * T;
    const int a = min(max(accept_len[b], 0), min(T, R) - 1);
    const int P = prefix_len[b];
    const int n0 = out_len ? out_len[b] : 0;
    for (int j = lane; j < R; j += 64) {
        const bool ok = j <= a;
        path_rows[(size_t)b * R + j] = ok ? (int)row + path[row + j] : -1;
        tok_ahead[(size_t)b * R + j] = ok ? out_tokens[row + j] : 0;
        if (out_seq && ok && n0 + j < cap) out_seq[(size_t)b * cap + n0 + j] = out_tokens[row + j];
    }
    __syncthreads();
    if (lane == 0) {
        start[b] = P;
        prefix_len[b] = P + a + 1;
        last_rows[b] = b * R + a;
        root[b] = out_tokens[row + a];
        if (out_len) out_len[b] = n0 + a + 1;
    }
}

}  // namespace

extern "C" int eagle3_tree_mask(const int32_t *parent, int B, int T, int W, uint64_t *mask, int32_t *depth,
                                int32_t *status, void *stream) {
    if (B < 0 || T < 1) return EAGLE3_ERR_ARG;
    if (W < 1 || W > 2 || T > 64 * W) return EAGLE3_ERR_UNSUPPORTED;
    if (B == 0) return EAGLE3_OK;
    if (!parent || !mask) return EAGLE3_ERR_ARG;
    if (W == 1)
        tree_mask_kernel<1><<<B, 64, 0, e3_stream(stream)>>>(parent, T, mask, depth, status);
    else
        tree_mask_kernel<2><<<B, 64, 0, e3_stream(stream)>>>(parent, T, mask, depth, status);
    E3_LAUNCH_CHECK();
    return EAGLE3_OK;
}

extern "C" int eagle3_accept_path(const int32_t *tokens, const int32_t *parent, const uint64_t *mask, int W,
                                  const int32_t *target_idx, int B, int T, int32_t *accept_len, int32_t *path,
                                  int32_t *out_tokens, int V, int32_t *status, void *stream) {
    if (B < 0 || T < 1) return EAGLE3_ERR_ARG;
    if (W < 1 || W > 2 || T > 64 * W) return EAGLE3_ERR_UNSUPPORTED;
    if (status && V < 1) return EAGLE3_ERR_ARG;
    if (B == 0) return EAGLE3_OK;
    if (!tokens || !target_idx || !accept_len || !path || !out_tokens) return EAGLE3_ERR_ARG;
    if ((parent == nullptr) == (mask == nullptr)) return EAGLE3_ERR_ARG;
    if (W == 1)
        accept_kernel<1><<<B, 64, 0, e3_stream(stream)>>>(tokens, parent, mask, target_idx, T, accept_len, path,
                                                         out_tokens, V, status);
    else
        accept_kernel<2><<<B, 64, 0, e3_stream(stream)>>>(tokens, parent, mask, target_idx, T, accept_len, path,
                                                         out_tokens, V, status);
    E3_LAUNCH_CHECK();
    return EAGLE3_OK;
}

extern "C" int eagle3_vocab_map(const int32_t *ids, int n, const int32_t *vmap, int V_sub, int32_t *out,
                                int32_t *status, void *stream) {
    if (n < 0 || V_sub < 1) return EAGLE3_ERR_ARG;
    if (n == 0 && !status) return EAGLE3_OK;
    if ((n > 0 && (!ids || !out)) || !vmap) return EAGLE3_ERR_ARG;
    vocab_map_kernel<<<1, 1024, 0, e3_stream(stream)>>>(ids, n, vmap, V_sub, out, status);
    E3_LAUNCH_CHECK();
    return EAGLE3_OK;
}

extern "C" int eagle3_node_positions(const int32_t *prefix_len, const int32_t *depth, int B, int T, int32_t *pos,
                                     void *stream) {
    if (B < 0 || T < 1 || (long)B * T > 0x7fffffffL) return EAGLE3_ERR_ARG;
    if (B == 0) return EAGLE3_OK;
    if (!prefix_len || !depth || !pos) return EAGLE3_ERR_ARG;
    const int n = B * T;
    node_positions_kernel<<<(n + 255) / 256, 256, 0, e3_stream(stream)>>>(prefix_len, depth, B, T, pos);
    E3_LAUNCH_CHECK();
    return EAGLE3_OK;
}

extern "C" int eagle3_spec_advance(const int32_t *accept_len, const int32_t *path, const int32_t *out_tokens, int B,
                                   int T, int R, int32_t *prefix_len, int32_t *start, int32_t *path_rows,
                                   int32_t *tok_ahead, int32_t *last_rows, int32_t *root, int32_t *out_seq,
                                   int32_t *out_len, int cap, void *stream) {
    if (B < 0 || T < 1 || R < 1 || (long)B * T > 0x7fffffffL || (long)B * R > 0x7fffffffL) return EAGLE3_ERR_ARG;
    if (out_seq && (!out_len || cap < 1)) return EAGLE3_ERR_ARG;
    if (B == 0) return EAGLE3_OK;
    if (!accept_len || !path || !out_tokens || !prefix_len || !start || !path_rows || !tok_ahead || !last_rows ||
        !root)
        return EAGLE3_ERR_ARG;
    spec_advance_kernel<<<B, 64, 0, e3_stream(stream)>>>(accept_len, path, out_tokens, T, R, prefix_len, start,
                                                         path_rows, tok_ahead, last_rows, root, out_seq, out_len,
                                                         cap);
    E3_LAUNCH_CHECK();
    return EAGLE3_OK;
}
