// LM head with a fused per-row top-k / gap / log-sum-exp; logits never reach
// memory. The target's argmax at every tree node decides acceptance (course
// lesson "EAGLE-3 speculative decoding: the tree-verifier method", section
// "Verify-accept semantics"); the draft head's top-k uses the same head (news
// write-up of the EAGLE-3 paper, draft-stage paragraphs).
//
// Pass 1 (one work-group per 256-row vocabulary tile x 64-row hidden tile):
//   bf16: MFMA 32x32x16. The vocabulary rows are the MFMA "row" operand and
//   the hidden rows the "column" operand, so every accumulator register of a
//   lane belongs to one hidden row: per-row selection needs no transposes.
//   Each lane streams 64 contiguous bytes of its weight row per 64-wide k
//   chunk (both operands use the same k permutation, so the contraction is
//   unchanged), two chunks in flight. fp32: plain FMA loop (small models).
//   The 64x256 logit tile is staged in LDS; 4 threads per row keep a sorted
//   top-KK list (value desc, id asc) and an online (max, sum exp) pair, then
//   merge by lane shuffles. One (list, max, sum) record per row and tile goes
//   to the workspace.
// Pass 2 (one work-group per row): merges the records of all tiles in a
//   fixed order -> deterministic results.
#include "common.h"

namespace {

constexpr int BN = 256;  // vocabulary rows per tile
constexpr int BK = 64;   // k per chunk (bf16 path)
constexpr int LDP = BN + 4;

struct Partials {
    float *val;  // [M, ntiles, KK]
    int *idx;    // [M, ntiles, KK]
    float *mx;   // [M, ntiles]
    float *se;   // [M, ntiles]
};

// Per-row selection over an LDS tile lg[BMt][LDP]; tpr threads per row.
template <int BMt, int KK, bool LSE>
__device__ __forceinline__ void tile_select(const float (*lg)[LDP], int m0, int M, int n0, int N, int tile, int ntiles,
                                            const Partials &p) {
    constexpr int TPR = 256 / BMt;
    constexpr int PER = BN / TPR;
    const int row = threadIdx.x / TPR, part = threadIdx.x % TPR;
    float lv[KK]; int li[KK];
    e3_topk_init<KK>(lv, li);
    float mx = -INFINITY, se = 0.f;
    const int vbeg = part * PER;
    for (int i = 0; i < PER; ++i) {
        const int vl = vbeg + i;
        const int v = n0 + vl;
        if (v >= N) break;
        const float x = lg[row][vl];
        if (e3_better(x, v, lv[KK - 1], li[KK - 1])) e3_topk_insert<KK>(lv, li, x, v);
        if (LSE) {
            if (x > mx) { se = se * __expf(mx - x) + 1.f; mx = x; }
            else se += __expf(x - mx);
        }
    }
#pragma unroll
    for (int off = 1; off < TPR; off <<= 1) {
        e3_topk_merge_xor<KK>(lv, li, off);
        if (LSE) {
            const float m2 = __shfl_xor(mx, off), s2 = __shfl_xor(se, off);
            e3_lse_combine(mx, se, m2, s2);
        }
    }
    const int m = m0 + row;
    if (part == 0 && m < M) {
        const size_t rec = (size_t)m * ntiles + tile;
#pragma unroll
        for (int s = 0; s < KK; ++s) { p.val[rec * KK + s] = lv[s]; p.idx[rec * KK + s] = li[s]; }
        if (LSE) { p.mx[rec] = mx; p.se[rec] = se; }
    }
}

template <int KK, bool LSE>
__global__ __launch_bounds__(256, 2) void lmhead_bf16_kernel(const uint16_t *__restrict__ h,
                                                             const uint16_t *__restrict__ w, int M, int N, int K,
                                                             int ntiles, Partials p) {
    constexpr int BM = 64;
    __shared__ float lg[BM][LDP];
    const int mt = blockIdx.x, tile = blockIdx.y;
    const int m0 = mt * BM, n0 = tile * BN;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int lr = lane & 31, lh = lane >> 5;

    const uint16_t *wrow[2];
    const uint16_t *hrow[2];
    bool hval[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        int v = n0 + wave * 64 + nb * 32 + lr;
        v = v < N ? v : N - 1;  // clamped rows are computed and ignored
        wrow[nb] = w + (size_t)v * K + lh * 32;
    }
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
        const int m = m0 + mb * 32 + lr;
        hval[mb] = m < M;
        hrow[mb] = h + (size_t)(m < M ? m : M - 1) * K + lh * 32;
    }

    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    u32x4_t a0[2][4], b0[2][4], a1[2][4], b1[2][4];
    const u32x4_t zero = {0u, 0u, 0u, 0u};

    auto load = [&](u32x4_t (&a)[2][4], u32x4_t (&b)[2][4], int kc) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int s = 0; s < 4; ++s) a[nb][s] = *reinterpret_cast<const u32x4_t *>(wrow[nb] + kc + 8 * s);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int s = 0; s < 4; ++s)
                b[mb][s] = hval[mb] ? *reinterpret_cast<const u32x4_t *>(hrow[mb] + kc + 8 * s) : zero;
    };
    auto compute = [&](const u32x4_t (&a)[2][4], const u32x4_t (&b)[2][4]) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
                    acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8_t, a[nb][s]), __builtin_bit_cast(bf16x8_t, b[mb][s]),
                        acc[nb][mb], 0, 0, 0);
    };

    load(a0, b0, 0);
    for (int kc = 0; kc < K; kc += 2 * BK) {
        if (kc + BK < K) load(a1, b1, kc + BK);
        compute(a0, b0);
        if (kc + 2 * BK < K) load(a0, b0, kc + 2 * BK);
        if (kc + BK < K) compute(a1, b1);
    }

    // D[vocab i][hidden j]: lane holds j = lr, i = 8*(r/4) + 4*lh + r%4
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                lg[mb * 32 + lr][wave * 64 + nb * 32 + 8 * (r >> 2) + 4 * lh + (r & 3)] = acc[nb][mb][r];
    __syncthreads();
    tile_select<BM, KK, LSE>(lg, m0, M, n0, N, tile, ntiles, p);
}

template <int KK, bool LSE>
__global__ __launch_bounds__(256) void lmhead_f32_kernel(const float *__restrict__ h, const float *__restrict__ w,
                                                         int M, int N, int K, int ntiles, Partials p) {
    constexpr int BM = 16;
    __shared__ float lg[BM][LDP];
    __shared__ float hs[BM][64];
    const int mt = blockIdx.x, tile = blockIdx.y;
    const int m0 = mt * BM, n0 = tile * BN;
    const int t = threadIdx.x;
    int v = n0 + t;
    v = v < N ? v : N - 1;
    const float *wr = w + (size_t)v * K;
    float acc[BM];
#pragma unroll
    for (int r = 0; r < BM; ++r) acc[r] = 0.f;
    for (int kc = 0; kc < K; kc += 64) {
        for (int e = t; e < BM * 64; e += 256) {
            const int r = e / 64, k = e % 64;
            const int m = m0 + r;
            hs[r][k] = (m < M && kc + k < K) ? h[(size_t)m * K + kc + k] : 0.f;
        }
        __syncthreads();
        const int kend = (K - kc) < 64 ? (K - kc) : 64;
        for (int k = 0; k < kend; ++k) {
            const float wv = wr[kc + k];
#pragma unroll
            for (int r = 0; r < BM; ++r) acc[r] = fmaf(hs[r][k], wv, acc[r]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int r = 0; r < BM; ++r) lg[r][t] = acc[r];
    __syncthreads();
    tile_select<BM, KK, LSE>(lg, m0, M, n0, N, tile, ntiles, p);
}

template <int KK, bool LSE>
__global__ __launch_bounds__(256) void lmhead_merge_kernel(int ntiles, Partials p, int topk, int32_t *__restrict__ idx,
                                                           float *__restrict__ val, float *__restrict__ gap,
                                                           float *__restrict__ lse) {
    __shared__ float sv[4][KK];
    __shared__ int si[4][KK];
    __shared__ float smx[4], sse[4];
    const int m = blockIdx.x;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    float lv[KK]; int li[KK];
    e3_topk_init<KK>(lv, li);
    float mx = -INFINITY, se = 0.f;
    for (int t = threadIdx.x; t < ntiles; t += 256) {
        const size_t rec = (size_t)m * ntiles + t;
#pragma unroll
        for (int s = 0; s < KK; ++s) e3_topk_insert<KK>(lv, li, p.val[rec * KK + s], p.idx[rec * KK + s]);
        if (LSE) e3_lse_combine(mx, se, p.mx[rec], p.se[rec]);
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        e3_topk_merge_xor<KK>(lv, li, off);
        if (LSE) {
            const float m2 = __shfl_xor(mx, off), s2 = __shfl_xor(se, off);
            e3_lse_combine(mx, se, m2, s2);
        }
    }
    if (lane == 0) {
#pragma unroll
        for (int s = 0; s < KK; ++s) { sv[wave][s] = lv[s]; si[wave][s] = li[s]; }
        smx[wave] = mx; sse[wave] = se;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int wv = 1; wv < 4; ++wv) {
#pragma unroll
            for (int s = 0; s < KK; ++s) e3_topk_insert<KK>(lv, li, sv[wv][s], si[wv][s]);
            if (LSE) e3_lse_combine(mx, se, smx[wv], sse[wv]);
        }
        for (int s = 0; s < topk; ++s) {
            idx[(size_t)m * topk + s] = li[s];
            if (val) val[(size_t)m * topk + s] = lv[s];
        }
        if (gap) gap[m] = lv[0] - lv[1];
        if (LSE) lse[m] = mx + __logf(se);
    }
}

int kk_for(int topk) {
    const int need = topk < 2 ? 2 : topk;
    return need <= 2 ? 2 : need <= 4 ? 4 : need <= 8 ? 8 : 16;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

Partials carve(void *ws, int M, int ntiles, int KK) {
    char *b = (char *)ws;
    const size_t rec = (size_t)M * ntiles;
    Partials p;
    p.val = (float *)b; b += align256(rec * KK * sizeof(float));
    p.idx = (int *)b;   b += align256(rec * KK * sizeof(int));
    p.mx = (float *)b;  b += align256(rec * sizeof(float));
    p.se = (float *)b;
    return p;
}

template <int KK, bool LSE>
void launch(const void *hidden, const void *w, int M, int N, int K, int topk, int dtype, int32_t *idx, float *val,
            float *gap, float *lse, void *ws, hipStream_t st) {
    const int ntiles = (N + BN - 1) / BN;
    const Partials p = carve(ws, M, ntiles, KK);
    if (dtype == EAGLE3_BF16) {
        dim3 grid((M + 63) / 64, ntiles);
        lmhead_bf16_kernel<KK, LSE><<<grid, 256, 0, st>>>((const uint16_t *)hidden, (const uint16_t *)w, M, N, K,
                                                          ntiles, p);
    } else {
        dim3 grid((M + 15) / 16, ntiles);
        lmhead_f32_kernel<KK, LSE><<<grid, 256, 0, st>>>((const float *)hidden, (const float *)w, M, N, K, ntiles, p);
    }
    lmhead_merge_kernel<KK, LSE><<<M, 256, 0, st>>>(ntiles, p, topk, idx, val, gap, lse);
}

template <int KK>
void launch_kk(bool want_lse, const void *hidden, const void *w, int M, int N, int K, int topk, int dtype,
               int32_t *idx, float *val, float *gap, float *lse, void *ws, hipStream_t st) {
    if (want_lse) launch<KK, true>(hidden, w, M, N, K, topk, dtype, idx, val, gap, lse, ws, st);
    else launch<KK, false>(hidden, w, M, N, K, topk, dtype, idx, val, gap, lse, ws, st);
}

}  // namespace

extern "C" size_t eagle3_lmhead_workspace(int M, int N, int K, int topk, int dtype) {
    if (M <= 0 || N <= 0 || topk < 1) return 0;
    const int ntiles = (N + BN - 1) / BN;
    const int KK = kk_for(topk);
    const size_t rec = (size_t)M * ntiles;
    return align256(rec * KK * 4) + align256(rec * KK * 4) + align256(rec * 4) + align256(rec * 4);
}

extern "C" int eagle3_lmhead_argmax(const void *hidden, const void *w, int M, int N, int K, int topk, int dtype,
                                    int32_t *idx, float *val, float *gap, float *lse, void *ws, size_t ws_bytes,
                                    void *stream) {
    if (M < 0 || N < 0 || K < 1 || topk < 1) return EAGLE3_ERR_ARG;
    if (topk > 16 || N < 2 || topk > N) return EAGLE3_ERR_UNSUPPORTED;
    if (dtype != EAGLE3_BF16 && dtype != EAGLE3_F32) return EAGLE3_ERR_UNSUPPORTED;
    if (dtype == EAGLE3_BF16 && K % 64 != 0) return EAGLE3_ERR_UNSUPPORTED;
    if (dtype == EAGLE3_F32 && K % 4 != 0) return EAGLE3_ERR_UNSUPPORTED;
    if (M == 0) return EAGLE3_OK;
    if (!hidden || !w || !idx || !ws) return EAGLE3_ERR_ARG;
    if (!e3_aligned16(hidden) || !e3_aligned16(w) || !e3_aligned16(ws)) return EAGLE3_ERR_ARG;
    if (ws_bytes < eagle3_lmhead_workspace(M, N, K, topk, dtype)) return EAGLE3_ERR_WORKSPACE;
    const hipStream_t st = e3_stream(stream);
    const bool want_lse = lse != nullptr;
    switch (kk_for(topk)) {
        case 2: launch_kk<2>(want_lse, hidden, w, M, N, K, topk, dtype, idx, val, gap, lse, ws, st); break;
        case 4: launch_kk<4>(want_lse, hidden, w, M, N, K, topk, dtype, idx, val, gap, lse, ws, st); break;
        case 8: launch_kk<8>(want_lse, hidden, w, M, N, K, topk, dtype, idx, val, gap, lse, ws, st); break;
        default: launch_kk<16>(want_lse, hidden, w, M, N, K, topk, dtype, idx, val, gap, lse, ws, st); break;
    }
    E3_LAUNCH_CHECK();
    return EAGLE3_OK;
}
