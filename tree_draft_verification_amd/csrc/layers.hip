// Dense layers around the verify step and the EAGLE-3 draft head: GEMM with a
// K-segmented, optionally row-gathered A operand (so the draft's fusion FCs
// read [l; m; h] and [g; E[token]] without building the concatenation), SiLU
// gating, rotary embedding, embedding gather and KV-cache commit.
//
// The draft stage ([news] draft-stage paragraphs of the write-up of "EAGLE-3:
// Scaling up Inference Acceleration of Large Language Models via Training-Time
// Test"): an FC takes the concatenated low/mid/high features (3k) to k; the
// result (or, from step 2 on, the draft's own output) is concatenated with the
// embedding of the token one step ahead and an FC takes 2k to k; a single
// transformer layer follows. reading: that layer is a Llama decoder layer
// (RMSNorm, GQA attention with rotate-half RoPE, SwiGLU MLP, residuals).
#include <algorithm>

#include "common.h"
#include "gemm_core.h"

namespace {

using namespace e3g;

// C[M, N] = A[M, K] . B[N, K]^T (+ R), bf16 in/out, fp32 accumulate. A is up
// to three K-segments, each optionally row-gathered.
//
// Split K (SPLIT): work-group w takes tile w % tiles and k chunks
// [s nch / S, (s + 1) nch / S) of split s = w / tiles, and stores its fp32
// partial tile to part[s][M][N]; gemm_reduce_kernel adds the splits in
// order (plus the residual) and rounds once.
//
// VEC: the output rows are 16-byte aligned with N % 8 == 0 (chosen on the
// host), so the epilogue stages the results in LDS and writes 16-byte
// pieces; otherwise each element is stored on its own. The two epilogues are
// separate instantiations: compiled into one kernel, the scattered one's
// register pressure made the compiler spill accumulators after the main loop.
//
// SWIGLU (with VEC): B is a gate/up weight in paired layout (each 256-row
// tile = 128 gate rows, then the 128 up rows of the same outputs), so the
// tile's two column halves are the gate and up values of 128 outputs; the
// epilogue writes y = silu(g) * u to C [M, N / 2] with g and u first rounded
// to bf16 and the product formed as the separate gating kernel forms it.
template <int BM, int NS, bool SPLIT, bool VEC = false, bool SWIGLU = false>
__global__ __launch_bounds__(256, NS == 3 ? 2 : 1) void gemm_bf16_kernel(GemmParams p, int nsplit, float *part) {
    using T = GTile<BM, NS>;
    __shared__ __attribute__((aligned(1024))) unsigned char ring[T::RING];
    __shared__ int arow[3][BM];  // source row of each tile row, per segment
    const int tiles = p.mt * p.nt;
    const int split = SPLIT ? (int)blockIdx.x / tiles : 0;
    int mt, nt;
    tile_of(SPLIT ? (int)blockIdx.x % tiles : (int)blockIdx.x, tiles, p.mt, p.nt, mt, nt);
    const int m0 = mt * BM, n0 = nt * GBN;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int lr = lane & 31, lh = lane >> 5, wm = wave >> 1, wn = wave & 1;
    fill_arow<BM>(p, m0, arow);
    f32x16_t acc[T::MB][T::NB];
    const int nch_all = p.K / GBK;
    const int c_begin = SPLIT ? (int)((long)split * nch_all / nsplit) : 0;
    const int c_end = SPLIT ? (int)((long)(split + 1) * nch_all / nsplit) : nch_all;
    mainloop<BM, NS>(p, m0, n0, c_begin, c_end - c_begin, ring, arow, acc);
    if constexpr (SPLIT) {
        float *dst = part + (size_t)split * p.M * p.N;
#pragma unroll
        for (int mb = 0; mb < T::MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < T::NB; ++nb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = m0 + wm * (BM / 2) + mb * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
                    const int n = n0 + wn * 128 + nb * 32 + lr;
                    if (m < p.M && n < p.N) dst[(size_t)m * p.N + n] = acc[mb][nb][r];
                }
        return;
    }
    // D[m][n]: lane holds n = lr of its block, m = 8 (r / 4) + 4 lh + r % 4
    const uint16_t *res = (const uint16_t *)p.res;
    uint16_t *cc = (uint16_t *)p.c;
    if constexpr (SWIGLU) {
        // Waves (wm, 0) and (wm, 1) hold the gate and the up values of the
        // same 128 outputs. Each stages its 32 x 128 block (rounded to bf16)
        // in the ring; after a barrier the pair reads both and writes 16
        // rows each.
        constexpr int PITCH = 136;
        static_assert(4 * 32 * PITCH * sizeof(float) <= T::RING, "staging must fit the ring");
        __syncthreads();  // every wave is done with the ring
        int tx = threadIdx.x;
        __asm__ volatile("" : "+v"(tx));
        const int wv = tx >> 6, ln = tx & 63, wmv = wv >> 1, half = wv & 1;
        float *stg = reinterpret_cast<float *>(ring) + wv * 32 * PITCH;
        float *wr = stg + 4 * (ln >> 5) * PITCH + (ln & 31);
        const float *gate = reinterpret_cast<float *>(ring) + (2 * wmv) * 32 * PITCH;
        const float *up = gate + 32 * PITCH;
        const int rsub = 16 * half + (ln >> 4);                        // rows rsub + 4 i, i < 4
        const float *gp = gate + rsub * PITCH + (ln & 15) * 8;
        const float *upp = up + rsub * PITCH + (ln & 15) * 8;
        const int mrow = m0 + wmv * (BM / 2) + rsub;
        const int ncol = (n0 >> 1) + (ln & 15) * 8;                    // output column (p.N / 2 of them)
        const bool ncol_ok = ncol < (p.N >> 1);
#pragma unroll
        for (int mb = 0; mb < T::MB; ++mb) {
#pragma unroll
            for (int nb = 0; nb < T::NB; ++nb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    wr[(8 * (r >> 2) + (r & 3)) * PITCH + nb * 32] = e3_bf16_to_f32(e3_f32_to_bf16(acc[mb][nb][r]));
            __syncthreads();
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = mrow + mb * 32 + 4 * i;
                if (m < p.M && ncol_ok) {
                    const f32x4_t g0 = *reinterpret_cast<const f32x4_t *>(gp + 4 * i * PITCH);
                    const f32x4_t g1 = *reinterpret_cast<const f32x4_t *>(gp + 4 * i * PITCH + 4);
                    const f32x4_t u0 = *reinterpret_cast<const f32x4_t *>(upp + 4 * i * PITCH);
                    const f32x4_t u1 = *reinterpret_cast<const f32x4_t *>(upp + 4 * i * PITCH + 4);
                    const float g[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
                    const float u[8] = {u0[0], u0[1], u0[2], u0[3], u1[0], u1[1], u1[2], u1[3]};
                    u32x4_t o;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float a = g[2 * q] / (1.f + expf(-g[2 * q])) * u[2 * q];
                        const float b = g[2 * q + 1] / (1.f + expf(-g[2 * q + 1])) * u[2 * q + 1];
                        o[q] = (uint32_t)e3_f32_to_bf16(a) | ((uint32_t)e3_f32_to_bf16(b) << 16);
                    }
                    *reinterpret_cast<u32x4_t *>(cc + (size_t)m * p.ldc + ncol) = o;
                }
            }
            __syncthreads();  // the pair is done before the next block overwrites
        }
        return;
    } else if constexpr (VEC) {
        // Each wave stages one 32 x 128 block of its fp32 results at a time in
        // the (now idle) ring, then writes 16-byte rows of 8 outputs: 32
        // stores of 1 KB per wave and block instead of 2-byte scattered
        // stores (those cost a quarter of the 3904 x 28672 x 4096 GEMM's
        // time). The residual is added in fp32 and the sum rounded once, as
        // in the direct path. Row pitch 136 floats: the two lane halves
        // (4 rows apart) write disjoint banks.
        constexpr int PITCH = 136;
        static_assert(4 * 32 * PITCH * sizeof(float) <= T::RING, "staging must fit the ring");
        __syncthreads();  // every wave is done with the ring
        // lane-dependent addresses are formed from an opaque copy of the
        // thread id, so none of them is computed before the main loop and
        // kept live (spilled) across it
        int tx = threadIdx.x;
        __asm__ volatile("" : "+v"(tx));
        const int wv = tx >> 6, ln = tx & 63;
        float *stg = reinterpret_cast<float *>(ring) + wv * 32 * PITCH;
        float *wr = stg + 4 * (ln >> 5) * PITCH + (ln & 31);           // accumulator layout
        const float *rdp = stg + (ln >> 4) * PITCH + (ln & 15) * 8;    // 16-byte chunks, row-major
        const int mrow = m0 + (wv >> 1) * (BM / 2) + (ln >> 4);
        const int ncol = n0 + (wv & 1) * 128 + (ln & 15) * 8;
        const bool ncol_ok = ncol < p.N;
#pragma unroll
        for (int mb = 0; mb < T::MB; ++mb) {
#pragma unroll
            for (int nb = 0; nb < T::NB; ++nb)
#pragma unroll
                for (int r = 0; r < 16; ++r) wr[(8 * (r >> 2) + (r & 3)) * PITCH + nb * 32] = acc[mb][nb][r];
            // the block's residual pieces are requested now (in the registers
            // its accumulators just left), so they arrive during the LDS pass
            u32x4_t rv[8];
            if (res) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int m = mrow + mb * 32 + 4 * i;
                    rv[i] = m < p.M && ncol_ok ? *reinterpret_cast<const u32x4_t *>(res + (size_t)m * p.ldc + ncol)
                                               : u32x4_t{0, 0, 0, 0};
                }
            }
            // a wave's LDS accesses complete in order: the reads see the writes,
            // and the next block's writes follow these reads
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int m = mrow + mb * 32 + 4 * i;
                if (m < p.M && ncol_ok) {
                    const f32x4_t lo = *reinterpret_cast<const f32x4_t *>(rdp + 4 * i * PITCH);
                    const f32x4_t hi = *reinterpret_cast<const f32x4_t *>(rdp + 4 * i * PITCH + 4);
                    float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    const size_t off = (size_t)m * p.ldc + ncol;
                    if (res) {
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            v[2 * q] += e3_bf16_to_f32((uint16_t)(rv[i][q] & 0xffffu));
                            v[2 * q + 1] += e3_bf16_to_f32((uint16_t)(rv[i][q] >> 16));
                        }
                    }
                    u32x4_t o;
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        o[q] = (uint32_t)e3_f32_to_bf16(v[2 * q]) | ((uint32_t)e3_f32_to_bf16(v[2 * q + 1]) << 16);
                    *reinterpret_cast<u32x4_t *>(cc + off) = o;
                }
            }
        }
        return;
    }
#pragma unroll
    for (int mb = 0; mb < T::MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < T::NB; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm * (BM / 2) + mb * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
                const int n = n0 + wn * 128 + nb * 32 + lr;
                if (m < p.M && n < p.N) {
                    float v = acc[mb][nb][r];
                    if (res) v += e3_bf16_to_f32(res[(size_t)m * p.ldc + n]);
                    cc[(size_t)m * p.ldc + n] = e3_f32_to_bf16(v);
                }
            }
}

// Sum of the split partials in split order (+ residual), rounded once to bf16.
__global__ __launch_bounds__(256) void gemm_reduce_kernel(const float *__restrict__ part, int nsplit, int M, int N,
                                                          const uint16_t *res, uint16_t *c, int ldc) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (size_t)M * N) return;
    const int m = (int)(i / N), n = (int)(i % N);
    float v = 0.f;
    for (int s = 0; s < nsplit; ++s) v += part[(size_t)s * M * N + i];
    if (res) v += e3_bf16_to_f32(res[(size_t)m * ldc + n]);
    c[(size_t)m * ldc + n] = e3_f32_to_bf16(v);
}

// fp32 GEMM for small models: 16 x 16 output tile per 256 threads, 16-wide k
// chunks through LDS; every output accumulates k in ascending order.
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmParams p) {
    __shared__ float As[16][17];
    __shared__ float Bs[16][17];
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    const int m = blockIdx.x * 16 + ty, n = blockIdx.y * 16 + tx;
    float acc = 0.f;
    for (int kc = 0; kc < p.K; kc += 16) {
        {   // A element (row ty, k tx) and B element (row ty, k tx) of this chunk
            const int k = kc + tx;
            const int ma = blockIdx.x * 16 + ty;
            float av = 0.f;
            if (ma < p.M && k < p.K) {
                int seg = 0;
                while (seg + 1 < p.nseg && k >= p.kofs[seg + 1]) ++seg;
                int row = ma;
                if (p.a_rows[seg]) row = min(max(p.a_rows[seg][ma], 0), p.a_nrows[seg] - 1);
                av = ((const float *)p.a[seg])[(size_t)row * p.k[seg] + (k - p.kofs[seg])];
            }
            As[ty][tx] = av;
            const int nb = blockIdx.y * 16 + ty;
            Bs[ty][tx] = (nb < p.N && k < p.K) ? ((const float *)p.b)[(size_t)nb * p.K + k] : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) acc = fmaf(As[ty][kk], Bs[tx][kk], acc);
        __syncthreads();
    }
    if (m < p.M && n < p.N) {
        float v = acc;
        if (p.res) v += ((const float *)p.res)[(size_t)m * p.ldc + n];
        ((float *)p.c)[(size_t)m * p.ldc + n] = v;
    }
}

// y[m][f] = silu(gu[m][f]) * gu[m][F + f]
template <bool BF16>
__global__ __launch_bounds__(256) void silu_mul_kernel(const void *__restrict__ gu, int M, int F, void *__restrict__ y) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (size_t)M * F) return;
    const size_t m = i / F, f = i % F;
    float g, u;
    if (BF16) {
        g = e3_bf16_to_f32(((const uint16_t *)gu)[m * 2 * F + f]);
        u = e3_bf16_to_f32(((const uint16_t *)gu)[m * 2 * F + F + f]);
    } else {
        g = ((const float *)gu)[m * 2 * F + f];
        u = ((const float *)gu)[m * 2 * F + F + f];
    }
    const float v = g / (1.f + expf(-g)) * u;
    if (BF16) ((uint16_t *)y)[i] = e3_f32_to_bf16(v);
    else ((float *)y)[i] = v;
}

// Rotate-half RoPE in place on x viewed as [M][H][D] with row stride ld
// (elements): pair (i, i + D/2) at position p = pos_offset + pos[m] turns by
// p * theta^(-2i/D); the angle is formed in double precision.
// One thread per (row, pair index): the angle depends on the position and
// the pair only, so its sine and cosine (double precision) are formed once
// and applied to every head of the row.
template <bool BF16>
__global__ __launch_bounds__(256) void rope_kernel(void *__restrict__ x, int M, int H, int D, int ld,
                                                   const int32_t *__restrict__ pos, int pos_offset, double log_theta) {
    const int half = D / 2;
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (size_t)M * half) return;
    const int j = (int)(i % half);
    const int m = (int)(i / half);
    const double ang = (double)(pos_offset + pos[m]) * exp(-2.0 * j / D * log_theta);
    double sn, cs;
    sincos(ang, &sn, &cs);
    for (int h = 0; h < H; ++h) {
        const size_t base = (size_t)m * ld + (size_t)h * D;
        if (BF16) {
            uint16_t *p = (uint16_t *)x;
            const double a = e3_bf16_to_f32(p[base + j]), b = e3_bf16_to_f32(p[base + j + half]);
            p[base + j] = e3_f32_to_bf16((float)(a * cs - b * sn));
            p[base + j + half] = e3_f32_to_bf16((float)(b * cs + a * sn));
        } else {
            float *p = (float *)x;
            const double a = p[base + j], b = p[base + j + half];
            p[base + j] = (float)(a * cs - b * sn);
            p[base + j + half] = (float)(b * cs + a * sn);
        }
    }
}

// out[m] = E[clamp(ids[m])], 16 bytes per thread
__global__ __launch_bounds__(256) void embed_kernel(const uint4 *__restrict__ E, const int32_t *__restrict__ ids,
                                                    int M, int row_vec, int V, uint4 *__restrict__ out) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (size_t)M * row_vec) return;
    const int m = (int)(i / row_vec), c = (int)(i % row_vec);
    const int id = min(max(ids[m], 0), V - 1);
    out[i] = E[(size_t)id * row_vec + c];
}

// Append rows to the paged cache: for sequence b, rows src[b][0..] (indices
// into k_rows/v_rows [B, rows_per_seq, Hkv, D]; the list ends at the first
// negative entry or after max_n; a null list means rows 0..max_n-1) land at
// positions start[b] + j. Cache layouts: K [blk][Hkv][16][D], V [blk][Hkv][D][16].
// One work-group per (entry j, sequence b).
template <bool BF16>
__global__ __launch_bounds__(256) void commit_kv_kernel(const void *__restrict__ k_rows, const void *__restrict__ v_rows,
                                                        int rows_per_seq, const int32_t *__restrict__ src, int max_n,
                                                        int Hkv, int D, void *__restrict__ k_cache,
                                                        void *__restrict__ v_cache,
                                                        const int32_t *__restrict__ block_table, int max_blocks,
                                                        int num_blocks, const int32_t *__restrict__ start) {
    const int j = blockIdx.x, b = blockIdx.y;
    int r = j;
    if (src) {
        const int32_t *s = src + (size_t)b * max_n;
        int ended = 0;
        for (int q = threadIdx.x; q <= j; q += blockDim.x) ended |= s[q] < 0;
        if (__syncthreads_or(ended)) return;  // the list ended before entry j
        r = s[j];
    }
    r = min(r, rows_per_seq - 1);
    const int posn = start[b] + j;
    if (posn < 0 || posn >= max_blocks * 16) return;
    const int blk = min(max(block_table[(size_t)b * max_blocks + posn / 16], 0), num_blocks - 1);
    const int slot = posn % 16;
    for (int i = threadIdx.x; i < Hkv * D; i += blockDim.x) {
        const int d = i % D, h = i / D;
        const size_t srow = (((size_t)b * rows_per_seq + r) * Hkv + h) * D + d;
        const size_t kdst = (((size_t)blk * Hkv + h) * 16 + slot) * D + d;
        const size_t vdst = (((size_t)blk * Hkv + h) * D + d) * 16 + slot;
        if (BF16) {
            ((uint16_t *)k_cache)[kdst] = ((const uint16_t *)k_rows)[srow];
            ((uint16_t *)v_cache)[vdst] = ((const uint16_t *)v_rows)[srow];
        } else {
            ((float *)k_cache)[kdst] = ((const float *)k_rows)[srow];
            ((float *)v_cache)[vdst] = ((const float *)v_rows)[srow];
        }
    }
}

// Persistent form of the SWIGLU tiles for one A segment without a row gather
// (tile-claim counters in the caller's workspace; see mainloop_persistent):
// eight waves per 256 x 256 tile with the MFMA operands swapped, so a lane
// holds one row and 16 columns of each 32 x 32 block. Of the four waves of a
// row half, waves 0-1 hold the gate values (tile columns 0-127) and waves 2-3
// the up values of the same outputs in the same lane and register positions.
// The gating is split between the two waves of a pair, which sit on
// different SIMDs: per 32-row block the up wave hands its bf16-rounded up
// values of its first 32 columns to the gate wave and the gate wave its gate
// values of the second 32 columns to the up wave, through LDS (the ring holds
// the next tile's chunks); each then writes y = silu(g) * u for its 32
// columns as 16-byte row pieces, with the same rounding and arithmetic as the
// other SWIGLU epilogue.
__global__ __launch_bounds__(512, 1) void gemm_swiglu_persistent_kernel(GemmParams p, uint32_t *ctr) {
    using T = GTile<256, 4, 8>;
    constexpr int BM = 256;
    static_assert(T::MB == 4 && T::NB == 2 && T::CW == 64, "wave tile 128 x 64");
    __shared__ __attribute__((aligned(1024))) unsigned char ring[T::RING];
    __shared__ uint32_t ub[2 * 2 * 2 * 8 * 64];  // [row half][pair][from up / from gate][bf16 pair][lane]
    __shared__ int tq[2];
    TileQueue queue;
    queue.init(ctr, tq, p.mt * p.nt);
    auto tile_at = [&](int t, int &m0, int &n0) {
        int mt, nt;
        tile_at_order(t, p.mt, p.nt, mt, nt);
        m0 = mt * BM;
        n0 = nt * GBN;
    };
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int lr = lane & 31, lh = lane >> 5, wm = wave / T::WN, wn = wave % T::WN;
    uint16_t *cc = (uint16_t *)p.c;
    uint32_t *pair_slot = ub + ((wm * 2 + (wn & 1)) * 2) * 8 * 64;
    auto epilogue = [&](int tile, const f32x16_t (&acc)[T::MB][T::NB]) {
        int m0, n0;
        tile_at(tile, m0, n0);
        const bool rows_here = __builtin_amdgcn_readfirstlane(m0 + wm * (BM / 2)) < p.M;
        const bool up = __builtin_amdgcn_readfirstlane(wn) >= 2;
        // this wave computes the outputs of block `own` (gate wave: 0, up
        // wave: 1) and hands its values of the other block to its partner
        const int own = up ? 1 : 0;
        uint32_t *to_partner = pair_slot + (up ? 0 : 1) * 8 * 64;
        const uint32_t *from_partner = pair_slot + (up ? 1 : 0) * 8 * 64;
        uint16_t *ybase = cc + (n0 >> 1) + (wn & 1) * T::CW + own * 32 + 4 * lh;
#pragma unroll
        for (int mb = 0; mb < T::MB; ++mb) {
            if (rows_here) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float v0 = up ? acc[mb][0][2 * e] : acc[mb][1][2 * e];
                    const float v1 = up ? acc[mb][0][2 * e + 1] : acc[mb][1][2 * e + 1];
                    to_partner[e * 64 + lane] = (uint32_t)e3_f32_to_bf16(v0) | ((uint32_t)e3_f32_to_bf16(v1) << 16);
                }
            }
            lds_barrier();
            const int m = m0 + wm * (BM / 2) + 32 * mb + lr;
            if (rows_here && m < p.M) {
                uint16_t *yrow = ybase + (size_t)m * p.ldc;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    // outputs 32 own + 8 q + 4 lh + (0..3) of this pair's 64
                    const uint32_t w01 = from_partner[(2 * q) * 64 + lane];
                    const uint32_t w23 = from_partner[(2 * q + 1) * 64 + lane];
                    const float other[4] = {e3_bf16_to_f32((uint16_t)w01), e3_bf16_to_f32((uint16_t)(w01 >> 16)),
                                            e3_bf16_to_f32((uint16_t)w23), e3_bf16_to_f32((uint16_t)(w23 >> 16))};
                    uint16_t y[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float mine = e3_bf16_to_f32(e3_f32_to_bf16(up ? acc[mb][1][4 * q + e]
                                                                            : acc[mb][0][4 * q + e]));
                        const float g = up ? other[e] : mine, u = up ? mine : other[e];
                        y[e] = e3_f32_to_bf16(g / (1.f + expf(-g)) * u);
                    }
                    uint2 o;
                    o.x = (uint32_t)y[0] | ((uint32_t)y[1] << 16);
                    o.y = (uint32_t)y[2] | ((uint32_t)y[3] << 16);
                    *reinterpret_cast<uint2 *>(yrow + 8 * q) = o;
                }
            }
            lds_barrier();  // the pair is done before the next block overwrites the slots
        }
    };
    mainloop_persistent<BM, T::NS, true, 8>(p, tile_at, queue, epilogue, ring);
}

// Persistent form of the 256-row tiles of the plain product (C = A . B^T,
// plus the residual with RES) for one A segment without a row gather
// (tile-claim counters in the caller's workspace; see mainloop_persistent),
// run on the persistent loop of the many-row LM head: eight waves per 256 x 256 tile with the MFMA operands
// swapped, so a lane holds one output row and, per 32 x 32 block, the column
// quads 8 q + 4 lh (q < 4) in registers 4 q .. 4 q + 3. Each quad leaves as
// one 8-byte store after the residual is added in fp32 and the sum rounded
// once: the arithmetic of the per-tile kernels, so results are identical.
// Requires N and ldc multiples of 8 and 16-byte aligned C and residual.
template <bool RES>
__global__ __launch_bounds__(512, 1) void gemm_persistent_kernel(GemmParams p, uint32_t *ctr) {
    using T = GTile<256, 4, 8>;
    constexpr int BM = 256;
    static_assert(T::MB == 4 && T::NB == 2 && T::CW == 64, "wave tile 128 x 64");
    __shared__ __attribute__((aligned(1024))) unsigned char ring[T::RING];
    __shared__ int tq[2];
    TileQueue queue;
    queue.init(ctr, tq, p.mt * p.nt);
    auto tile_at = [&](int t, int &m0, int &n0) {
        int mt, nt;
        tile_at_order(t, p.mt, p.nt, mt, nt);
        m0 = mt * BM;
        n0 = nt * GBN;
    };
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int lr = lane & 31, lh = lane >> 5, wm = wave / T::WN, wn = wave % T::WN;
    uint16_t *cc = (uint16_t *)p.c;
    const uint16_t *res = (const uint16_t *)p.res;
    auto epilogue = [&](int tile, const f32x16_t (&acc)[T::MB][T::NB]) {
        int m0, n0;
        tile_at(tile, m0, n0);
        const int mw = __builtin_amdgcn_readfirstlane(m0 + wm * (BM / 2));
        if (mw >= p.M) return;  // a last tile's upper half past M
        const int nw = n0 + wn * T::CW + 4 * lh;
#pragma unroll
        for (int mb = 0; mb < T::MB; ++mb) {
            const int m = mw + 32 * mb + lr;
            if (m < p.M) {
                const size_t row = (size_t)m * p.ldc;
                uint2 rv[T::NB][4];
                if constexpr (RES) {
#pragma unroll
                    for (int nb = 0; nb < T::NB; ++nb)
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int n = nw + 32 * nb + 8 * q;
                            rv[nb][q] = n < p.N ? *reinterpret_cast<const uint2 *>(res + row + n) : uint2{0, 0};
                        }
                }
#pragma unroll
                for (int nb = 0; nb < T::NB; ++nb)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int n = nw + 32 * nb + 8 * q;
                        if (n < p.N) {
                            float v[4];
#pragma unroll
                            for (int e = 0; e < 4; ++e) v[e] = acc[mb][nb][4 * q + e];
                            if constexpr (RES) {
                                v[0] += e3_bf16_to_f32((uint16_t)(rv[nb][q].x & 0xffffu));
                                v[1] += e3_bf16_to_f32((uint16_t)(rv[nb][q].x >> 16));
                                v[2] += e3_bf16_to_f32((uint16_t)(rv[nb][q].y & 0xffffu));
                                v[3] += e3_bf16_to_f32((uint16_t)(rv[nb][q].y >> 16));
                            }
                            uint2 o;
                            o.x = (uint32_t)e3_f32_to_bf16(v[0]) | ((uint32_t)e3_f32_to_bf16(v[1]) << 16);
                            o.y = (uint32_t)e3_f32_to_bf16(v[2]) | ((uint32_t)e3_f32_to_bf16(v[3]) << 16);
                            *reinterpret_cast<uint2 *>(cc + row + n) = o;
                        }
                    }
            }
        }
    };
    mainloop_persistent<BM, T::NS, true, 8>(p, tile_at, queue, epilogue, ring);
}

// dst[dst_rows[i]] = src[src_rows[i]] for i < n, 16 bytes per thread; a null
// table is the identity; rows outside [0, nrows) are skipped.
__global__ __launch_bounds__(256) void copy_rows_kernel(const uint4 *__restrict__ src,
                                                        const int32_t *__restrict__ src_rows, int src_nrows,
                                                        uint4 *__restrict__ dst, const int32_t *__restrict__ dst_rows,
                                                        int dst_nrows, int n, int row_vec) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (size_t)n * row_vec) return;
    const int m = (int)(i / row_vec), c = (int)(i % row_vec);
    const int sr = src_rows ? src_rows[m] : m;
    const int dr = dst_rows ? dst_rows[m] : m;
    if (sr < 0 || sr >= src_nrows || dr < 0 || dr >= dst_nrows) return;
    dst[(size_t)dr * row_vec + c] = src[(size_t)sr * row_vec + c];
}

unsigned grid1(size_t n) { return (unsigned)((n + 255) / 256); }

// Splits of K for a bf16 call whose 128-row tiles would leave more than half
// of the CUs idle: enough splits to give every CU a work-group, at least 16
// chunks (512 columns) each, at most 8.
int gemm_splits(const eagle3_gemm_args *a, int K) {
    if (a->dtype != EAGLE3_BF16 || a->M < 1 || a->N < 1) return 1;
    const long tiles = (long)((a->M + 127) / 128) * ((a->N + GBN - 1) / GBN);
    const long cus = e3_cu_count();
    if (2 * tiles > cus) return 1;
    long s = cus / tiles;
    s = std::min(s, (long)(K / GBK / 16));
    s = std::min(s, 8L);
    return s < 2 ? 1 : (int)s;
}

int gemm_k(const eagle3_gemm_args *a) {
    int K = 0;
    for (int s = 0; s < a->nseg && s < 3; ++s) K += a->k[s] > 0 ? a->k[s] : 0;
    return K;
}

// Tile shape of an unsplit bf16 call by the amount of work (measured):
// 256-row tiles once they make four passes over the CUs (most reuse,
// 65536 x 4096 x 12288: 1.01 vs 0.90 PFLOP/s per-tile); else 128-row tiles
// two per CU while those fill both slots of every CU (640 x 28672 x 4096:
// 0.59 vs 0.50); else 256-row tiles if they fill the CUs once (3904 x 4096 x
// 4096: 0.82 vs 0.72); below that 128-row tiles one per CU with the deeper
// ring (640 x 4096 x 14336: 0.39 vs 0.33).
bool gemm_rows256(int M, int N) {
    const int nt = (N + GBN - 1) / GBN;
    const long t256 = (long)((M + 255) / 256) * nt, t128 = (long)((M + 127) / 128) * nt;
    const long cus = e3_cu_count();
    return t256 >= 4 * cus || (t128 < 2 * cus && t256 >= cus);
}

// 16-byte row pieces in the output (and the residual)
bool gemm_vec(const eagle3_gemm_args *a, int ldc) {
    return a->N % 8 == 0 && ldc % 8 == 0 && e3_aligned16(a->c) && (!a->residual || e3_aligned16(a->residual));
}

// Whether an unsplit bf16 call runs the persistent 256-row kernel given a
// workspace for its tile counters: one A segment without a row gather,
// vector output, at least 4 chunks of K, and 256-row tiles that make at
// least four passes over the CUs or at most one (measured against the
// per-tile kernel: 65536 x 4096 x 4096..12288 and 65536 x 1024 x 4096
// 1.10-1.18 against 0.94-1.07 PFLOP/s; one tile per CU, 3904 x 4096 x 14336
// 407 against 448-460 us, 3904 x 4096 x 4096 alike). In between, the queue's
// start (two tiles per work-group) would leave CUs idle.
bool gemm_persistent(const eagle3_gemm_args *a, int K, int ldc) {
    if (a->dtype != EAGLE3_BF16 || a->nseg != 1 || a->a_rows[0] || K / GBK < 4 || !gemm_vec(a, ldc)) return false;
    const long t256 = (long)((a->M + 255) / 256) * ((a->N + GBN - 1) / GBN), cus = e3_cu_count();
    return t256 >= 4 * cus || t256 <= cus;
}

}  // namespace

extern "C" size_t eagle3_gemm_workspace(const eagle3_gemm_args *a) {
    if (!a || a->nseg < 1 || a->nseg > 3 || a->M < 1 || a->N < 1) return 0;
    const int K = gemm_k(a);
    const int S = gemm_splits(a, K);
    if (S > 1) return (size_t)S * a->M * a->N * sizeof(float);
    return gemm_persistent(a, K, a->ldc > 0 ? a->ldc : a->N) ? EAGLE3_PERSIST_WS_BYTES : 0;
}

extern "C" int eagle3_gemm(const eagle3_gemm_args *a, void *stream) {
    if (!a) return EAGLE3_ERR_ARG;
    if (a->M < 0 || a->N < 1 || a->nseg < 1 || a->nseg > 3) return EAGLE3_ERR_ARG;
    if (a->dtype != EAGLE3_BF16 && a->dtype != EAGLE3_F32) return EAGLE3_ERR_UNSUPPORTED;
    if (a->M == 0) return EAGLE3_OK;
    if (!a->b || !a->c) return EAGLE3_ERR_ARG;
    const int ldc = a->ldc > 0 ? a->ldc : a->N;
    if (ldc < a->N) return EAGLE3_ERR_ARG;
    GemmParams p{};
    int K = 0;
    for (int s = 0; s < a->nseg; ++s) {
        if (!a->a[s] || a->k[s] < 1) return EAGLE3_ERR_ARG;
        if (a->a_rows[s] && a->a_nrows[s] < 1) return EAGLE3_ERR_ARG;
        // the core addresses an A segment by 32-bit byte offsets
        if (a->dtype == EAGLE3_BF16 && (uint64_t)(a->a_rows[s] ? a->a_nrows[s] : a->M) * a->k[s] * 2 >= (1ull << 32))
            return EAGLE3_ERR_UNSUPPORTED;
        if (a->dtype == EAGLE3_BF16 && (a->k[s] % GSEG_ALIGN != 0 || !e3_aligned16(a->a[s])))
            return EAGLE3_ERR_UNSUPPORTED;
        p.a[s] = a->a[s];
        p.a_rows[s] = a->a_rows[s];
        p.a_nrows[s] = a->a_rows[s] ? a->a_nrows[s] : a->M;
        p.k[s] = a->k[s];
        p.kofs[s] = K;
        K += a->k[s];
    }
    if (a->dtype == EAGLE3_BF16 && !e3_aligned16(a->b)) return EAGLE3_ERR_ARG;
    p.nseg = a->nseg; p.b = a->b; p.res = a->residual; p.c = a->c;
    p.M = a->M; p.N = a->N; p.K = K; p.ldc = ldc;
    const hipStream_t st = e3_stream(stream);
    const int S = a->dtype == EAGLE3_BF16 ? gemm_splits(a, K) : 1;
    if (S > 1 && a->ws && a->ws_bytes >= (size_t)S * a->M * a->N * sizeof(float) && e3_aligned16(a->ws)) {
        // few tiles: split K so every CU gets a work-group, then reduce
        p.nt = (a->N + GBN - 1) / GBN;
        p.mt = (a->M + 127) / 128;
        float *part = (float *)a->ws;
        gemm_bf16_kernel<128, 4, true><<<p.mt * p.nt * S, 256, 0, st>>>(p, S, part);
        gemm_reduce_kernel<<<grid1((size_t)a->M * a->N), 256, 0, st>>>(part, S, a->M, a->N,
                                                                       (const uint16_t *)a->residual,
                                                                       (uint16_t *)a->c, ldc);
    } else if (a->dtype == EAGLE3_BF16) {
        const int nt = (a->N + GBN - 1) / GBN;
        const long t256 = (long)((a->M + 255) / 256) * nt, t128 = (long)((a->M + 127) / 128) * nt;
        const long cus = e3_cu_count();
        p.nt = nt;
        const bool vec = gemm_vec(a, ldc);
        if (gemm_rows256(a->M, a->N)) {
            p.mt = (a->M + 255) / 256;
            if (a->ws && a->ws_bytes >= EAGLE3_PERSIST_WS_BYTES && e3_aligned16(a->ws) && gemm_persistent(a, K, ldc)) {
                // persistent work-groups (one per CU) taking tiles from the
                // counters in the workspace
                uint32_t *ctr = (uint32_t *)a->ws;
                const int grid = (int)std::min<long>(t256, cus);
                ctr_zero_kernel<<<1, 64, 0, st>>>(ctr);
                if (a->residual) gemm_persistent_kernel<true><<<grid, 512, 0, st>>>(p, ctr);
                else gemm_persistent_kernel<false><<<grid, 512, 0, st>>>(p, ctr);
            } else if (vec) {
                gemm_bf16_kernel<256, 4, false, true><<<p.mt * nt, 256, 0, st>>>(p, 1, nullptr);
            } else {
                gemm_bf16_kernel<256, 4, false><<<p.mt * nt, 256, 0, st>>>(p, 1, nullptr);
            }
        } else if (t128 >= 2 * cus) {
            p.mt = (a->M + 127) / 128;
            if (vec) gemm_bf16_kernel<128, 3, false, true><<<p.mt * nt, 256, 0, st>>>(p, 1, nullptr);
            else gemm_bf16_kernel<128, 3, false><<<p.mt * nt, 256, 0, st>>>(p, 1, nullptr);
        } else {
            p.mt = (a->M + 127) / 128;
            if (vec) gemm_bf16_kernel<128, 4, false, true><<<p.mt * nt, 256, 0, st>>>(p, 1, nullptr);
            else gemm_bf16_kernel<128, 4, false><<<p.mt * nt, 256, 0, st>>>(p, 1, nullptr);
        }
    } else {
        dim3 grid((a->M + 15) / 16, (a->N + 15) / 16);
        gemm_f32_kernel<<<grid, 256, 0, st>>>(p);
    }
    E3_LAUNCH_CHECK();
    return EAGLE3_OK;
}

extern "C" int eagle3_gemm_swiglu(const eagle3_gemm_args *a, void *stream) {
    if (!a) return EAGLE3_ERR_ARG;
    if (a->M < 0 || a->N < 1 || a->nseg < 1 || a->nseg > 3) return EAGLE3_ERR_ARG;
    if (a->dtype != EAGLE3_BF16 || a->N % 256 != 0 || a->residual) return EAGLE3_ERR_UNSUPPORTED;
    if (a->M == 0) return EAGLE3_OK;
    if (!a->b || !a->c) return EAGLE3_ERR_ARG;
    const int F = a->N / 2;
    const int ldc = a->ldc > 0 ? a->ldc : F;
    if (ldc < F || ldc % 8 != 0 || !e3_aligned16(a->c) || !e3_aligned16(a->b)) return EAGLE3_ERR_ARG;
    GemmParams p{};
    int K = 0;
    for (int s = 0; s < a->nseg; ++s) {
        if (!a->a[s] || a->k[s] < 1) return EAGLE3_ERR_ARG;
        if (a->a_rows[s] && a->a_nrows[s] < 1) return EAGLE3_ERR_ARG;
        // the core addresses an A segment by 32-bit byte offsets
        if (a->dtype == EAGLE3_BF16 && (uint64_t)(a->a_rows[s] ? a->a_nrows[s] : a->M) * a->k[s] * 2 >= (1ull << 32))
            return EAGLE3_ERR_UNSUPPORTED;
        if (a->k[s] % GSEG_ALIGN != 0 || !e3_aligned16(a->a[s])) return EAGLE3_ERR_UNSUPPORTED;
        p.a[s] = a->a[s];
        p.a_rows[s] = a->a_rows[s];
        p.a_nrows[s] = a->a_rows[s] ? a->a_nrows[s] : a->M;
        p.k[s] = a->k[s];
        p.kofs[s] = K;
        K += a->k[s];
    }
    p.nseg = a->nseg; p.b = a->b; p.res = nullptr; p.c = a->c;
    p.M = a->M; p.N = a->N; p.K = K; p.ldc = ldc;
    const hipStream_t st = e3_stream(stream);
    // tile shape as eagle3_gemm chooses it for the same product
    const int nt = a->N / GBN;
    const long t256 = (long)((a->M + 255) / 256) * nt, t128 = (long)((a->M + 127) / 128) * nt;
    const long cus = e3_cu_count();
    p.nt = nt;
    if (gemm_rows256(a->M, a->N)) {
        p.mt = (a->M + 255) / 256;
        // persistent work-groups when the workspace can hold the tile counters
        // (one A segment without a row gather; at least 4 chunks of K)
        if (a->ws && a->ws_bytes >= EAGLE3_PERSIST_WS_BYTES && e3_aligned16(a->ws) && a->nseg == 1 &&
            !a->a_rows[0] && K / GBK >= 4) {
            uint32_t *ctr = (uint32_t *)a->ws;
            ctr_zero_kernel<<<1, 64, 0, st>>>(ctr);
            gemm_swiglu_persistent_kernel<<<(int)std::min<long>(t256, cus), 512, 0, st>>>(p, ctr);
        } else {
            gemm_bf16_kernel<256, 4, false, true, true><<<p.mt * nt, 256, 0, st>>>(p, 1, nullptr);
        }
    } else if (t128 >= 2 * cus) {
        p.mt = (a->M + 127) / 128;
        gemm_bf16_kernel<128, 3, false, true, true><<<p.mt * nt, 256, 0, st>>>(p, 1, nullptr);
    } else {
        p.mt = (a->M + 127) / 128;
        gemm_bf16_kernel<128, 4, false, true, true><<<p.mt * nt, 256, 0, st>>>(p, 1, nullptr);
    }
    E3_LAUNCH_CHECK();
    return EAGLE3_OK;
}

extern "C" int eagle3_silu_mul(const void *gu, int M, int F, int dtype, void *y, void *stream) {
    if (M < 0 || F < 1) return EAGLE3_ERR_ARG;
    if (dtype != EAGLE3_BF16 && dtype != EAGLE3_F32) return EAGLE3_ERR_UNSUPPORTED;
    if (M == 0) return EAGLE3_OK;
    if (!gu || !y) return EAGLE3_ERR_ARG;
    const size_t n = (size_t)M * F;
    if (dtype == EAGLE3_BF16) silu_mul_kernel<true><<<grid1(n), 256, 0, e3_stream(stream)>>>(gu, M, F, y);
    else silu_mul_kernel<false><<<grid1(n), 256, 0, e3_stream(stream)>>>(gu, M, F, y);
    E3_LAUNCH_CHECK();
    return EAGLE3_OK;
}

extern "C" int eagle3_rope(void *x, int M, int H, int D, int ld, const int32_t *pos, int pos_offset, float theta,
                           int dtype, void *stream) {
    if (M < 0 || H < 1 || D < 2 || (D & 1) || !(theta > 1.f)) return EAGLE3_ERR_ARG;
    if (dtype != EAGLE3_BF16 && dtype != EAGLE3_F32) return EAGLE3_ERR_UNSUPPORTED;
    if (ld < H * D) return EAGLE3_ERR_ARG;
    if (M == 0) return EAGLE3_OK;
    if (!x || !pos) return EAGLE3_ERR_ARG;
    const size_t n = (size_t)M * (D / 2);
    const double lt = log((double)theta);
    if (dtype == EAGLE3_BF16) rope_kernel<true><<<grid1(n), 256, 0, e3_stream(stream)>>>(x, M, H, D, ld, pos, pos_offset, lt);
    else rope_kernel<false><<<grid1(n), 256, 0, e3_stream(stream)>>>(x, M, H, D, ld, pos, pos_offset, lt);
    E3_LAUNCH_CHECK();
    return EAGLE3_OK;
}

extern "C" int eagle3_embed(const void *E, const int32_t *ids, int M, int K, int V, int dtype, void *out,
                            void *stream) {
    if (M < 0 || K < 1 || V < 1) return EAGLE3_ERR_ARG;
    if (dtype != EAGLE3_BF16 && dtype != EAGLE3_F32) return EAGLE3_ERR_UNSUPPORTED;
    const int esz = dtype == EAGLE3_BF16 ? 2 : 4;
    if (((size_t)K * esz) % 16 != 0) return EAGLE3_ERR_UNSUPPORTED;
    if (M == 0) return EAGLE3_OK;
    if (!E || !ids || !out || !e3_aligned16(E) || !e3_aligned16(out)) return EAGLE3_ERR_ARG;
    const int row_vec = (int)((size_t)K * esz / 16);
    embed_kernel<<<grid1((size_t)M * row_vec), 256, 0, e3_stream(stream)>>>((const uint4 *)E, ids, M, row_vec, V,
                                                                           (uint4 *)out);
    E3_LAUNCH_CHECK();
    return EAGLE3_OK;
}

extern "C" int eagle3_commit_kv(const void *k_rows, const void *v_rows, int rows_per_seq, const int32_t *src,
                                int max_n, int B, int Hkv, int D, int dtype, void *k_cache, void *v_cache,
                                const int32_t *block_table, int max_blocks, int num_blocks, const int32_t *start,
                                void *stream) {
    if (B < 0 || max_n < 0 || rows_per_seq < 1 || Hkv < 1 || D < 1 || max_blocks < 1 || num_blocks < 1)
        return EAGLE3_ERR_ARG;
    if (dtype != EAGLE3_BF16 && dtype != EAGLE3_F32) return EAGLE3_ERR_UNSUPPORTED;
    if (B == 0 || max_n == 0) return EAGLE3_OK;
    if (!k_rows || !v_rows || !k_cache || !v_cache || !block_table || !start) return EAGLE3_ERR_ARG;
    if (B > 65535) return EAGLE3_ERR_UNSUPPORTED;
    dim3 grid(max_n, B);
    if (dtype == EAGLE3_BF16)
        commit_kv_kernel<true><<<grid, 256, 0, e3_stream(stream)>>>(k_rows, v_rows, rows_per_seq, src, max_n, Hkv, D,
                                                                   k_cache, v_cache, block_table, max_blocks,
                                                                   num_blocks, start);
    else
        commit_kv_kernel<false><<<grid, 256, 0, e3_stream(stream)>>>(k_rows, v_rows, rows_per_seq, src, max_n, Hkv, D,
                                                                    k_cache, v_cache, block_table, max_blocks,
                                                                    num_blocks, start);
    E3_LAUNCH_CHECK();
    return EAGLE3_OK;
}

extern "C" int eagle3_copy_rows(const void *src, const int32_t *src_rows, int src_nrows, void *dst,
                                const int32_t *dst_rows, int dst_nrows, int n, size_t row_bytes, void *stream) {
    if (n < 0 || src_nrows < 0 || dst_nrows < 0 || row_bytes == 0) return EAGLE3_ERR_ARG;
    if (row_bytes % 16 != 0 || row_bytes / 16 > 0x7fffffff) return EAGLE3_ERR_UNSUPPORTED;
    if (n == 0) return EAGLE3_OK;
    if (!src || !dst || !e3_aligned16(src) || !e3_aligned16(dst)) return EAGLE3_ERR_ARG;
    const int row_vec = (int)(row_bytes / 16);
    copy_rows_kernel<<<grid1((size_t)n * row_vec), 256, 0, e3_stream(stream)>>>(
        (const uint4 *)src, src_rows, src_nrows, (uint4 *)dst, dst_rows, dst_nrows, n, row_vec);
    E3_LAUNCH_CHECK();
    return EAGLE3_OK;
}
