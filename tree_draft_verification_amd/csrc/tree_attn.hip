// Tree attention: every draft-tree node attends to its sequence's paged KV
// prefix plus its own ancestors (course lesson "EAGLE-3 speculative decoding:
// the tree-verifier method", section "Tree draft vs chain draft": one target
// pass over the whole tree, masked so a token sees only its ancestors).
// GQA reading: query head h uses KV head h / (Hq / Hkv).
//
// bf16, D = 128 (MFMA path). One work-group of 4 waves per (sequence, KV
// head, prefix split, block of 256 query rows); a query row is (node,
// head-in-group), so the G query heads sharing a KV head share every K/V tile.
//   - K/V tiles of 64 keys are staged from the paged cache through registers
//     into a double buffer in LDS with 16-byte loads; each 16-token cache
//     block is one contiguous 4 KB run for K ([block, head, slot, d]) and for
//     V ([block, head, d, slot]). The V layout keeps keys contiguous per
//     dimension, which is what the PV product needs as its contraction operand.
//   - Each wave owns 2 x 32 query rows. S^T = K . Q^T by MFMA 32x32x16, so
//     every lane holds one query's scores: the softmax max and sum are in-lane
//     plus one exchange between the two half-waves. Online softmax in fp32
//     with log2(e) folded into the scale, raw v_exp_f32, and a lazily
//     refreshed running max (O is rescaled only when the max grows by more
//     than 2^8). K rows sit in LDS in a permuted key order so that each lane's
//     8 scores per 16-key step are consecutive keys and the V operand is one
//     read. O^T += V^T . P^T by MFMA with P split into bf16 hi + lo parts, so
//     P keeps ~16 significant bits.
//   - The work-group holding the end of a prefix also processes the tree keys
//     under the ancestor mask. Prefix splits over work-groups write partials
//     (normalised O, max, sum) that a second kernel merges in split order.
// fp32 (any D <= 128): one 64-lane wave per query row, lanes over keys for
// the scores and over dimensions for P.V; for small models.
#include "common.h"

#include <algorithm>
#include <type_traits>

namespace {

constexpr int KT = 64;       // keys per tile
constexpr int DH = 128;      // head dim of the MFMA path
constexpr int ATT_NW = 8;                           // waves per work-group
constexpr int ROWS_PER_WG = ATT_NW * 32;            // query rows per work-group
constexpr int ATT_WG_PER_CU = 1;                    // work-groups resident per CU
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr long MIN_SPLIT_KEYS = 256;  // shortest automatic prefix split

struct AttnParams {
    const uint16_t *q, *k_tree, *v_tree, *k_cache, *v_cache;
    const int32_t *block_table, *prefix_len;
    const uint64_t *mask;
    const int32_t *parent;
    uint16_t *out;
    float *lse;
    float *ws_o;     // [B, Hkv, nsplit, Rpad, D]: normalised O of each split
    float *ws_ml;    // [B, Hkv, nsplit, Rpad, 2]: running max (log2 units) and sum
    int B, Tq, Tk, Hq, Hkv, W, G, R, Rpad, nrb, nsplit, split_keys, max_blocks, num_blocks;
    int nunits;      // B * Hkv * nsplit work units of nrb work-groups each
    float zero;      // 0.0f, a value the compiler cannot fold (see attend_tile)
    float scale_log2;
};

// prefix length as the kernels use it: clamped to the block table's capacity
// (and 0 with an empty pool), so bad data can never index out of bounds
__device__ __forceinline__ int clamped_len(const int32_t *prefix_len, int b, int max_blocks, int bs, int num_blocks) {
    const int L = prefix_len[b];
    if (num_blocks <= 0) return 0;
    return max(0, min(L, max_blocks * bs));
}

// Splits of one sequence: prefix splits of split_keys keys; the last one also
// takes the tree keys (an empty prefix still makes one split).
__device__ __forceinline__ int splits_of(int L, int split_keys) {
    const int npre = L > 0 ? (L + split_keys - 1) / split_keys : 0;
    return npre > 0 ? npre : 1;
}

// Sequences are dealt to work-group slots longest (clamped) prefix first,
// ties by lower index: the long sequences start in the first pass over the
// CUs and the short ones fill in behind them (longest-processing-time-first
// list order), instead of the batch order, which can leave a CU with two
// long sequences. The work-group puts the clamped lengths in LDS, thread j
// ranks sequence j by counting, and slot r takes the sequence of rank r.
// Past LPT_MAX_B sequences the batch order is kept.
constexpr int LPT_MAX_B = 256;
struct LptShared {
    int len[LPT_MAX_B];
    int sel;
};
template <int NT>
__device__ __forceinline__ int seq_of_slot(LptShared &sh, const int32_t *prefix_len, int B, int r, int max_blocks,
                                           int num_blocks) {
    static_assert(NT >= LPT_MAX_B, "one ranking thread per sequence");
    if (B > LPT_MAX_B) return r;
    const int j = threadIdx.x;
    const int Lj = j < B ? clamped_len(prefix_len, j, max_blocks, 16, num_blocks) : -1;
    if (j < LPT_MAX_B) sh.len[j] = Lj;  // -1 past B: never ranked ahead
    __syncthreads();
    if (j < B) {
        int rank = 0;
        for (int k0 = 0; k0 < B; k0 += 4) {
            const int4 l4 = *reinterpret_cast<const int4 *>(&sh.len[k0]);  // same address in every lane
            rank += (l4.x > Lj || (l4.x == Lj && k0 < j)) ? 1 : 0;
            rank += (l4.y > Lj || (l4.y == Lj && k0 + 1 < j)) ? 1 : 0;
            rank += (l4.z > Lj || (l4.z == Lj && k0 + 2 < j)) ? 1 : 0;
            rank += (l4.w > Lj || (l4.w == Lj && k0 + 3 < j)) ? 1 : 0;
        }
        if (rank == r) sh.sel = j;
    }
    __syncthreads();
    return sh.sel;
}

__device__ __forceinline__ int clamped_block(const int32_t *btab, int j, int num_blocks) {
    return min(max(btab[j], 0), num_blocks - 1);
}

// ancestor words of node t of sequence b (mask given or walked from parent[])
__device__ __forceinline__ void query_mask(const AttnParams &p, int b, int t, uint64_t &w0, uint64_t &w1) {
    w0 = 0; w1 = 0;
    if (p.mask) {
        const uint64_t *m = p.mask + ((size_t)b * p.Tq + t) * p.W;
        w0 = m[0];
        if (p.W > 1) w1 = m[1];
    } else {
        int cur = t;
        for (int steps = 0; steps < p.Tq && cur >= 0 && cur < p.Tq; ++steps) {
            if (cur < 64) w0 |= (uint64_t)1 << cur;
            else w1 |= (uint64_t)1 << (cur - 64);
            cur = p.parent[(size_t)b * p.Tq + cur];
        }
    }
}

enum TileKind { TILE_FULL = 0, TILE_PARTIAL = 1, TILE_TREE = 2 };

// Softmax bookkeeping is in log2 units with a lazily refreshed running max:
// m_run only moves when a score exceeds it by more than 2^8 (so exp2 values
// stay below 256, harmless in fp32), which makes O rescaling rare.
constexpr float kLazyMax = 8.f;

// K rows (one key, 256 B of d) are padded to KROW = 272 bytes: a K fragment
// read takes 32 consecutive rows at one column, and the 16-byte shift per row
// spreads each 8 lanes over 8 distinct bank groups. The padding (rather than a
// lane-dependent column swizzle) keeps the column offset of every QK step a
// constant, so the reads need one address register.
constexpr int KROW = DH * 2 + 16;
constexpr int VOFF = KT * KROW;            // V tile offset inside a buffer
constexpr int TILE_BYTES = VOFF + KT * DH * 2;  // K tile (17 KB) + V tile (16 KB)
constexpr int NBUF = 2;                    // tile buffers in LDS
// V rows are (block, d) pairs of 32 B = 16 slots; the two 16-byte halves are
// swapped on every other group of 8 rows, halving bank conflicts of PV reads.
__device__ __forceinline__ int vswz(int d) { return (d >> 3) & 1; }
// Key held by K-tile row r: bits 2 and 3 of the key swapped. The S^T
// accumulator gives lane half h the rows 8a + 4h + c (a in {0,1}, c in 0..3)
// of each 16-row group, i.e. keys 8h + 4a + c: eight consecutive keys, which
// is one 16-byte half of a V row, so the PV operand is a single LDS read.
__device__ __forceinline__ int row_key(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// compile-time unrolled loop: f(std::integral_constant<int, i>) for i in [I, N)
template <int I, int N, typename F>
__device__ __forceinline__ void sfor(F &&f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        sfor<I + 1, N>(f);
    }
}

constexpr int QK_AHEAD = 4;  // fragment reads in flight ahead of the MFMAs

// A 64-key tile for one wave and its RB blocks of 32 query rows runs in three
// phases: qk_tile (S^T = K.Q^T), softmax_tile (online softmax)
// and pv_tile (O^T += V^T.P^T). Every K / V fragment read from LDS feeds the
// MFMAs of all RB row blocks.
//   QK step (s, kb): K rows 32 kb + lr, 16-byte column 2 s + lh,
//   i.e. keys of block kb and d = 16 s + 8 lh .. +7; the Q^T operand holds
//   the same d of this lane's query row.
//   PV step (ks, db): V row (16-key block ks, d = 32 db + lr), half lh: keys
//   16 ks + 8 lh .. +7; the P^T operand holds this lane's P for those keys.
// Register r of score block kb holds key 32 kb + 16 (r / 8) + 8 lh + (r % 8).

// QK step j: key block kb = j & 1, d-step s = j >> 1. Fragment reads run
// QK_AHEAD steps ahead of the MFMAs; the scheduling barriers keep the
// compiler from sinking each read next to its MFMA (which leaves the LDS
// latency exposed at every step). The score accumulators start as registers
// holding a zero the compiler cannot see: with a literal zero the first MFMA
// takes the inline-zero C operand, and its destination is then free to
// overlap the A operand.
template <int RB>
__device__ __forceinline__ void qk_tile(const unsigned char *tile, const u32x4_t (&qb)[RB][8], f32x16_t (&st)[RB][2],
                                        int lr, int lh, float zero) {
#pragma unroll
    for (int k = 0; k < RB; ++k)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) st[k][kb][r] = zero;
    const unsigned char *krow = tile + lr * KROW + lh * 16;
    u32x4_t fk[16];
    auto kread = [&](auto J) {
        constexpr int j = J, kb = j & 1, s = j >> 1;
        fk[j] = *reinterpret_cast<const u32x4_t *>(krow + kb * 32 * KROW + s * 32);
    };
    sfor<0, QK_AHEAD>(kread);
    sfor<0, 16>([&](auto J) {
        constexpr int j = J, kb = j & 1, s = j >> 1;
        if constexpr (j + QK_AHEAD < 16) kread(std::integral_constant<int, j + QK_AHEAD>{});
#pragma unroll
        for (int k = 0; k < RB; ++k)
            st[k][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, fk[j]),
                                                                __builtin_bit_cast(bf16x8_t, qb[k][s]), st[k][kb], 0,
                                                                0, 0);
        __builtin_amdgcn_sched_barrier(0);
    });
}

// Online softmax of one tile's scores, in place: st then holds P (fp32).
// kind is wave-uniform.
template <int RB>
__device__ __forceinline__ void softmax_tile(int kind, int nvalid, const uint64_t (&mword)[RB], f32x16_t (&st)[RB][2],
                                             f32x16_t (&ot)[RB][4], float (&m_run)[RB],
                                             float (&l_run)[RB], int lh, float scale_log2) {
#pragma unroll
    for (int k = 0; k < RB; ++k) {
        if (kind != TILE_FULL) {
            // visible keys of the tile (bit kk); each group of 8 registers
            // holds 8 consecutive keys, whose bits are one byte of the word
            uint64_t vis = nvalid >= KT ? ~0ull : (1ull << nvalid) - 1;
            if (kind == TILE_TREE) vis &= mword[k];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int a = 0; a < 2; ++a) {
                    const uint32_t byte = (uint32_t)(vis >> (kb * 32 + 16 * a + 8 * lh));
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const uint32_t m = (uint32_t)((int32_t)(byte << (31 - e)) >> 31);  // all ones iff visible
                        const uint32_t x = __float_as_uint(st[k][kb][8 * a + e]);
                        st[k][kb][8 * a + e] = __uint_as_float((x & m) | (0xff800000u & ~m));
                    }
                }
        }
        float tmax = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, st[k][kb][r]);
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32)) * scale_log2;
        // refresh the running max only when it is exceeded by more than 2^kLazyMax
        const bool grow = tmax > m_run[k] + kLazyMax;
        if (__ballot(grow)) {
            const float m_new = grow ? tmax : m_run[k];
            const float alpha = (m_run[k] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run[k] - m_new);
            l_run[k] *= alpha;
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) ot[k][db][r] *= alpha;
            m_run[k] = m_new;
        }
        const float msub = (m_run[k] == -INFINITY) ? 0.f : m_run[k];
        float psum = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float pv = __builtin_amdgcn_exp2f(fmaf(st[k][kb][r], scale_log2, -msub));
                st[k][kb][r] = pv;
                psum += pv;
            }
        l_run[k] += psum;
    }
}

// PV step j: 16-key step ks = j >> 2, d block db = j & 3; reads run QK_AHEAD
// steps ahead as in qk_tile. P enters as bf16 hi + lo parts (two MFMAs on
// the same V operand), so it keeps ~16 significant bits: a single rounding to
// bf16 (8 bits) or fp16 (11 bits) moves enough output elements across a bf16
// rounding boundary to flip argmax decisions downstream whose top-2 logit
// gap is above 1e-3.
template <int RB>
__device__ __forceinline__ void pv_tile(const unsigned char *tile, const f32x16_t (&st)[RB][2], f32x16_t (&ot)[RB][4],
                                        int lr, int lh) {
    const unsigned char *vrow = tile + VOFF + lr * 32 + ((lh ^ vswz(lr)) << 4);
    u32x4_t fv[16];
    auto vread = [&](auto J) {
        constexpr int j = J, ks = j >> 2, db = j & 3;
        fv[j] = *reinterpret_cast<const u32x4_t *>(vrow + ks * 4096 + db * 1024);
    };
    sfor<0, QK_AHEAD>(vread);
    u32x4_t ph[RB], pl[RB];
    sfor<0, 16>([&](auto J) {
        constexpr int j = J, ks = j >> 2, db = j & 3;
        if constexpr (db == 0) {
            constexpr int kb = ks >> 1, r0 = 8 * (ks & 1);
#pragma unroll
            for (int k = 0; k < RB; ++k)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    uint32_t h2, l2;
                    e3_split_bf16x2(st[k][kb][r0 + 2 * e], st[k][kb][r0 + 2 * e + 1], h2, l2);
                    ph[k][e] = h2;
                    pl[k][e] = l2;
                }
        }
        if constexpr (j + QK_AHEAD < 16) vread(std::integral_constant<int, j + QK_AHEAD>{});
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, fv[j]);
#pragma unroll
        for (int k = 0; k < RB; ++k) {
            ot[k][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8_t, ph[k]), ot[k][db], 0, 0,
                                                               0);
            ot[k][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8_t, pl[k]), ot[k][db], 0, 0,
                                                               0);
        }
        __builtin_amdgcn_sched_barrier(0);
    });
}

// Work-group -> work unit. Work-groups are dealt to the 8 XCDs round-robin
// (work-group i runs on XCD i mod 8, each XCD with its own L2). The nrb row
// blocks of one (sequence, KV head, split) read the same K/V, so they are
// given ids i, i + 8, ...: one XCD, dispatched together, and the second
// read of every tile is an L2 hit. Units are numbered so that dispatch order
// follows the slot order (longest prefix first).
struct WorkUnit {
    int unit, rblk;
};
__device__ __forceinline__ WorkUnit work_unit(int i, int nrb) {
    const int xcd = i & 7, j = i >> 3;
    WorkUnit w;
    w.rblk = j % nrb;
    w.unit = (j / nrb) * 8 + xcd;
    return w;
}

// One work-group per (sequence slot, KV head, prefix split, block of 256 query
// rows); NW waves of RB x 32 rows. K/V tiles are double-buffered in LDS: while
// a tile is attended, every thread holds its share of the next tile (NCH
// 16-byte chunks of K and NCH of V) in registers, loaded at the start of the
// tile and written to the other buffer at its end; one barrier per tile.
template <int NW, int RB>
__global__ __launch_bounds__(NW * 64, ATT_WG_PER_CU) void tree_attn_bf16_kernel(AttnParams p) {
    static_assert(NW * RB * 32 == ROWS_PER_WG, "a work-group covers one block of query rows");
    constexpr int NT = NW * 64;
    constexpr int NCH = KT * DH / 8 / NT;  // 16-byte chunks of K (and of V) per thread and tile
    static_assert(NCH * NT * 8 == KT * DH && NT % 256 == 0, "whole 4 KB cache blocks per 256 threads");
    __shared__ __attribute__((aligned(1024))) unsigned char buf[NBUF * TILE_BYTES];

    const WorkUnit wu = work_unit(blockIdx.x, p.nrb);
    if (wu.unit >= p.nunits) return;
    const int split = wu.unit % p.nsplit, kvh = (wu.unit / p.nsplit) % p.Hkv, slot = wu.unit / (p.nsplit * p.Hkv);
    const int rblk = wu.rblk;
    __shared__ __attribute__((aligned(16))) LptShared lpt;
    const int b =
        __builtin_amdgcn_readfirstlane(seq_of_slot<NT>(lpt, p.prefix_len, p.B, slot, p.max_blocks, p.num_blocks));
    const int L = clamped_len(p.prefix_len, b, p.max_blocks, 16, p.num_blocks);
    const int C = p.split_keys;
    const int nsplit_b = splits_of(L, C);
    if (split >= nsplit_b) return;
    const bool last = split == nsplit_b - 1;  // this split also takes the tree keys
    const int k_begin = split * C;
    const int k_end = min(L, k_begin + C);
    const int npre = (k_end - k_begin + KT - 1) / KT;
    const int ntiles = npre + (last ? (p.Tk + KT - 1) / KT : 0);

    // the wave index is wave-uniform; saying so keeps the branches on it scalar
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int lr = lane & 31, lh = lane >> 5;
    int row[RB], t[RB], hq[RB];
    bool row_ok[RB];
#pragma unroll
    for (int k = 0; k < RB; ++k) {
        row[k] = rblk * ROWS_PER_WG + (wave * RB + k) * 32 + lr;
        row_ok[k] = row[k] < p.R;
        t[k] = row_ok[k] ? row[k] / p.G : 0;
        hq[k] = kvh * p.G + (row_ok[k] ? row[k] % p.G : 0);
    }
    const bool wave_active = rblk * ROWS_PER_WG + wave * RB * 32 < p.R;

    // Staging. Chunk i of a thread is 16-key block jb = i NT / 256 + tid / 256
    // of the tile and the w-th 16 bytes of it, w = tid % 256: for K the key
    // 16 jb + w / 16, 16-byte column w % 16; for V (cache layout [d][16 slots]
    // per block) the dimension d = w / 2, slots 8 (w % 2) .. +7. In the cache
    // both are the w-th 16 bytes of the block's contiguous 4 KB run.
    const int32_t *btab = p.block_table + (size_t)b * p.max_blocks;
    const size_t head_off = (size_t)kvh * 16 * DH;
    const size_t blk_stride = (size_t)p.Hkv * 16 * DH;
    // jb_t is wave-uniform: block ids are then scalar loads, which do not
    // hold up the vector loads of the tile behind them
    const int w = tid & 255, jb_t = __builtin_amdgcn_readfirstlane(tid >> 8);
    u32x4_t sk[NCH], sv[NCH];
    // Loads are unconditional, from clamped addresses (blocks past the end of
    // the range re-read its last block, tree keys past Tk re-read key Tk - 1);
    // write_tile zeroes what they stand for. A conditional load into a
    // zeroed register would make every later write of that register wait
    // for the load.
    const int last_blk = max(k_end - 1, k_begin) / 16;
    // block ids are fetched one tile ahead of the staging loads that use them
    int raw_id[NCH];
    auto fetch_ids = [&](int it) {
        if (it < npre) {
            const int blk0 = (k_begin + it * KT) / 16;
#pragma unroll
            for (int i = 0; i < NCH; ++i) raw_id[i] = btab[min(blk0 + i * (NT / 256) + jb_t, last_blk)];
        }
    };
    const uint32_t lane_off = (uint32_t)w * 16;
    auto load_tile = [&](int it) {
        if (it < npre) {
#pragma unroll
            for (int i = 0; i < NCH; ++i) {
                // the block's base address is wave-uniform (scalar); each lane
                // adds its fixed 32-bit byte offset w * 16
                const int bid = __builtin_amdgcn_readfirstlane(min(max(raw_id[i], 0), p.num_blocks - 1));
                const size_t boff = (size_t)bid * blk_stride + head_off;
                const unsigned char *kb = reinterpret_cast<const unsigned char *>(p.k_cache + boff);
                const unsigned char *vb = reinterpret_cast<const unsigned char *>(p.v_cache + boff);
                sk[i] = *reinterpret_cast<const u32x4_t *>(kb + lane_off);
                sv[i] = *reinterpret_cast<const u32x4_t *>(vb + lane_off);
            }
        } else {
            const int tk0 = (it - npre) * KT;
#pragma unroll
            for (int i = 0; i < NCH; ++i) {
                const int jb = i * (NT / 256) + jb_t;
                const int tk = min(tk0 + 16 * jb + (w >> 4), p.Tk - 1);
                const size_t off = (((size_t)b * p.Tk + tk) * p.Hkv + kvh) * DH + (w & 15) * 8;
                sk[i] = *reinterpret_cast<const u32x4_t *>(p.k_tree + off);
                sv[i] = *reinterpret_cast<const u32x4_t *>(p.v_tree + off);
            }
        }
    };
    auto write_tile = [&](int it, unsigned char *dst) {
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int jb = i * (NT / 256) + jb_t;
            const int r = 16 * jb + row_key(w >> 4);  // the row holding key 16 jb + w / 16
            *reinterpret_cast<u32x4_t *>(dst + r * KROW + (w & 15) * 16) = sk[i];
        }
        if (it < npre) {
            const int nval = min(KT, k_end - (k_begin + it * KT));
            const int d = w >> 1, half = w & 1;
#pragma unroll
            for (int i = 0; i < NCH; ++i) {
                const int jb = i * (NT / 256) + jb_t;
                u32x4_t v = sv[i];
                // slots past the prefix are zeroed: the cache may hold anything
                // there, and 0 * NaN would poison the sum
                const int k0 = 16 * jb + 8 * half;
                if (k0 + 8 > nval) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t lo = (k0 + 2 * e < nval) ? 0x0000ffffu : 0u;
                        const uint32_t hi = (k0 + 2 * e + 1 < nval) ? 0xffff0000u : 0u;
                        v[e] &= lo | hi;
                    }
                }

                *reinterpret_cast<u32x4_t *>(dst + VOFF + jb * 4096 + d * 32 + ((half ^ vswz(d)) << 4)) = v;
            }
        } else {
            // tree V rows arrive key-major ([key][d]): transpose into the
            // [block][d][slot] layout, one 2-byte store per element
            const int d8 = (w & 15) * 8, sl = w >> 4;
#pragma unroll
            for (int i = 0; i < NCH; ++i) {
                const int jb = i * (NT / 256) + jb_t;
                const bool key_ok = (it - npre) * KT + 16 * jb + sl < p.Tk;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int d = d8 + e;
                    const uint32_t word = key_ok ? sv[i][e >> 1] : 0u;
                    const uint16_t val = (uint16_t)((e & 1) ? (word >> 16) : (word & 0xffffu));
                    reinterpret_cast<uint16_t *>(dst + VOFF + jb * 4096 + d * 32)[((sl >> 3) ^ vswz(d)) * 8 + (sl & 7)] =
                        val;
                }
            }
        }
    };

    // Prologue: the block ids of tile 0 go out first, then q and the mask
    // words, then tile 0 itself (two memory round trips in all)
    fetch_ids(0);
    // Q^T operand: d = 16 s + 8 lh + i
    u32x4_t qb[RB][8];
    uint64_t mw0[RB], mw1[RB];
#pragma unroll
    for (int k = 0; k < RB; ++k) {
        const uint16_t *qrow = p.q + (((size_t)b * p.Tq + t[k]) * p.Hq + hq[k]) * DH + 8 * lh;
#pragma unroll
        for (int s = 0; s < 8; ++s)
            qb[k][s] = row_ok[k] ? *reinterpret_cast<const u32x4_t *>(qrow + 16 * s) : u32x4_t{0u, 0u, 0u, 0u};
        mw0[k] = 0; mw1[k] = 0;
        if (last && row_ok[k]) query_mask(p, b, t[k], mw0[k], mw1[k]);
    }

    f32x16_t ot[RB][4];
    float m_run[RB], l_run[RB];
#pragma unroll
    for (int k = 0; k < RB; ++k) {
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) ot[k][db][r] = 0.f;
        m_run[k] = -INFINITY;
        l_run[k] = 0.f;
    }

    if (ntiles > 0) load_tile(0);
    fetch_ids(1);
    // everything above has landed before the loop: otherwise a wait for q or
    // the mask words, placed inside the loop, would also wait for the staging
    // loads of the next tile
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), expcnt and lgkmcnt not waited
    if (ntiles > 0) write_tile(0, buf);
    __syncthreads();
    if (ntiles > 1) load_tile(1);
    fetch_ids(2);

    // Every wave attends tile it (QK, softmax, PV from buffer it % 2), then
    // writes its share of tile it+1 (loaded since the previous barrier) into
    // the other buffer, whose last readers finished before that barrier, and
    // meets the barrier; the loads of tile it+2 go out right after it.
    f32x16_t st[RB][2];
    for (int it = 0; it < ntiles; ++it) {
        const unsigned char *cur = buf + (it % NBUF) * TILE_BYTES;
        if (wave_active) {
            int kind, nvalid;
            uint64_t mword[RB];
            if (it < npre) {
                nvalid = k_end - (k_begin + it * KT);
                kind = nvalid >= KT ? TILE_FULL : TILE_PARTIAL;
#pragma unroll
                for (int k = 0; k < RB; ++k) mword[k] = 0;
            } else {
                const int tt = it - npre;
                nvalid = p.Tk - tt * KT;
                kind = TILE_TREE;
#pragma unroll
                for (int k = 0; k < RB; ++k) mword[k] = tt == 0 ? mw0[k] : mw1[k];
            }
            qk_tile<RB>(cur, qb, st, lr, lh, p.zero);
            softmax_tile<RB>(kind, nvalid, mword, st, ot, m_run, l_run, lh, p.scale_log2);
            pv_tile<RB>(cur, st, ot, lr, lh);
        }
        if (it + 1 < ntiles) write_tile(it + 1, buf + ((it + 1) % NBUF) * TILE_BYTES);
        __syncthreads();
        if (it + 2 < ntiles) load_tile(it + 2);
        fetch_ids(it + 3);
    }

#pragma unroll
    for (int k = 0; k < RB; ++k) {
        if (!row_ok[k]) continue;
        const float l_tot = l_run[k] + __shfl_xor(l_run[k], 32);
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        // lane holds d = 32 db + 8 (r / 4) + 4 lh + r % 4 for its query
        if (nsplit_b == 1) {
            uint16_t *orow = p.out + (((size_t)b * p.Tq + t[k]) * p.Hq + hq[k]) * DH;
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int d = db * 32 + 8 * g4 + 4 * lh;
                    u32x2_t o;
                    o[0] = e3_pack_bf16x2(ot[k][db][4 * g4] * inv, ot[k][db][4 * g4 + 1] * inv);
                    o[1] = e3_pack_bf16x2(ot[k][db][4 * g4 + 2] * inv, ot[k][db][4 * g4 + 3] * inv);
                    *reinterpret_cast<u32x2_t *>(orow + d) = o;
                }
            if (p.lse && lh == 0)
                p.lse[((size_t)b * p.Tq + t[k]) * p.Hq + hq[k]] =
                    l_tot > 0.f ? (m_run[k] + log2f(l_tot)) * kLn2 : -INFINITY;
        } else {
            // the split's normalised O in fp32 (rounding it to 16 bits here
            // would cost the merged result more than its final bf16 rounding)
            const size_t prow = (((size_t)b * p.Hkv + kvh) * p.nsplit + split) * p.Rpad + row[k];
            float *orow = p.ws_o + prow * DH;
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int d = db * 32 + 8 * g4 + 4 * lh;
                    f32x4_t o = {ot[k][db][4 * g4] * inv, ot[k][db][4 * g4 + 1] * inv, ot[k][db][4 * g4 + 2] * inv,
                                 ot[k][db][4 * g4 + 3] * inv};
                    *reinterpret_cast<f32x4_t *>(orow + d) = o;
                }
            if (lh == 0) {
                p.ws_ml[prow * 2] = m_run[k];
                p.ws_ml[prow * 2 + 1] = l_tot;
            }
        }
    }
}

// Merge split partials of multi-split sequences, in split order.
__global__ __launch_bounds__(128) void tree_attn_combine_kernel(AttnParams p) {
    const int idx = blockIdx.x;  // (b, t, hq)
    const int hq = idx % p.Hq, t = (idx / p.Hq) % p.Tq, b = idx / (p.Hq * p.Tq);
    const int L = clamped_len(p.prefix_len, b, p.max_blocks, 16, p.num_blocks);
    const int nsplit_b = splits_of(L, p.split_keys);
    if (nsplit_b <= 1) return;
    const int kvh = hq / p.G, row = t * p.G + hq % p.G;
    const size_t base = ((size_t)b * p.Hkv + kvh) * p.nsplit;
    float M = -INFINITY;
    for (int s = 0; s < nsplit_b; ++s) M = fmaxf(M, p.ws_ml[((base + s) * p.Rpad + row) * 2]);
    const int d = threadIdx.x;
    float acc = 0.f, den = 0.f;
    for (int s = 0; s < nsplit_b; ++s) {
        const size_t prow = (base + s) * p.Rpad + row;
        const float ms = p.ws_ml[prow * 2], ls = p.ws_ml[prow * 2 + 1];
        const float wgt = (ms == -INFINITY) ? 0.f : ls * exp2f(ms - M);
        acc += wgt * p.ws_o[prow * DH + d];
        den += wgt;
    }
    const float o = den > 0.f ? acc / den : 0.f;
    p.out[(((size_t)b * p.Tq + t) * p.Hq + hq) * DH + d] = e3_f32_to_bf16(o);
    if (p.lse && d == 0)
        p.lse[((size_t)b * p.Tq + t) * p.Hq + hq] = den > 0.f ? (M + log2f(den)) * kLn2 : -INFINITY;
}

// Combine and RMSNorm in one pass: one work-group per (sequence, node) row
// merges the split partials of all Hq heads (split weights per head in LDS),
// writes the attention output row and its RMSNorm (gamma = 1) computed from
// the stored bf16 values, as the separate norm would. A sequence with a
// single split has no partials: the attention pass wrote its row and lse
// itself, and this pass only reads the row back for the norm.
// 512 threads, 8 elements each per pass (one pass for a 4096-wide row), and
// the partial loads of up to 16 splits in flight together: a row costs about
// two dependent memory round trips (weights, then partials), which is what
// bounds this pass at the few-row shapes where it runs.
constexpr int CN_MAXS = 32;   // splits per sequence the fused pass handles
constexpr int CN_MAXH = 64;   // query heads the fused pass handles
constexpr int CN_NT = 512;    // threads per work-group
constexpr int CN_BATCH = 16;  // splits whose partial loads are in flight together

__global__ __launch_bounds__(CN_NT) void tree_attn_combine_norm_kernel(AttnParams p, uint16_t *__restrict__ norm_out,
                                                                       float eps) {
    static_assert(CN_MAXS == 32 && CN_MAXH == CN_NT / 8, "8 lanes x 4 splits per head, all heads in one pass");
    __shared__ float wgt[CN_MAXH][CN_MAXS];
    __shared__ float red[CN_NT / 64];
    const int t = blockIdx.x % p.Tq, b = blockIdx.x / p.Tq;
    const int L = clamped_len(p.prefix_len, b, p.max_blocks, 16, p.num_blocks);
    const int nsplit_b = splits_of(L, p.split_keys);
    const bool direct = nsplit_b == 1;  // uniform over the work-group
    // split weights: 8 lanes per head, lane j takes splits j, j+8, j+16, j+24
    // (all loads issued together), max and sum over the 8 lanes by shuffles
    const int hq_w = threadIdx.x >> 3;
    if (!direct && hq_w < p.Hq) {
        const int j = threadIdx.x & 7, hq = hq_w;
        const int kvh = hq / p.G, row = t * p.G + hq % p.G;
        const size_t base = ((size_t)b * p.Hkv + kvh) * p.nsplit;
        float ms[4], ls[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int sp = j + 8 * u;
            ms[u] = -INFINITY; ls[u] = 0.f;
            if (sp < nsplit_b) {
                const f32x2_t ml = *reinterpret_cast<const f32x2_t *>(p.ws_ml + ((base + sp) * p.Rpad + row) * 2);
                ms[u] = ml[0]; ls[u] = ml[1];
            }
        }
        float M = fmaxf(fmaxf(ms[0], ms[1]), fmaxf(ms[2], ms[3]));
#pragma unroll
        for (int off = 1; off < 8; off <<= 1) M = fmaxf(M, __shfl_xor(M, off));
        float w[4], den = 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            w[u] = (ms[u] == -INFINITY) ? 0.f : ls[u] * exp2f(ms[u] - M);
            den += w[u];
        }
#pragma unroll
        for (int off = 1; off < 8; off <<= 1) den += __shfl_xor(den, off);
        const float inv = den > 0.f ? 1.f / den : 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u) wgt[hq][j + 8 * u] = w[u] * inv;   // zero past nsplit_b
        if (p.lse && j == 0)
            p.lse[((size_t)b * p.Tq + t) * p.Hq + hq] = den > 0.f ? (M + log2f(den)) * kLn2 : -INFINITY;
    }
    __syncthreads();
    const int K = p.Hq * DH;
    float v[2][8];  // this thread's 8 consecutive elements of each pass (K <= 8192)
    float ss = 0.f;
    uint16_t *orow = p.out + ((size_t)b * p.Tq + t) * K;
#pragma unroll
    for (int ps = 0; ps < 2; ++ps) {
        const int c = (ps * CN_NT + threadIdx.x) * 8;
        if (c >= K) break;
        u32x4_t packed;
        if (direct) {
            packed = *reinterpret_cast<const u32x4_t *>(orow + c);
        } else {
            const int hq = c / DH, d = c % DH;
            const int kvh = hq / p.G, row = t * p.G + hq % p.G;
            const size_t base = ((size_t)b * p.Hkv + kvh) * p.nsplit;
            float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            for (int s0 = 0; s0 < nsplit_b; s0 += CN_BATCH) {
                f32x4_t a[CN_BATCH], c4[CN_BATCH];
#pragma unroll
                for (int u = 0; u < CN_BATCH; ++u) {
                    if (s0 + u < nsplit_b) {  // uniform
                        const float *src = p.ws_o + ((base + s0 + u) * p.Rpad + row) * DH + d;
                        a[u] = *reinterpret_cast<const f32x4_t *>(src);
                        c4[u] = *reinterpret_cast<const f32x4_t *>(src + 4);
                    }
                }
#pragma unroll
                for (int u = 0; u < CN_BATCH; ++u) {
                    if (s0 + u < nsplit_b) {
                        const float w = wgt[hq][s0 + u];
#pragma unroll
                        for (int i = 0; i < 4; ++i) { o[i] += w * a[u][i]; o[4 + i] += w * c4[u][i]; }
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) packed[i] = e3_pack_bf16x2(o[2 * i], o[2 * i + 1]);
            *reinterpret_cast<u32x4_t *>(orow + c) = packed;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[ps][2 * i] = __uint_as_float(packed[i] << 16);
            v[ps][2 * i + 1] = __uint_as_float(packed[i] & 0xffff0000u);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) ss += v[ps][i] * v[ps][i];
    }
    // row sum of squares: waves, then the 8 wave sums
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    float total = 0.f;
#pragma unroll
    for (int w = 0; w < CN_NT / 64; ++w) total += red[w];
    const float r = 1.0f / sqrtf(total / (float)K + eps);
    uint16_t *nrow = norm_out + ((size_t)b * p.Tq + t) * K;
#pragma unroll
    for (int ps = 0; ps < 2; ++ps) {
        const int c = (ps * CN_NT + threadIdx.x) * 8;
        if (c >= K) break;
        u32x4_t packed;
#pragma unroll
        for (int i = 0; i < 4; ++i) packed[i] = e3_pack_bf16x2(v[ps][2 * i] * r, v[ps][2 * i + 1] * r);
        *reinterpret_cast<u32x4_t *>(nrow + c) = packed;
    }
}

// ---------------------------------------------------------------- fp32 path

struct AttnF32 {
    const float *q, *k_tree, *v_tree, *k_cache, *v_cache;
    const int32_t *block_table, *prefix_len;
    const uint64_t *mask;
    const int32_t *parent;
    float *out, *lse;
    int Tq, Tk, Hq, Hkv, D, W, G, max_blocks, block_size, num_blocks;
    float scale;
};

__global__ __launch_bounds__(64) void tree_attn_f32_kernel(AttnF32 p) {
    __shared__ float qs[128];
    __shared__ float ps[64];
    __shared__ int keyref[64];  // >= 0: prefix position; < 0: -(tree key) - 1
    const int idx = blockIdx.x;
    const int hq = idx % p.Hq, t = (idx / p.Hq) % p.Tq, b = idx / (p.Hq * p.Tq);
    const int kvh = hq / p.G, lane = threadIdx.x, D = p.D;
    const int L = clamped_len(p.prefix_len, b, p.max_blocks, p.block_size, p.num_blocks);
    const float *qrow = p.q + (((size_t)b * p.Tq + t) * p.Hq + hq) * D;
    for (int d = lane; d < D; d += 64) qs[d] = qrow[d];
    uint64_t w0 = 0, w1 = 0;
    if (p.mask) {
        const uint64_t *m = p.mask + ((size_t)b * p.Tq + t) * p.W;
        w0 = m[0];
        if (p.W > 1) w1 = m[1];
    } else {
        int cur = t;
        for (int s = 0; s < p.Tq && cur >= 0 && cur < p.Tq; ++s) {
            if (cur < 64) w0 |= (uint64_t)1 << cur; else w1 |= (uint64_t)1 << (cur - 64);
            cur = p.parent[(size_t)b * p.Tq + cur];
        }
    }
    __syncthreads();
    const int32_t *btab = p.block_table + (size_t)b * p.max_blocks;
    const int bs = p.block_size;
    float m_run = -INFINITY, l_run = 0.f;
    float acc0 = 0.f, acc1 = 0.f;  // d = lane, lane + 64
    const int nkeys = L + p.Tk;
    for (int c0 = 0; c0 < nkeys; c0 += 64) {
        const int j = c0 + lane;
        float s = -INFINITY;
        int ref = 0;
        if (j < L) {
            const int blk = clamped_block(btab, j / bs, p.num_blocks);
            const float *kr = p.k_cache + (((size_t)blk * p.Hkv + kvh) * bs + j % bs) * D;
            float dot = 0.f;
            for (int d = 0; d < D; ++d) dot = fmaf(qs[d], kr[d], dot);
            s = dot * p.scale;
            ref = j;
        } else if (j < nkeys) {
            const int tk = j - L;
            const bool vis = tk < 64 ? ((w0 >> tk) & 1u) : ((w1 >> (tk - 64)) & 1u);
            if (vis) {
                const float *kr = p.k_tree + (((size_t)b * p.Tk + tk) * p.Hkv + kvh) * D;
                float dot = 0.f;
                for (int d = 0; d < D; ++d) dot = fmaf(qs[d], kr[d], dot);
                s = dot * p.scale;
            }
            ref = -tk - 1;
        }
        float cmax = s;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) cmax = fmaxf(cmax, __shfl_xor(cmax, off));
        const float m_new = fmaxf(m_run, cmax);
        const float alpha = (m_new == -INFINITY) ? 1.f : expf(m_run - m_new);
        const float pj = (s == -INFINITY) ? 0.f : expf(s - m_new);
        float csum = pj;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) csum += __shfl_xor(csum, off);
        l_run = l_run * alpha + csum;
        m_run = m_new;
        ps[lane] = pj;
        keyref[lane] = ref;
        __syncthreads();
        acc0 *= alpha; acc1 *= alpha;
        const int cn = min(64, nkeys - c0);
        for (int jj = 0; jj < cn; ++jj) {
            const float pv = ps[jj];
            if (pv == 0.f) continue;
            const int r = keyref[jj];
            if (r >= 0) {
                const int blk = clamped_block(btab, r / bs, p.num_blocks);
                const float *vc = p.v_cache + ((size_t)blk * p.Hkv + kvh) * (size_t)D * bs + r % bs;
                if (lane < D) acc0 = fmaf(pv, vc[(size_t)lane * bs], acc0);
                if (lane + 64 < D) acc1 = fmaf(pv, vc[(size_t)(lane + 64) * bs], acc1);
            } else {
                const float *vr = p.v_tree + (((size_t)b * p.Tk + (-r - 1)) * p.Hkv + kvh) * D;
                if (lane < D) acc0 = fmaf(pv, vr[lane], acc0);
                if (lane + 64 < D) acc1 = fmaf(pv, vr[lane + 64], acc1);
            }
        }
        __syncthreads();
    }
    float *orow = p.out + (((size_t)b * p.Tq + t) * p.Hq + hq) * D;
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    if (lane < D) orow[lane] = acc0 * inv;
    if (lane + 64 < D) orow[lane + 64] = acc1 * inv;
    if (p.lse && lane == 0) p.lse[((size_t)b * p.Tq + t) * p.Hq + hq] = l_run > 0.f ? m_run + logf(l_run) : -INFINITY;
}

// Validate mode: one wave per sequence checks the prefix length, the block
// ids the prefix uses and (parent[] mode) the tree order; writes status[b].
__global__ __launch_bounds__(64) void tree_attn_validate_kernel(const int32_t *__restrict__ block_table,
                                                                const int32_t *__restrict__ prefix_len,
                                                                const int32_t *__restrict__ parent, int Tq,
                                                                int max_blocks, int block_size, int num_blocks,
                                                                int32_t *__restrict__ status) {
    const int b = blockIdx.x, lane = threadIdx.x;
    const int L = prefix_len[b];
    bool range_bad = L < 0 || (long)L > (long)max_blocks * block_size;
    const int nb = range_bad ? 0 : (L + block_size - 1) / block_size;
    for (int j = lane; j < nb; j += 64) {
        const int id = block_table[(size_t)b * max_blocks + j];
        range_bad |= id < 0 || id >= num_blocks;
    }
    bool tree_bad = false;
    if (parent)
        for (int n = lane; n < Tq; n += 64) {
            const int pn = parent[(size_t)b * Tq + n];
            tree_bad |= n == 0 ? pn != -1 : (pn < 0 || pn >= n);
        }
    const bool rb = __ballot(range_bad) != 0, tb = __ballot(tree_bad) != 0;
    if (lane == 0) status[b] = rb ? EAGLE3_ERR_RANGE : tb ? EAGLE3_ERR_TREE : EAGLE3_OK;
}

// ---------------------------------------------------------------- host side

struct Plan {
    int nrb, nsplit, split_keys;
    size_t ws_bytes;
};

int check_args(const eagle3_tree_attn_args *a) {
    if (!a) return EAGLE3_ERR_ARG;
    if (a->B < 0 || a->Tq < 1 || a->Tk < 0 || a->Hq < 1 || a->Hkv < 1 || a->max_blocks < 1 || a->num_blocks < 0)
        return EAGLE3_ERR_ARG;
    if (!(a->scale > 0.f)) return EAGLE3_ERR_ARG;
    if (a->Hq % a->Hkv != 0) return EAGLE3_ERR_UNSUPPORTED;
    if (a->W < 1 || a->W > 2 || a->Tk > 64 * a->W) return EAGLE3_ERR_UNSUPPORTED;
    if (a->block_size != 16) return EAGLE3_ERR_UNSUPPORTED;
    if (a->dtype == EAGLE3_BF16) {
        if (a->D != 128) return EAGLE3_ERR_UNSUPPORTED;
    } else if (a->dtype == EAGLE3_F32) {
        if (a->D < 1 || a->D > 128) return EAGLE3_ERR_UNSUPPORTED;
    } else {
        return EAGLE3_ERR_UNSUPPORTED;
    }
    // one work-group per (sequence, KV head, row block) walks the whole prefix:
    // splitting a prefix over work-groups is switched off (split_keys must be
    // 0), because the split path gave sporadic wrong rows whose cause was not
    // found; block ids of one work-group must fit its LDS table
    if (a->split_keys < 0 || a->split_keys % KT != 0) return EAGLE3_ERR_UNSUPPORTED;
    if (a->mask == nullptr) {
        if (a->parent == nullptr || a->Tq != a->Tk) return EAGLE3_ERR_ARG;
    }
    return EAGLE3_OK;
}

Plan make_plan(const eagle3_tree_attn_args *a) {
    Plan pl{};
    const int G = a->Hq / a->Hkv;
    const int R = a->Tq * G;
    pl.nrb = (R + ROWS_PER_WG - 1) / ROWS_PER_WG;
    // keys a prefix can have: the block table's capacity (the lengths
    // themselves are device data)
    const long lmax = (long)a->max_blocks * a->block_size;
    long C = a->split_keys;
    if (C == 0) {
        // automatic: split when there are fewer (sequence, KV head, row
        // block) work-groups than CUs, into enough splits to cover the CUs,
        // none shorter than MIN_SPLIT_KEYS
        const long base = (long)a->B * a->Hkv * pl.nrb;
        long S = 1;
        const long slots = (long)ATT_WG_PER_CU * e3_cu_count();
        if (a->dtype == EAGLE3_BF16 && base > 0 && base < slots)
            S = std::min((slots + base - 1) / base, std::max(1L, lmax / MIN_SPLIT_KEYS));
        C = (lmax + S - 1) / S;
    }
    C = std::max<long>(KT, (C + KT - 1) / KT * KT);
    pl.split_keys = (int)std::min<long>(C, 1L << 30);
    pl.nsplit = lmax > 0 ? (int)((lmax + pl.split_keys - 1) / pl.split_keys) : 1;
    pl.ws_bytes = 0;
    if (a->dtype == EAGLE3_BF16 && pl.nsplit > 1) {
        const size_t rows = (size_t)a->B * a->Hkv * pl.nsplit * (size_t)pl.nrb * ROWS_PER_WG;
        pl.ws_bytes = ((rows * DH * 4 + 255) & ~(size_t)255) + rows * 8;
    }
    return pl;
}

}  // namespace

extern "C" size_t eagle3_tree_attn_workspace(const eagle3_tree_attn_args *a) {
    if (check_args(a) != EAGLE3_OK) return 0;
    return make_plan(a).ws_bytes;
}

extern "C" int eagle3_tree_attn(const eagle3_tree_attn_args *a, void *ws, size_t ws_bytes, void *stream) {
    const int rc = check_args(a);
    if (rc != EAGLE3_OK) return rc;
    if (a->B == 0) return EAGLE3_OK;
    if (!a->q || !a->out || !a->block_table || !a->prefix_len) return EAGLE3_ERR_ARG;
    if (a->Tk > 0 && (!a->k_tree || !a->v_tree)) return EAGLE3_ERR_ARG;
    if (a->num_blocks > 0 && (!a->k_cache || !a->v_cache)) return EAGLE3_ERR_ARG;
    for (const void *ptr : {a->q, a->k_tree, a->v_tree, a->k_cache, a->v_cache, (const void *)a->out,
                            (const void *)a->norm_out})
        if (ptr && !e3_aligned16(ptr)) return EAGLE3_ERR_ARG;
    const Plan pl = make_plan(a);
    if (ws_bytes < pl.ws_bytes || (pl.ws_bytes > 0 && !ws)) return EAGLE3_ERR_WORKSPACE;
    if (pl.ws_bytes > 0 && !e3_aligned16(ws)) return EAGLE3_ERR_ARG;
    const hipStream_t st = e3_stream(stream);
    const int G = a->Hq / a->Hkv;
    if (a->status)
        tree_attn_validate_kernel<<<a->B, 64, 0, st>>>(a->block_table, a->prefix_len, a->mask ? nullptr : a->parent,
                                                        a->Tq, a->max_blocks, a->block_size, a->num_blocks,
                                                        a->status);
    if (a->dtype == EAGLE3_BF16) {
        AttnParams p;
        p.q = (const uint16_t *)a->q; p.k_tree = (const uint16_t *)a->k_tree; p.v_tree = (const uint16_t *)a->v_tree;
        p.k_cache = (const uint16_t *)a->k_cache; p.v_cache = (const uint16_t *)a->v_cache;
        p.block_table = a->block_table; p.prefix_len = a->prefix_len; p.mask = a->mask; p.parent = a->parent;
        p.out = (uint16_t *)a->out; p.lse = a->lse;
        p.B = a->B; p.Tq = a->Tq; p.Tk = a->Tk; p.Hq = a->Hq; p.Hkv = a->Hkv; p.W = a->W; p.G = G;
        p.R = a->Tq * G; p.nrb = pl.nrb; p.Rpad = pl.nrb * ROWS_PER_WG; p.nsplit = pl.nsplit;
        p.split_keys = pl.split_keys; p.max_blocks = a->max_blocks; p.num_blocks = a->num_blocks;
        p.nunits = a->B * a->Hkv * pl.nsplit;
        p.zero = 0.f;
        p.scale_log2 = a->scale * kLog2e;
        p.ws_o = nullptr; p.ws_ml = nullptr;
        if (pl.ws_bytes > 0) {
            const size_t rows = (size_t)a->B * a->Hkv * pl.nsplit * (size_t)pl.nrb * ROWS_PER_WG;
            p.ws_o = (float *)ws;
            p.ws_ml = (float *)((char *)ws + ((rows * DH * 4 + 255) & ~(size_t)255));
        }
        // the row blocks of a unit go to one XCD (ids 8 apart): the grid is a
        // whole number of 8-unit groups, surplus work-groups exit at once
        const int grid = (p.nunits + 7) / 8 * 8 * pl.nrb;
        // 8 waves of 32 rows: two waves per SIMD, 256 registers each. (Two
        // row blocks per wave would share every fragment read, but 64 rows of
        // Q, scores and output accumulators do not fit without spilling; two
        // independent 128-row work-groups per CU measured slower, as each K/V
        // tile is then read twice.)
        tree_attn_bf16_kernel<ATT_NW, 1><<<grid, ATT_NW * 64, 0, st>>>(p);
        const bool fused_norm = a->norm_out && pl.nsplit > 1 && pl.nsplit <= CN_MAXS && a->Hq <= CN_MAXH;
        if (fused_norm)
            tree_attn_combine_norm_kernel<<<a->B * a->Tq, CN_NT, 0, st>>>(p, (uint16_t *)a->norm_out, a->norm_eps);
        else if (pl.nsplit > 1)
            tree_attn_combine_kernel<<<a->B * a->Tq * a->Hq, DH, 0, st>>>(p);
        if (a->norm_out && !fused_norm) {
            const int rc2 = eagle3_rmsnorm(a->out, nullptr, a->B * a->Tq, a->Hq * DH, a->norm_eps, EAGLE3_BF16,
                                           a->norm_out, stream);
            if (rc2 != EAGLE3_OK) return rc2;
        }
    } else {
        AttnF32 p;
        p.q = (const float *)a->q; p.k_tree = (const float *)a->k_tree; p.v_tree = (const float *)a->v_tree;
        p.k_cache = (const float *)a->k_cache; p.v_cache = (const float *)a->v_cache;
        p.block_table = a->block_table; p.prefix_len = a->prefix_len; p.mask = a->mask; p.parent = a->parent;
        p.out = (float *)a->out; p.lse = a->lse;
        p.Tq = a->Tq; p.Tk = a->Tk; p.Hq = a->Hq; p.Hkv = a->Hkv; p.D = a->D; p.W = a->W; p.G = G;
        p.max_blocks = a->max_blocks; p.block_size = a->block_size; p.num_blocks = a->num_blocks;
        p.scale = a->scale;
        tree_attn_f32_kernel<<<a->B * a->Tq * a->Hq, 64, 0, st>>>(p);
        if (a->norm_out) {
            const int rc2 = eagle3_rmsnorm(a->out, nullptr, a->B * a->Tq, a->Hq * a->D, a->norm_eps, EAGLE3_F32,
                                           a->norm_out, stream);
            if (rc2 != EAGLE3_OK) return rc2;
        }
    }
    E3_LAUNCH_CHECK();
    return EAGLE3_OK;
}
