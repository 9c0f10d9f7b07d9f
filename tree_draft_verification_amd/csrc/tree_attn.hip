// Tree attention: every draft-tree node attends to its sequence's paged KV
// prefix plus its own ancestors (course lesson "EAGLE-3 speculative decoding:
// the tree-verifier method", section "Tree draft vs chain draft": one target
// pass over the whole tree, masked so a token sees only its ancestors).
// GQA reading: query head h uses KV head h / (Hq / Hkv).
//
// bf16, D = 128 (MFMA path). One work-group per (prefix split, KV head,
// sequence, block of 256 query rows); a query row is (node, head-in-group),
// so the G query heads sharing a KV head share every K/V tile read.
//   - K/V tiles of 64 keys are copied from the paged cache into LDS with
//     16-byte loads; each 16-token cache block is one contiguous 4 KB run for
//     K ([block, head, slot, d]) and for V ([block, head, d, slot]). The V
//     layout keeps keys contiguous per dimension, which is what the PV
//     product needs as its contraction operand.
//   - Each wave owns 32 query rows. S^T = K . Q^T by MFMA 32x32x16, so every
//     lane holds one query's scores: the softmax max and sum are in-lane plus
//     one exchange between the two half-waves. Online softmax in fp32 with
//     log2(e) folded into the scale, raw v_exp_f32, and a lazily refreshed
//     running max (O is rescaled only when the max grows by more than 2^8).
//     K rows sit in LDS in a permuted key order so that each lane's 8 scores
//     per 16-key step are consecutive keys and the V operand is one read. O^T += V^T . P^T by MFMA with P split
//     into bf16 hi + lo parts, so P keeps ~16 significant bits.
//   - Prefix keys are split across work-groups when there are too few
//     (sequence, head) pairs to fill the chip; the split holding the end of
//     the prefix also processes the tree keys under the ancestor mask.
//     Split partials (normalised O, max, sum) are merged in split order by a
//     second kernel, so results are deterministic.
// fp32 (any D <= 128): one 64-lane wave per query row, lanes over keys for
// the scores and over dimensions for P.V; for small models.
#include "common.h"

#include <type_traits>

namespace {

constexpr int KT = 64;       // keys per tile
constexpr int DH = 128;      // head dim of the MFMA path
constexpr int ROWS_PER_WG = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct AttnParams {
    const uint16_t *q, *k_tree, *v_tree, *k_cache, *v_cache;
    const int32_t *block_table, *prefix_len;
    const uint64_t *mask;
    const int32_t *parent;
    uint16_t *out;
    float *lse;
    float *ws_o;   // [B, Hkv, nsplit, Rpad, D]
    float *ws_ml;  // [B, Hkv, nsplit, Rpad, 2]
    int B, Tq, Tk, Hq, Hkv, W, G, R, Rpad, nrb, nsplit, split_keys, max_blocks, num_blocks;
    int tree_split;  // 1: the tree keys are a split of their own (after the prefix splits)
    float scale_log2;
};

// prefix length as the kernels use it: clamped to the block table's capacity
// (and 0 with an empty pool), so bad data can never index out of bounds
__device__ __forceinline__ int clamped_len(const int32_t *prefix_len, int b, int max_blocks, int bs, int num_blocks) {
    const int L = prefix_len[b];
    if (num_blocks <= 0) return 0;
    return max(0, min(L, max_blocks * bs));
}

// Splits of one sequence: prefix splits of split_keys keys, plus (tree_split)
// one more for the tree keys; without tree_split the last prefix split also
// takes the tree keys (an empty prefix still makes one split).
__device__ __forceinline__ int splits_of(int L, int split_keys, int tree_split) {
    const int npre = L > 0 ? (L + split_keys - 1) / split_keys : 0;
    return tree_split ? npre + 1 : (npre > 0 ? npre : 1);
}

// Sequences are dealt to work-group slots longest (clamped) prefix first,
// ties by lower index: the long sequences start in the first pass over the
// CUs and the short ones fill in behind them (longest-processing-time-first
// list order), instead of the batch order, which can leave a CU with two
// long sequences. Every wave ranks the sequences by counting; slot r takes
// the sequence of rank r. Past LPT_MAX_B sequences the batch order is kept.
constexpr int LPT_MAX_B = 256;
__device__ __forceinline__ int seq_of_slot(const int32_t *prefix_len, int B, int r, int max_blocks, int num_blocks) {
    if (B > LPT_MAX_B) return r;
    const int lane = threadIdx.x & 63;
    for (int j0 = 0; j0 < B; j0 += 64) {
        const int j = j0 + lane;
        int rank = -1;
        if (j < B) {
            const int Lj = clamped_len(prefix_len, j, max_blocks, 16, num_blocks);
            rank = 0;
            for (int k = 0; k < B; ++k) {
                const int Lk = clamped_len(prefix_len, k, max_blocks, 16, num_blocks);
                rank += (Lk > Lj || (Lk == Lj && k < j)) ? 1 : 0;
            }
        }
        const uint64_t hit = __ballot(rank == r);
        if (hit) return j0 + __ffsll((unsigned long long)hit) - 1;
    }
    return r;  // not reached: the ranks are a permutation of 0..B-1
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

typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int NSTAGE = 3;                  // depth of the K/V ring
constexpr int STAGE = 2 * KT * DH * 2;     // bytes per stage: K tile + V tile (16 KB each)
constexpr int VOFF = KT * DH * 2;          // V tile offset inside a stage
constexpr int MAX_SPLIT_BLOCKS = 1024;     // cache blocks one work-group may cover (prefixes up to 16384 keys)

// 16-byte column swizzle of K rows (a tile row is one key, 256 B): K reads of
// 16 consecutive rows then hit 16 distinct bank groups.
__device__ __forceinline__ int kswz(int row) { return row & 15; }
// V rows are (block, d) pairs of 32 B = 16 slots; the two 16-byte halves are
// swapped on every other group of 8 rows, halving bank conflicts of PV reads.
__device__ __forceinline__ int vswz(int d) { return (d >> 3) & 1; }
// Key held by K-tile row r: bits 2 and 3 of the key swapped. The S^T
// accumulator gives lane half h the rows 8a + 4h + c (a in {0,1}, c in 0..3)
// of each 16-row group, i.e. keys 8h + 4a + c: eight consecutive keys, which
// is one 16-byte half of a V row, so the PV operand is a single LDS read.
__device__ __forceinline__ int row_key(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

enum TileKind { TILE_FULL = 0, TILE_PARTIAL = 1, TILE_TREE = 2 };

// Softmax bookkeeping is in log2 units with a lazily refreshed running max:
// m_run only moves when a score exceeds it by more than 2^8 (so exp2 values
// stay below 256, harmless in fp32), which makes O rescaling rare.
constexpr float kLazyMax = 8.f;

// LDS fragment reads are inline ds_read_b128: the compiler cannot tell ring
// stages apart and would otherwise wait for every K/V DMA still in flight
// (the whole ring) before the first read of a tile. Each read is awaited
// explicitly (lgkmcnt), with the wait tied to its destination register.
__device__ __forceinline__ void lds_read16(u32x4_t &r, uint32_t addr) {
    __asm__ volatile("ds_read_b128 %0, %1" : "=v"(r) : "v"(addr));
}
template <int N>
__device__ __forceinline__ void lgkm_wait1(u32x4_t &r) {
    __asm__ volatile("s_waitcnt lgkmcnt(%1)" : "+v"(r) : "i"(N));
}
// wait until at most n (0..2) LDS reads are outstanding
__device__ __forceinline__ void lgkm_upto(int n, u32x4_t &r) {
    if (n >= 2) lgkm_wait1<2>(r);
    else if (n == 1) lgkm_wait1<1>(r);
    else lgkm_wait1<0>(r);
}

// compile-time unrolled loop: f(std::integral_constant<int, i>) for i in [I, N)
template <int I, int N, typename F>
__device__ __forceinline__ void sfor(F &&f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        sfor<I + 1, N>(f);
    }
}

// LDS fragment read at a per-lane address plus a constant byte offset (the
// instruction's offset field), so the constant parts take no registers
template <int OFF>
__device__ __forceinline__ void lds_read16_at(u32x4_t &r, uint32_t addr) {
    static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
    __asm__ volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
}

// Per-lane parts of the fragment addresses inside a ring stage. QK step j
// (key block kb = j & 1, d-step s = j >> 1) reads koff[s] + 8192 kb: row
// 32 kb + lr, 16-byte column (2 s + lh) ^ kswz(lr) (kswz of the row only sees
// lr); lane half lh holds d = 16 s + 8 lh .. +7. PV step j (16-key step
// ks = j >> 2, d block db = j & 3) reads voff + 4096 ks + 1024 db: row
// (ks, d = 32 db + lr), half lh ^ vswz(lr).
struct FragOffsets {
    uint32_t k[8];
    uint32_t v;
};
__device__ __forceinline__ FragOffsets frag_offsets(int lr, int lh) {
    FragOffsets f;
#pragma unroll
    for (int s = 0; s < 8; ++s) f.k[s] = lr * 256 + (((2 * s + lh) ^ kswz(lr)) << 4);
    f.v = VOFF + lr * 32 + ((lh ^ vswz(lr)) << 4);
    return f;
}

// Fragment reads run RA steps ahead through an NF-slot buffer: with one
// 32 x 32 x 16 MFMA (QK) or two (PV) per read, two reads ahead left the
// LDS latency exposed at every step.
constexpr int RA = 4, NF = RA + 2;

// One 64-key tile for one wave and its RB blocks of 32 query rows: S^T =
// K.Q^T, online softmax, O^T += V^T.P^T. Every K / V fragment read from LDS
// feeds the MFMAs of all RB row blocks, and the row blocks' independent
// softmax work interleaves with the MFMAs of the others. kind is wave-uniform.
// Operand fragments are read two steps ahead through a 4-slot buffer.
template <int RB>
__device__ __forceinline__ void attend_tile(int kind, const unsigned char *stage, const u32x4_t (&qb)[RB][8],
                                            f32x16_t (&ot)[RB][4], float (&m_run)[RB], float (&l_run)[RB],
                                            const FragOffsets &fo, int lh, int nvalid, const uint64_t (&mword)[RB],
                                            float scale_log2) {
    const uint32_t sb = (uint32_t)(uintptr_t)(lds_void_t *)stage;
    u32x4_t fr[NF];
    // QK step j: key block kb = j & 1 (alternating accumulators), d-step s = j >> 1
    auto kread = [&](auto J) {
        constexpr int j = J;
        lds_read16_at<(j & 1) * 8192>(fr[j % NF], sb + fo.k[j >> 1]);
    };
    f32x16_t st[RB][2];
    // the score accumulators start as registers holding zero, not the MFMA's
    // inline-zero operand: with the inline zero the destination is not tied
    // to an input and the compiler placed it over the A operand's registers
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) st[rb][kb][r] = 0.f;
            __asm__ volatile("" : "+v"(st[rb][kb]));
        }
    sfor<0, RA>(kread);
    sfor<0, 16>([&](auto J) {
        constexpr int j = J, kb = j & 1, s = j >> 1;
        if constexpr (j + RA < 16) kread(std::integral_constant<int, j + RA>{});
        lgkm_wait1<(15 - j < RA ? 15 - j : RA)>(fr[j % NF]);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
            st[rb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, fr[j % NF]),
                                                                 __builtin_bit_cast(bf16x8_t, qb[rb][s]), st[rb][kb],
                                                                 0, 0, 0);
    });
    // PV step j: 16-key step ks = j >> 2, d block db = j & 3; the first RA V
    // fragments are read now and land during the softmax
    auto vread = [&](auto J) {
        constexpr int j = J;
        lds_read16_at<(j >> 2) * 4096 + (j & 3) * 1024>(fr[j % NF], sb + fo.v);
    };
    sfor<0, RA>(vread);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        // register r of block kb holds key 32 kb + 16 (r / 8) + 8 lh + (r % 8)
        if (kind != TILE_FULL) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int kk = kb * 32 + 16 * (r >> 3) + 8 * lh + (r & 7);
                    const bool vis = kk < nvalid && (kind != TILE_TREE || ((mword[rb] >> kk) & 1u));
                    st[rb][kb][r] = vis ? st[rb][kb][r] : -INFINITY;
                }
        }
        float tmax = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, st[rb][kb][r]);
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32)) * scale_log2;
        // refresh the running max only when it is exceeded by more than 2^kLazyMax
        const bool grow = tmax > m_run[rb] + kLazyMax;
        if (__ballot(grow)) {
            const float m_new = grow ? tmax : m_run[rb];
            const float alpha = (m_run[rb] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run[rb] - m_new);
            l_run[rb] *= alpha;
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) ot[rb][db][r] *= alpha;
            m_run[rb] = m_new;
        }
        const float msub = (m_run[rb] == -INFINITY) ? 0.f : m_run[rb];
        float psum = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float pv = __builtin_amdgcn_exp2f(fmaf(st[rb][kb][r], scale_log2, -msub));
                st[rb][kb][r] = pv;
                psum += pv;
            }
        l_run[rb] += psum;
    }
    // 16 keys per step = one cache block of the tile; this lane's 8 P values
    // are keys 8 lh .. 8 lh + 7 of the block. P enters as bf16 hi + lo (two
    // MFMAs on the same V operand): a single bf16 rounding of P would leave
    // ~2e-3 relative error in the output.
    u32x4_t ph[RB], pl[RB];
    sfor<0, 16>([&](auto J) {
        constexpr int j = J, ks = j >> 2, db = j & 3;
        if constexpr (db == 0) {
            constexpr int kb = ks >> 1, r0 = 8 * (ks & 1);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    uint32_t h2, l2;
                    e3_split_bf16x2(st[rb][kb][r0 + 2 * e], st[rb][kb][r0 + 2 * e + 1], h2, l2);
                    ph[rb][e] = h2;
                    pl[rb][e] = l2;
                }
        }
        if constexpr (j + RA < 16) vread(std::integral_constant<int, j + RA>{});
        lgkm_wait1<(15 - j < RA ? 15 - j : RA)>(fr[j % NF]);
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, fr[j % NF]);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            ot[rb][db] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8_t, ph[rb]), ot[rb][db], 0, 0, 0);
            ot[rb][db] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8_t, pl[rb]), ot[rb][db], 0, 0, 0);
        }
    });
}

// NW waves of RB x 32 query rows each (NW * RB * 32 = ROWS_PER_WG).
template <int NW, int RB>
__global__ __launch_bounds__(NW * 64) void tree_attn_bf16_kernel(AttnParams p) {
    static_assert(NW * RB * 32 == ROWS_PER_WG, "a work-group covers one block of query rows");
    __shared__ __attribute__((aligned(1024))) unsigned char ring[NSTAGE * STAGE];
    __shared__ int bids[MAX_SPLIT_BLOCKS];
    constexpr int NT = NW * 64;
    constexpr int LOADS = 32 / NW;  // 1 KB DMA loads per wave per stage (16 for K, 16 for V)

    const int split = blockIdx.x / p.nrb, rb = blockIdx.x % p.nrb;
    const int kvh = blockIdx.y;
    const int b = __builtin_amdgcn_readfirstlane(seq_of_slot(p.prefix_len, p.B, blockIdx.z, p.max_blocks, p.num_blocks));
    const int L = clamped_len(p.prefix_len, b, p.max_blocks, 16, p.num_blocks);
    const int C = p.split_keys;
    const int nsplit_b = splits_of(L, C, p.tree_split);
    if (split >= nsplit_b) return;
    const bool last = split == nsplit_b - 1;           // this split takes the tree keys
    const bool tree_only = p.tree_split && last;       // ... and no prefix keys
    const int k_begin = tree_only ? 0 : split * C;
    const int k_end = tree_only ? 0 : min(L, k_begin + C);

    // the wave index is wave-uniform; saying so keeps the branches on it scalar
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int lr = lane & 31, lh = lane >> 5;
    // this lane's query rows, one per row block
    int row[RB], t[RB], hq[RB];
    bool row_ok[RB];
#pragma unroll
    for (int k = 0; k < RB; ++k) {
        row[k] = rb * ROWS_PER_WG + (wave * RB + k) * 32 + lr;
        row_ok[k] = row[k] < p.R;
        t[k] = row_ok[k] ? row[k] / p.G : 0;
        hq[k] = kvh * p.G + (row_ok[k] ? row[k] % p.G : 0);
    }
    const bool wave_active = rb * ROWS_PER_WG + wave * RB * 32 < p.R;

    // physical ids of the cache blocks this split reads
    const int blk0 = k_begin / 16;
    const int nblk = (k_end - k_begin + 15) / 16;
    const int32_t *btab = p.block_table + (size_t)b * p.max_blocks;
    for (int i = tid; i < nblk; i += NT) bids[i] = clamped_block(btab, blk0 + i, p.num_blocks);

    // this lane's part of each DMA load: element offset inside a cache block
    // ([16 slots][128 d] for K, [128 d][16 slots] for V)
    int dma_off[LOADS];
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
        const int q = wave * LOADS + j;
        if (q < 16) {
            const int rib = 4 * (q & 3) + lane / 16;    // tile row in block (rows are 16-aligned per block)
            dma_off[j] = row_key(rib) * DH + 8 * ((lane & 15) ^ kswz(rib));
        } else {
            const int d = 32 * ((q - 16) & 3) + lane / 2;
            dma_off[j] = d * 16 + 8 * ((lane & 1) ^ vswz(d));
        }
    }
    const size_t head_off = (size_t)kvh * 16 * DH;
    const size_t blk_stride = (size_t)p.Hkv * 16 * DH;
    // a wave's LOADS = 4 loads of a stage all come from one cache block (K
    // for waves 0-3, V for waves 4-7): its address is a scalar base plus a
    // 32-bit per-lane offset
    static_assert(LOADS == 4, "one cache block per wave and stage");
    auto issue = [&](int stage, int tile) {
        unsigned char *base = ring + stage * STAGE;
        const int lb = min(4 * tile + (wave & 3), nblk - 1);  // blocks past the prefix re-read the last
        const int bid = __builtin_amdgcn_readfirstlane(bids[lb]);
        const uint16_t *blk = (wave < 4 ? p.k_cache : p.v_cache) + (size_t)bid * blk_stride + head_off;
#pragma unroll
        for (int j = 0; j < LOADS; ++j) {
            const int q = wave * LOADS + j;
            __builtin_amdgcn_global_load_lds((const void *)(blk + dma_off[j]), (lds_void_t *)(base + q * 1024), 16,
                                             0, 0);
        }
    };

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

    const FragOffsets fo = frag_offsets(lr, lh);
    const int ntile = (k_end - k_begin + KT - 1) / KT;
    // q and mask words have landed before any K/V DMA is queued behind them
    // (otherwise the first use of q inside the tile loop waits for the ring)
    wait_vmcnt<0>();
    __syncthreads();  // block ids are in
#pragma unroll
    for (int st = 0; st < NSTAGE - 1; ++st)
        if (st < ntile) issue(st, st);

    // prefix tiles stream through the ring; the tree keys (only in the split
    // holding the end of the prefix) follow through registers, since their V
    // rows must be transposed into the [block][d][slot] layout
    const int ntree = last ? (p.Tk + KT - 1) / KT : 0;
    for (int it = 0; it < ntile + ntree; ++it) {
        const unsigned char *stage;
        int kind, nvalid;
        uint64_t mword[RB];
#pragma unroll
        for (int k = 0; k < RB; ++k) mword[k] = 0;
        if (it < ntile) {
            // all of this wave's ring loads, not just those of tile it: the
            // wait then holds whatever order the DMA completions take (tile
            // it + 1 was issued a tile earlier and has landed by now; measured
            // at no cost against waiting for tile it alone)
            wait_vmcnt<0>();
            // tile it has landed for every wave and every wave is done with the
            // buffer refilled below; a fenced barrier would also wait for the
            // compiler's own outstanding operations
            __builtin_amdgcn_s_barrier();
            __asm__ volatile("" ::: "memory");
            stage = ring + (it % NSTAGE) * STAGE;
            nvalid = k_end - (k_begin + it * KT);
            kind = nvalid >= KT ? TILE_FULL : TILE_PARTIAL;
            if (nvalid < KT) {
                // last, partial tile: zero the V slots past the prefix (the
                // cache may hold anything there, and 0 * NaN would poison the sum)
                unsigned char *vb = ring + (it % NSTAGE) * STAGE + VOFF;
                for (int r = tid; r < 4 * DH; r += NT) {
                    const int jb = r / DH, d = r % DH;
                    uint16_t *rowp = reinterpret_cast<uint16_t *>(vb + jb * 4096 + d * 32);
                    for (int sl = 0; sl < 16; ++sl)
                        if (16 * jb + sl >= nvalid) rowp[((sl >> 3) ^ vswz(d)) * 8 + (sl & 7)] = 0;
                }
                __syncthreads();
            }
            if (it + NSTAGE - 1 < ntile) issue((it + NSTAGE - 1) % NSTAGE, it + NSTAGE - 1);
        } else {
            const int tt = it - ntile;
            __syncthreads();  // everyone is done with stage 0 (and the ring is drained)
            unsigned char *Kb = ring, *Vb = ring + VOFF;
            for (int c = tid; c < KT * DH / 8; c += NT) {
                const int key = c >> 4, d8 = (c & 15) * 8;
                const int tk = tt * KT + key;
                u32x4_t kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
                if (tk < p.Tk) {
                    const size_t off = (((size_t)b * p.Tk + tk) * p.Hkv + kvh) * DH + d8;
                    kv = *reinterpret_cast<const u32x4_t *>(p.k_tree + off);
                    vv = *reinterpret_cast<const u32x4_t *>(p.v_tree + off);
                }
                const int krow = row_key(key);  // the row holding this key (the permutation is an involution)
                *reinterpret_cast<u32x4_t *>(Kb + krow * 256 + (((c & 15) ^ kswz(krow)) << 4)) = kv;
                const int jb = key >> 4, sl = key & 15;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int d = d8 + e;
                    const uint16_t val = (uint16_t)((e & 1) ? (vv[e >> 1] >> 16) : (vv[e >> 1] & 0xffffu));
                    reinterpret_cast<uint16_t *>(Vb + jb * 4096 + d * 32)[((sl >> 3) ^ vswz(d)) * 8 + (sl & 7)] = val;
                }
            }
            __syncthreads();
            stage = ring;
            kind = TILE_TREE;
            nvalid = p.Tk - tt * KT;
#pragma unroll
            for (int k = 0; k < RB; ++k) mword[k] = tt == 0 ? mw0[k] : mw1[k];
        }
        if (wave_active) attend_tile<RB>(kind, stage, qb, ot, m_run, l_run, fo, lh, nvalid, mword, p.scale_log2);
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
    const int nsplit_b = splits_of(L, p.split_keys, p.tree_split);
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
    const int nsplit_b = splits_of(L, p.split_keys, p.tree_split);
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
    int nrb, nsplit, split_keys, tree_split;
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
    if (a->split_keys != 0) return EAGLE3_ERR_UNSUPPORTED;
    if (a->dtype == EAGLE3_BF16 && (long)a->max_blocks * a->block_size > 16L * MAX_SPLIT_BLOCKS)
        return EAGLE3_ERR_UNSUPPORTED;
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
    // a single split covering the largest prefix the block table can address
    const long lmax = (long)a->max_blocks * a->block_size;
    const long keys = lmax > 0 ? (lmax + KT - 1) / KT * KT : KT;
    pl.split_keys = (int)keys;
    pl.nsplit = 1;
    pl.tree_split = 0;
    pl.ws_bytes = 0;
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
        p.tree_split = pl.tree_split;
        p.scale_log2 = a->scale * kLog2e;
        p.ws_o = nullptr; p.ws_ml = nullptr;
        if (pl.ws_bytes > 0) {
            const size_t rows = (size_t)a->B * a->Hkv * pl.nsplit * (size_t)pl.nrb * ROWS_PER_WG;
            p.ws_o = (float *)ws;
            p.ws_ml = (float *)((char *)ws + ((rows * DH * 4 + 255) & ~(size_t)255));
        }
        dim3 grid(pl.nsplit * pl.nrb, a->Hkv, a->B);
        // 8 waves of 32 rows cover the 256-row block (two row blocks per wave
        // would share every fragment read, but 64 rows of Q, scores and output
        // accumulators do not fit the register file)
        tree_attn_bf16_kernel<8, 1><<<grid, 512, 0, st>>>(p);
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
