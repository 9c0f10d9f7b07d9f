// LM head with a fused per-row top-k / gap / log-sum-exp; logits never reach
// memory. The target's argmax at every tree node decides acceptance (course
// lesson "EAGLE-3 speculative decoding: the tree-verifier method", section
// "Verify-accept semantics"); the draft head's top-k uses the same head (news
// write-up of the EAGLE-3 paper, draft-stage paragraphs), and every forward
// streams the whole head from memory (the same write-up's opening remark that
// each forward reads all parameters), so for few rows this is an HBM stream.
//
// Pass 1, bf16 (one work-group per 128-row vocabulary tile x 64-row hidden
// tile, 4 waves, 2 work-groups per CU; for argmax-only calls with one hidden
// tile, 8 waves over a 256-row vocabulary tile, 1 work-group per CU):
//   - 64-wide k chunks of the weight tile (128 rows x 128 B) and of the hidden
//     tile (64 rows x 128 B) go straight from global memory into a 3-stage LDS
//     ring with 16-byte global_load_lds (no VGPR round trip); each 1 KB load
//     instruction covers 8 full 128 B row segments. A wave waits only for the
//     oldest stage (explicit vmcnt) and the stage hand-off uses a bare barrier
//     (a fenced barrier would drain the stages still in flight).
//   - 16-byte columns are XOR-swizzled by row pair, so the MFMA operand reads
//     (ds_read_b128, 32 rows per instruction) are bank-conflict free.
//   - Each tile starts its k sweep at a different chunk (tile * 7 mod K/64):
//     tiles running together then read different column ranges of their rows
//     instead of all hitting the same 128 B column of rows 8 KB apart.
//   - MFMA 32x32x16: vocabulary rows are the "row" operand and hidden rows the
//     "column" operand, so each accumulator register of a lane belongs to one
//     hidden row.
// Pass 1, fp32: plain FMA loop over a 256-row vocabulary tile (small models).
//   - With one hidden tile the weight rows are loaded non-temporal: the
//     head is streamed once per call and should not evict the hidden rows.
// Epilogue (both): the logit tile is staged in LDS; a few threads per row keep
// a sorted top-KK list of 64-bit selection keys (value desc, id asc; one
// unsigned compare per step, branch-free inserts) and a (max, sum exp) pair,
// merged by lane shuffles; one record per (row, tile) goes to the workspace.
// Pass 2 (one work-group per row): merges all tiles' records in a fixed order,
// so results are deterministic.
#include <mutex>

#include "common.h"
#include "gemm_core.h"

namespace {

constexpr int BN_B = 128;  // vocabulary rows per tile of the 4-wave few-row kernel (32 per wave)
constexpr int BN_F = 256;  // vocabulary rows per tile, fp32 path
constexpr int BK = 64;     // k per chunk, bf16 path
constexpr int NSTAGE = 3;  // LDS ring depth, bf16 path
constexpr int ROT = 7;     // chunk rotation per tile

struct Partials {
    uint64_t *key;  // [M, ntiles, KK] selection keys, descending
    float *mx;      // [M, ntiles]
    float *se;      // [M, ntiles]
    uint32_t *ctr;  // tile counters of the persistent top-2 pass, one per XCD, CTR_STRIDE apart
};
using e3g::CTR_BYTES;

// one record: a row's sorted list over one tile (KK even: 16-byte stores)
template <int KK>
__device__ __forceinline__ void store_record(const Partials &p, size_t rec, const uint64_t (&L)[KK]) {
    static_assert(KK % 2 == 0, "records are written 16 bytes at a time");
    u32x4_t *dst = reinterpret_cast<u32x4_t *>(p.key + rec * KK);
#pragma unroll
    for (int s = 0; s < KK; s += 2) {
        u32x4_t q;
        q[0] = (uint32_t)L[s]; q[1] = (uint32_t)(L[s] >> 32);
        q[2] = (uint32_t)L[s + 1]; q[3] = (uint32_t)(L[s + 1] >> 32);
        dst[s / 2] = q;
    }
}

// Per-row selection over an LDS tile lg[BMt][BNt + 4]; NT / BMt threads per row.
template <int BMt, int BNt, int KK, bool LSE, int NT = 256>
__device__ __forceinline__ void tile_select(const float (*lg)[BNt + 4], int m0, int M, int n0, int N, int tile,
                                            int ntiles, const Partials &p) {
    constexpr int TPR = NT / BMt;
    constexpr int PER = BNt / TPR;
    const int row = threadIdx.x / TPR, part = threadIdx.x % TPR;
    static_assert(PER % 4 == 0, "16-byte reads of a thread's run");
    uint64_t L[KK];
    e3_kinit<KK>(L);
    const int vbeg = part * PER;
    // the thread's whole run in a few wide reads first: one LDS round trip
    // per element would serialise the scan on LDS latency
    float xs[PER];
#pragma unroll
    for (int i = 0; i < PER; i += 4) {
        const f32x4_t q = *reinterpret_cast<const f32x4_t *>(&lg[row][vbeg + i]);
        xs[i] = q[0]; xs[i + 1] = q[1]; xs[i + 2] = q[2]; xs[i + 3] = q[3];
    }
    const int nv = N - (n0 + vbeg);   // valid entries of the run (may exceed PER)
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        if (i >= nv) xs[i] = -INFINITY;
        const uint64_t k = i < nv ? e3_key(xs[i], n0 + vbeg + i) : 0;
        if (k > L[KK - 1]) e3_kinsert<KK>(L, k);
    }
    float mx = -INFINITY, se = 0.f;
    if (LSE) {
#pragma unroll
        for (int i = 0; i < PER; ++i) mx = fmaxf(mx, xs[i]);
        if (mx != -INFINITY) {
#pragma unroll
            for (int i = 0; i < PER; ++i) se += __expf(xs[i] - mx);
        }
    }
#pragma unroll
    for (int off = 1; off < TPR; off <<= 1) {
        e3_kmerge_xor<KK>(L, off);
        if (LSE) {
            const float m2 = __shfl_xor(mx, off), s2 = __shfl_xor(se, off);
            e3_lse_combine(mx, se, m2, s2);
        }
    }
    const int m = m0 + row;
    if (part == 0 && m < M) {
        const size_t rec = (size_t)m * ntiles + tile;
        store_record<KK>(p, rec, L);
        if (LSE) { p.mx[rec] = mx; p.se[rec] = se; }
    }
}

typedef __attribute__((address_space(3))) void lds_void_t;

// 16-byte column swizzle of an LDS row (row pairs share a permutation)
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

// wait until at most N vector-memory operations of this wave are outstanding
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

template <int KK, bool LSE, bool NTW, int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void lmhead_bf16_kernel(const uint16_t *__restrict__ h,
                                                             const uint16_t *__restrict__ w, int M, int N, int K,
                                                             int ntiles, Partials p) {
    constexpr int BM = 64, BN = 32 * NW, NS = NSTAGE;
    constexpr int WST = BN * 128, HST = BM * 128;   // bytes of one stage (128 B = 64 bf16 per row)
    constexpr int WBLK = WST / 1024;                 // 1 KB load blocks of the weight part
    constexpr int LOADS = (WST + HST) / 1024 / NW;  // 1 KB loads per wave per stage
    static_assert((WST + HST) % (1024 * NW) == 0, "stage must split evenly over the waves");
    __shared__ __attribute__((aligned(1024))) unsigned char smem[NS * (WST + HST)];
    static_assert(sizeof(float) * BM * (BN + 4) <= sizeof(smem), "logit tile must fit the ring");

    const int mt = blockIdx.x, tile = blockIdx.y;
    const int m0 = mt * BM, n0 = tile * BN;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int lr = lane & 31, lh = lane >> 5;

    // global source of each of this lane's loads (chunk offset added per stage):
    // block b of a stage holds rows 8b..8b+7; lane l fills row 8b + l/8, 16-byte
    // column l%8, which receives global column (l%8) ^ swz(row)
    const uint16_t *src[LOADS];
    int dst[LOADS];
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
        const int blk = wave * LOADS + j;
        if (blk < WBLK) {
            const int row = blk * 8 + lane / 8;
            const int v = min(n0 + row, N - 1);   // rows past N are computed and dropped
            src[j] = w + (size_t)v * K + 8 * ((lane & 7) ^ swz(row));
            dst[j] = blk * 1024;
        } else {
            const int row = (blk - WBLK) * 8 + lane / 8;
            const int m = min(m0 + row, M - 1);   // rows past M are computed and dropped
            src[j] = h + (size_t)m * K + 8 * ((lane & 7) ^ swz(row));
            dst[j] = WST + (blk - WBLK) * 1024;
        }
    }
    auto issue = [&](int stage, int kc) {
        unsigned char *base = smem + stage * (WST + HST);
#pragma unroll
        for (int j = 0; j < LOADS; ++j) {
            // with one hidden tile the weight is read once per call: then
            // non-temporal, so the stream does not evict the hidden rows
            // every tile re-reads
            if (NTW && wave * LOADS + j < WBLK)
                __builtin_amdgcn_global_load_lds((const void *)(src[j] + kc), (lds_void_t *)(base + dst[j]), 16, 0,
                                                 E3_CPOL_NT);
            else
                __builtin_amdgcn_global_load_lds((const void *)(src[j] + kc), (lds_void_t *)(base + dst[j]), 16, 0,
                                                 0);
        }
    };

    f32x16_t acc[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;

    const int nch = K / BK;
    const int rot = (tile * ROT) % nch;
#pragma unroll
    for (int st = 0; st < NS - 1; ++st)
        if (st < nch) issue(st, ((st + rot) % nch) * BK);

    const int vrow = wave * 32 + lr;  // this lane's weight row in the tile (MFMA row operand)
    for (int c = 0; c < nch; ++c) {
        if (c + NS - 2 < nch) wait_vmcnt<(NS - 2) * LOADS>();
        else wait_vmcnt<0>();
        // stage c has landed for every wave, and every wave is done with the
        // buffer about to be refilled; a fenced barrier would also drain the
        // stages still in flight, so the barrier is a bare one
        __builtin_amdgcn_s_barrier();
        __asm__ volatile("" ::: "memory");
        if (c + NS - 1 < nch) issue((c + NS - 1) % NS, ((c + NS - 1 + rot) % nch) * BK);
        const unsigned char *wb = smem + (c % NS) * (WST + HST);
        const unsigned char *hb = wb + WST;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            // both operands take k = 32 lh + 8 s .. +7 of the chunk
            const int col = 4 * lh + s;
            const u32x4_t a = *reinterpret_cast<const u32x4_t *>(wb + vrow * 128 + ((col ^ swz(vrow)) << 4));
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
                const int hrow = mb * 32 + lr;
                const u32x4_t b = *reinterpret_cast<const u32x4_t *>(hb + hrow * 128 + ((col ^ swz(hrow)) << 4));
                acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                                  __builtin_bit_cast(bf16x8_t, b), acc[mb], 0, 0, 0);
            }
        }
    }
    __syncthreads();  // the ring is reused for the logit tile
    float (*lg)[BN + 4] = reinterpret_cast<float (*)[BN + 4]>(smem);
    // D[vocab i][hidden j]: lane holds j = lr, i = 8 (r / 4) + 4 lh + r % 4
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            lg[mb * 32 + lr][wave * 32 + 8 * (r >> 2) + 4 * lh + (r & 3)] = acc[mb][r];
    __syncthreads();
    tile_select<BM, BN, KK, LSE, 64 * NW>(lg, m0, M, n0, N, tile, ntiles, p);
}

// Many hidden rows (verify batches of whole trees, draft steps): the head is
// a dense bf16 GEMM on the shared GEMM core, BM hidden rows x 256 vocabulary
// rows per work-group. BM = 256 (one work-group per CU, the most reuse) for
// short lists; BM = 128 (two per CU, so one's long selection epilogue
// overlaps the other's MFMAs) for lists of 8 and more. Each wave's logit
// block is then staged in LDS 64 (BM = 256) or 32 (BM = 128) hidden rows at a
// time for the per-row selection.
constexpr int BIG_BN = e3g::GBN;  // vocabulary rows per tile, many-row path
constexpr int big_bm(int KK) { return KK >= 8 ? 128 : 256; }

// Top-2 of one row over the 128 vocabulary columns a wave holds in the
// transposed accumulator layout (lane lr: the row; lane half lh: every other
// group of 4 columns), with the lowest column first among equal values; NaN
// and -inf never enter the list. The two lane halves then merge by (value
// desc, column asc).
constexpr int NO_COL = 0x7fffffff;
__device__ __forceinline__ bool e3_before(float a, int ia, float b, int ib) { return a > b || (a == b && ia < ib); }

// max(a, b) as one v_max_f32 (a NaN operand yields the other); written out so
// that no canonicalising copy of each operand is added
__device__ __forceinline__ float e3_vmax(float a, float b) {
    float r;
    __asm__("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// One lane's two largest values and their lowest columns; MASK: columns from
// nvalid on hold no vocabulary row and count as -inf.
template <int NB, bool MASK>
__device__ __forceinline__ void top2_lane(const f32x16_t (&blk)[NB], int lh, int nvalid, float &b0, int &i0, float &b1,
                                          int &i1) {
    // the two largest values with multiplicity: b0 = max, b1 = the median of
    // (b0, b1, v), two VALU operations per value; both pass over NaN
    b0 = -INFINITY; b1 = -INFINITY;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int col = 32 * nb + 8 * (r >> 2) + 4 * lh + (r & 3);
            const float v = MASK && col >= nvalid ? -INFINITY : blk[nb][r];
            const float t = __builtin_amdgcn_fmed3f(b0, b1, v);
            b0 = e3_vmax(b0, v);
            b1 = t;
        }
    // their columns: a scan in decreasing column order keeps the lowest column
    // holding each value; when b0 == b1 in some lane, the second column is the
    // second-lowest holding b0 (a branch uniform over the wave)
    i0 = NO_COL; i1 = NO_COL;
    if (__builtin_amdgcn_ballot_w64(b0 == b1 && b0 > -INFINITY) == 0) {
#pragma unroll
        for (int nb = NB - 1; nb >= 0; --nb)
#pragma unroll
            for (int r = 15; r >= 0; --r) {
                const int col = 32 * nb + 8 * (r >> 2) + 4 * lh + (r & 3);
                const float v = MASK && col >= nvalid ? -INFINITY : blk[nb][r];
                i0 = v == b0 ? col : i0;
                i1 = v == b1 ? col : i1;
            }
    } else {
#pragma unroll
        for (int nb = NB - 1; nb >= 0; --nb)
#pragma unroll
            for (int r = 15; r >= 0; --r) {
                const int col = 32 * nb + 8 * (r >> 2) + 4 * lh + (r & 3);
                const float v = MASK && col >= nvalid ? -INFINITY : blk[nb][r];
                const bool e0 = v == b0, e1 = v == b1;
                i1 = e1 ? (e0 ? i0 : col) : i1;
                i0 = e0 ? col : i0;
            }
    }
    // -inf (and masked columns) never enter the list
    if (!(b0 > -INFINITY)) i0 = NO_COL;
    if (!(b1 > -INFINITY)) i1 = NO_COL;
}

template <int NB>
__device__ __forceinline__ void top2_row(const f32x16_t (&blk)[NB], int lh, int nvalid, float &b0, int &i0, float &b1,
                                         int &i1) {
    if (nvalid >= NB * 32) top2_lane<NB, false>(blk, lh, nvalid, b0, i0, b1, i1);  // uniform
    else top2_lane<NB, true>(blk, lh, nvalid, b0, i0, b1, i1);
    const float ob0 = __shfl_xor(b0, 32), ob1 = __shfl_xor(b1, 32);
    const int oi0 = __shfl_xor(i0, 32), oi1 = __shfl_xor(i1, 32);
    if (e3_before(ob0, oi0, b0, i0)) {
        const bool keep = e3_before(b0, i0, ob1, oi1);
        b1 = keep ? b0 : ob1; i1 = keep ? i0 : oi1;
        b0 = ob0; i0 = oi0;
    } else {
        const bool take = e3_before(ob0, oi0, b1, i1);
        b1 = take ? ob0 : b1; i1 = take ? oi0 : i1;
    }
}

// One lane's top-KK keys (value desc, column asc) and, with LSE, (max, sum
// of exp) over the first nvalid of its CPL staged columns (column c at
// rowp[(c0 + c + rot) & 127]), in two passes over the staged row:
// (1) the KK largest values with multiplicity, by a median-of-three network
//     (slot s takes the median of slots s - 1 and s and the value, slot 0
//     the maximum): KK branch-free operations per value, NaN passing over;
// (2) the columns holding a value >= the KK-th largest, marked in bitmasks
//     and walked in column order: each takes the first free slot from the
//     first slot that holds its value, so equal values keep column order and
//     values equal to the KK-th largest beyond the list are dropped. Only
//     the marked columns (about KK per lane) run the slot search.
// Unfilled slots are empty keys (0), as a list that saw fewer values.
template <int KK, int CPL, bool LSE>
__device__ __forceinline__ void select_lane(const float *rowp, int c0, int rot, int nvalid, int colbase,
                                            uint64_t (&L)[KK], float &mx, float &se) {
    static_assert(KK <= 16 && CPL % 64 == 0, "list and mask sizes");
    constexpr int NB8 = CPL / 8, NM = CPL / 64;
    auto load8 = [&](int b, float (&xs)[8]) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const f32x4_t t = *reinterpret_cast<const f32x4_t *>(rowp + ((c0 + b * 8 + 4 * q + rot) & 127));
            xs[4 * q] = t[0]; xs[4 * q + 1] = t[1]; xs[4 * q + 2] = t[2]; xs[4 * q + 3] = t[3];
        }
    };
    float lv[KK];
#pragma unroll
    for (int t = 0; t < KK; ++t) lv[t] = -INFINITY;
    mx = -INFINITY;
    se = 0.f;
#pragma unroll
    for (int b = 0; b < NB8; ++b) {
        const int jv = nvalid - b * 8;  // valid columns in this batch
        if (jv > 0) {
            float xs[8];
            load8(b, xs);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if (i >= jv) xs[i] = -INFINITY;
                const float x = xs[i];
#pragma unroll
                for (int t = KK - 1; t > 0; --t) lv[t] = __builtin_amdgcn_fmed3f(lv[t - 1], lv[t], x);
                lv[0] = e3_vmax(lv[0], x);
            }
            if (LSE) {
                float bm = xs[0];
#pragma unroll
                for (int i = 1; i < 8; ++i) bm = fmaxf(bm, xs[i]);
                const float nm = fmaxf(mx, bm);
                if (nm != -INFINITY) {
                    float sb = 0.f;
#pragma unroll
                    for (int i = 0; i < 8; ++i) sb += __expf(xs[i] - nm);
                    se = se * __expf(mx - nm) + sb;
                    mx = nm;
                }
            }
        }
    }
    const float thr = lv[KK - 1];
    uint64_t cand[NM];
#pragma unroll
    for (int w = 0; w < NM; ++w) cand[w] = 0;
#pragma unroll
    for (int b = 0; b < NB8; ++b) {
        const int jv = nvalid - b * 8;
        if (jv > 0) {
            float xs[8];
            load8(b, xs);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (i < jv && xs[i] >= thr) cand[(b * 8 + i) / 64] |= 1ull << ((b * 8 + i) % 64);
        }
    }
    int idx[KK];
#pragma unroll
    for (int t = 0; t < KK; ++t) idx[t] = 0;
    uint32_t taken = 0;
#pragma unroll
    for (int w = 0; w < NM; ++w) {
        uint64_t cm = cand[w];
        while (cm) {
            const int col = w * 64 + (int)__builtin_ctzll(cm);
            cm &= cm - 1;
            const float v = rowp[(c0 + col + rot) & 127];
            int s0 = 0;
#pragma unroll
            for (int t = 0; t < KK; ++t) s0 += lv[t] > v ? 1 : 0;
            const uint32_t fr = ~taken & (((1u << KK) - 1u) & ~((1u << s0) - 1u));
            if (fr) {
                const int slot = (int)__builtin_ctz(fr);
                taken |= 1u << slot;
#pragma unroll
                for (int t = 0; t < KK; ++t) idx[t] = t == slot ? col : idx[t];
            }
        }
    }
#pragma unroll
    for (int t = 0; t < KK; ++t) L[t] = (taken >> t) & 1u ? e3_key(lv[t], colbase + idx[t]) : 0;
}

template <int BM, int KK, bool LSE>
__global__ __launch_bounds__(256, BM == 128 ? 2 : 1) void lmhead_big_kernel(e3g::GemmParams gp, int nrec,
                                                                             Partials p) {
    using T = e3g::GTile<BM, BM == 128 ? 3 : 4>;
    constexpr int LPR = BM == 256 ? 1 : 2;  // lanes per hidden row in the selection
    constexpr int RP = 64 / LPR;            // hidden rows staged per pass
    constexpr int CPL = 128 / LPR;          // columns one lane scans
    constexpr int MBP = RP / 32;            // 32-row accumulator blocks per pass
    __shared__ __attribute__((aligned(1024))) unsigned char ring[T::RING];
    __shared__ int arow[3][BM];
    static_assert(4 * RP * 128 * sizeof(float) <= sizeof(ring), "per-wave staging must fit the ring");
    // the GEMM core's order: each XCD a contiguous run of tiles, vocabulary
    // tiles fastest within groups of 8 hidden tiles, so the 32 work-groups an
    // XCD runs together share 8 hidden and 4 vocabulary tiles in its L2
    // (hidden tiles fastest over all of them left each hidden tile shared by
    // 2: 13.4 GB of L2 misses per 3904-row launch against 8.1 GB here)
    // (4 hidden tiles per group: measured 3.75 -> 3.47 ms together with the
    // loop's issue priority on the 3904-row shape, against groups of 8)
    int mt, nt;
    e3g::tile_of<4>(blockIdx.x, gridDim.x, gp.mt, gp.nt, mt, nt);
    const int m0 = mt * BM, n0 = nt * BIG_BN;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int lr = lane & 31, lh = lane >> 5, wm = wave >> 1, wn = wave & 1;
    e3g::fill_arow<BM>(gp, m0, arow);
    f32x16_t acc[T::MB][T::NB];
    // Top-2 lists without a log-sum-exp (the verify step's argmax and gap):
    // the transposed tile puts one hidden row in each lane, so the selection
    // runs on the accumulators directly, with no LDS staging.
    constexpr bool REG_TOP2 = KK == 2 && !LSE && BM == 256;
    e3g::mainloop<BM, T::NS, REG_TOP2>(gp, m0, n0, 0, gp.K / e3g::GBK, ring, arow, acc);
    if constexpr (REG_TOP2) {
        const int vbase = n0 + wn * 128;
        const int nvalid = gp.N - vbase;
        const int rec_tile = 2 * nt + wn;
#pragma unroll
        for (int mb = 0; mb < T::MB; ++mb) {
            float b0, b1;
            int i0, i1;
            top2_row<T::NB>(acc[mb], lh, nvalid, b0, i0, b1, i1);
            const int m = m0 + wm * (BM / 2) + 32 * mb + lr;
            if (lh == 0 && m < gp.M) {
                uint64_t L[KK];
                L[0] = i0 == NO_COL ? 0 : e3_key(b0, vbase + i0);
                L[1] = i1 == NO_COL ? 0 : e3_key(b1, vbase + i1);
                store_record<KK>(p, (size_t)m * nrec + rec_tile, L);
            }
        }
        return;
    }
    __syncthreads();  // every wave is done with the ring
    // Each wave selects over its own (BM/2) x 128 block, RP hidden rows at a
    // time, staged in a private slice of the ring (columns rotated by 4 per
    // row). Lane (row, ch) scans CPL columns of its row; with two lanes per
    // row the halves merge by one shuffle. The record is (row, 2 * tile + wn).
    float *st = reinterpret_cast<float *>(ring) + wave * RP * 128;
    const int vbase = n0 + wn * 128;
    const int rec_tile = 2 * nt + wn;
    const int row = lane % RP, ch = lane / RP;
#pragma unroll
    for (int pass = 0; pass < T::MB / MBP; ++pass) {
#pragma unroll
        for (int mbi = 0; mbi < MBP; ++mbi)
#pragma unroll
            for (int nb = 0; nb < T::NB; ++nb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int sr = mbi * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
                    st[sr * 128 + ((nb * 32 + lr + 4 * sr) & 127)] = acc[pass * MBP + mbi][nb][r];
                }
        // a wave's LDS accesses complete in order: the scan below sees the stores
        uint64_t L[KK];
        float mx, se;
        const int c0 = CPL * ch;
        const int nvalid = min(CPL, gp.N - vbase - c0);
        select_lane<KK, CPL, LSE>(st + row * 128, c0, 4 * row, nvalid, vbase + c0, L, mx, se);
        if constexpr (LPR == 2) {
            e3_kmerge_xor<KK>(L, 32);
            if (LSE) {
                const float m2 = __shfl_xor(mx, 32), s2 = __shfl_xor(se, 32);
                e3_lse_combine(mx, se, m2, s2);
            }
        }
        const int m = m0 + wm * (BM / 2) + pass * RP + row;
        if (ch == 0 && m < gp.M) {
            const size_t rec = (size_t)m * nrec + rec_tile;
            store_record<KK>(p, rec, L);
            if (LSE) { p.mx[rec] = mx; p.se[rec] = se; }
        }
    }
}

// Top-2 lists without a log-sum-exp over many rows with eight waves per
// 256 x 256 tile (two per SIMD, each 128 rows x 64 vocabulary columns): while
// one wave of a SIMD waits on a barrier or a load, the other issues MFMAs.
// The two waves of each 128-column half merge their lists through LDS, so
// the records are those of the four-wave kernel: one per (hidden row,
// 128-column half tile).
__global__ __launch_bounds__(512, 1) void lmhead_top2_w8_kernel(e3g::GemmParams gp, int nrec, Partials p) {
    using T = e3g::GTile<256, 4, 8>;
    constexpr int BM = 256;
    __shared__ __attribute__((aligned(1024))) unsigned char ring[T::RING];
    __shared__ int arow[3][BM];
    static_assert(T::WN == 4 && T::CW == 64, "two waves per 128-column half");
    int mt, nt;
    e3g::tile_of<4>(blockIdx.x, gridDim.x, gp.mt, gp.nt, mt, nt);
    const int m0 = mt * BM, n0 = nt * BIG_BN;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int lr = lane & 31, lh = lane >> 5, wm = wave / T::WN, wn = wave % T::WN;
    e3g::fill_arow<BM>(gp, m0, arow);
    f32x16_t acc[T::MB][T::NB];
    e3g::mainloop<BM, T::NS, true, 8>(gp, m0, n0, 0, gp.K / e3g::GBK, ring, arow, acc);
    const int vbase = n0 + wn * T::CW;
    const int nvalid = gp.N - vbase;
    uint64_t own[T::MB][2];
#pragma unroll
    for (int mb = 0; mb < T::MB; ++mb) {
        float b0, b1;
        int i0, i1;
        top2_row<T::NB>(acc[mb], lh, nvalid, b0, i0, b1, i1);
        own[mb][0] = i0 == NO_COL ? 0 : e3_key(b0, vbase + i0);
        own[mb][1] = i1 == NO_COL ? 0 : e3_key(b1, vbase + i1);
    }
    // odd waves hand their lists to the even wave of the same half
    __syncthreads();  // every wave is done with the ring
    uint64_t *xk = reinterpret_cast<uint64_t *>(ring) + ((wm * 2 + (wn >> 1)) * T::MB) * 64;
    if ((wn & 1) && lh == 0) {
#pragma unroll
        for (int mb = 0; mb < T::MB; ++mb) {
            xk[mb * 64 + 2 * lr] = own[mb][0];
            xk[mb * 64 + 2 * lr + 1] = own[mb][1];
        }
    }
    __syncthreads();
    if (!(wn & 1) && lh == 0) {
        const int rec_tile = 2 * nt + (wn >> 1);
#pragma unroll
        for (int mb = 0; mb < T::MB; ++mb) {
            const int m = m0 + wm * (BM / 2) + 32 * mb + lr;
            if (m < gp.M) {
                const uint64_t y0 = xk[mb * 64 + 2 * lr], y1 = xk[mb * 64 + 2 * lr + 1];
                const uint64_t x0 = own[mb][0], x1 = own[mb][1];
                uint64_t L[2];
                if (x0 >= y0) { L[0] = x0; L[1] = x1 > y0 ? x1 : y0; }
                else { L[0] = y0; L[1] = y1 > x0 ? y1 : x0; }
                store_record<2>(p, (size_t)m * nrec + rec_tile, L);
            }
        }
    }
}

// The same top-2 tiles, persistent: one work-group per CU takes tiles from
// the run of the tile order that belongs to its XCD (work-group w is
// dispatched to XCD w mod 8), so an XCD's work-groups work on neighbouring
// tiles together, and the LDS-DMA ring runs on from one tile into the next:
// the next tile's first chunks load during the last chunks and the selection
// of the current one. Tiles are claimed from a counter per XCD run (zeroed
// before the pass); a work-group whose XCD's run is used up takes tiles from
// the other runs, so XCDs that run slower (by ~10% on the 3904-row head) do
// not set the end. Claims are made by thread 0 one tile ahead of need: the
// claim for the tile after next is issued at a tile boundary and read at the
// next boundary, after that boundary's wait for all loads. The lists are
// exchanged through a buffer of their own (the ring holds chunks in flight).
// Same records as above, whichever work-group computes a tile.
__global__ __launch_bounds__(512, 1) void lmhead_top2_w8p_kernel(e3g::GemmParams gp, int nrec, Partials p) {
    using T = e3g::GTile<256, 4, 8>;
    constexpr int BM = 256;
    __shared__ __attribute__((aligned(1024))) unsigned char ring[T::RING];
    __shared__ uint64_t xk_all[2 * 2 * T::MB * 64];
    __shared__ int tq[2];
    static_assert(T::WN == 4 && T::CW == 64, "two waves per 128-column half");
    e3g::TileQueue queue;
    queue.init(p.ctr, tq, gp.mt * gp.nt);
    auto tile_at = [&](int t, int &m0, int &n0) {
        int mt, nt;
        e3g::tile_at_order<4>(t, gp.mt, gp.nt, mt, nt);
        m0 = mt * BM;
        n0 = nt * BIG_BN;
    };
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int lr = lane & 31, lh = lane >> 5, wm = wave / T::WN, wn = wave % T::WN;
    auto epilogue = [&](int tile, const f32x16_t (&acc)[T::MB][T::NB]) {
        int m0, n0;
        tile_at(tile, m0, n0);
        const int nt = n0 / BIG_BN;
        const int vbase = n0 + wn * T::CW;
        const int nvalid = gp.N - vbase;
        // a wave whose rows all lie past M selects nothing
        const bool rows_here = __builtin_amdgcn_readfirstlane(m0 + wm * (BM / 2)) < gp.M;
        uint64_t own[T::MB][2];
        if (rows_here) {
#pragma unroll
            for (int mb = 0; mb < T::MB; ++mb) {
                float b0, b1;
                int i0, i1;
                top2_row<T::NB>(acc[mb], lh, nvalid, b0, i0, b1, i1);
                own[mb][0] = i0 == NO_COL ? 0 : e3_key(b0, vbase + i0);
                own[mb][1] = i1 == NO_COL ? 0 : e3_key(b1, vbase + i1);
            }
        }
        // odd waves hand their lists to the even wave of the same half
        uint64_t *xk = xk_all + ((wm * 2 + (wn >> 1)) * T::MB) * 64;
        if (rows_here && (wn & 1) && lh == 0) {
#pragma unroll
            for (int mb = 0; mb < T::MB; ++mb) {
                xk[mb * 64 + 2 * lr] = own[mb][0];
                xk[mb * 64 + 2 * lr + 1] = own[mb][1];
            }
        }
        // LDS-only barrier: a full one would also wait for the next tile's chunks in flight
        e3g::lds_barrier();
        if (rows_here && !(wn & 1) && lh == 0) {
            const int rec_tile = 2 * nt + (wn >> 1);
#pragma unroll
            for (int mb = 0; mb < T::MB; ++mb) {
                const int m = m0 + wm * (BM / 2) + 32 * mb + lr;
                if (m < gp.M) {
                    const uint64_t y0 = xk[mb * 64 + 2 * lr], y1 = xk[mb * 64 + 2 * lr + 1];
                    const uint64_t x0 = own[mb][0], x1 = own[mb][1];
                    uint64_t L[2];
                    if (x0 >= y0) { L[0] = x0; L[1] = x1 > y0 ? x1 : y0; }
                    else { L[0] = y0; L[1] = y1 > x0 ? y1 : x0; }
                    store_record<2>(p, (size_t)m * nrec + rec_tile, L);
                }
            }
        }
        // the buffer is written again only after the next tile's K loop and its barriers
    };
    e3g::mainloop_persistent<BM, T::NS, true, 8>(gp, tile_at, queue, epilogue, ring);
}

template <int KK, bool LSE>
__global__ __launch_bounds__(256) void lmhead_f32_kernel(const float *__restrict__ h, const float *__restrict__ w,
                                                         int M, int N, int K, int ntiles, Partials p) {
    constexpr int BM = 16, BN = BN_F;
    __shared__ float lg[BM][BN + 4];
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
    tile_select<BM, BN, KK, LSE>(lg, m0, M, n0, N, tile, ntiles, p);
}

template <int KK, bool LSE>
__global__ __launch_bounds__(256) void lmhead_merge_kernel(int M, int ntiles, Partials p, int topk,
                                                           int32_t *__restrict__ idx, float *__restrict__ val,
                                                           float *__restrict__ gap, float *__restrict__ lse) {
    // one wave per row, four rows per work-group: lane l merges the records
    // l, l + 64, ... into its own list, then the wave's 64 lists meet in a
    // butterfly (the list and the row's (max, sum-exp) do not depend on the
    // order in which records meet, up to the rounding of the sum)
    const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (m >= M) return;  // the whole wave
    uint64_t L[KK];
    e3_kinit<KK>(L);
    float mx = -INFINITY, se = 0.f;
    // four records per lane and step, all loaded before any is merged (a
    // 128256-row head has 501 or 1002 records per row: four memory round
    // trips per lane)
    constexpr int U = 4;
    for (int t0 = lane; t0 < ntiles; t0 += 64 * U) {
        uint64_t rk[U][KK];
        float rmx[U], rse[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int t = t0 + 64 * u;
            rmx[u] = -INFINITY;
            rse[u] = 0.f;
#pragma unroll
            for (int s = 0; s < KK; ++s) rk[u][s] = 0;  // below every key: never enters
            if (t < ntiles) {
                const size_t rec = (size_t)m * ntiles + t;
                const u32x4_t *src = reinterpret_cast<const u32x4_t *>(p.key + rec * KK);
#pragma unroll
                for (int s = 0; s < KK; s += 2) {
                    const u32x4_t q = src[s / 2];
                    rk[u][s] = ((uint64_t)q[1] << 32) | q[0];
                    rk[u][s + 1] = ((uint64_t)q[3] << 32) | q[2];
                }
                if (LSE) { rmx[u] = p.mx[rec]; rse[u] = p.se[rec]; }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            // a record is sorted: once an entry cannot enter, none after it can
#pragma unroll
            for (int s = 0; s < KK; ++s) {
                if (!(rk[u][s] > L[KK - 1])) break;
                e3_kinsert<KK>(L, rk[u][s]);
            }
            if (LSE) e3_lse_combine(mx, se, rmx[u], rse[u]);
        }
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        e3_kmerge_xor<KK>(L, off);
        if (LSE) {
            const float m2 = __shfl_xor(mx, off), s2 = __shfl_xor(se, off);
            e3_lse_combine(mx, se, m2, s2);
        }
    }
    if (lane == 0) {
#pragma unroll
        for (int s = 0; s < KK; ++s) {
            if (s < topk) {
                idx[(size_t)m * topk + s] = e3_key_idx(L[s]);
                if (val) val[(size_t)m * topk + s] = e3_key_val(L[s]);
            }
        }
        if (gap) gap[m] = e3_key_val(L[0]) - e3_key_val(L[1]);
        if (LSE) lse[m] = mx + __logf(se);
    }
}

int kk_for(int topk) {
    const int need = topk < 2 ? 2 : topk;
    return need <= 2 ? 2 : need <= 4 ? 4 : need <= 8 ? 8 : need <= 10 ? 10 : 16;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

Partials carve(void *ws, int M, int ntiles, int KK) {
    char *b = (char *)ws;
    const size_t rec = (size_t)M * ntiles;
    Partials p;
    p.key = (uint64_t *)b; b += align256(rec * KK * sizeof(uint64_t));
    p.mx = (float *)b;     b += align256(rec * sizeof(float));
    p.se = (float *)b;     b += align256(rec * sizeof(float));
    p.ctr = (uint32_t *)b;
    return p;
}

// from this many hidden rows on, the bf16 head runs as a dense GEMM
constexpr int BIG_M = 128;

bool use_big(int M, int K, int dtype) { return dtype == EAGLE3_BF16 && M >= BIG_M && K % e3g::GSEG_ALIGN == 0; }

// partial records per row (the many-row path keeps one per 128-column half tile)
// few rows, shortest lists (argmax and gap), one hidden tile: 8 waves over a
// 256-row vocabulary tile, one work-group per CU, halve the hidden-row
// traffic per weight byte (8B batch-1 tile pass 179 -> 171 us); longer
// lists keep 4 waves over 128 rows, whose selection is cheaper per tile
bool wide_tiles(int M, int KK, int dtype) { return dtype == EAGLE3_BF16 && KK == 2 && M <= 64; }

int tiles_for(int M, int N, int K, int dtype, int KK) {
    if (use_big(M, K, dtype)) return 2 * ((N + BIG_BN - 1) / BIG_BN);
    const int bn = dtype == EAGLE3_BF16 ? (wide_tiles(M, KK, dtype) ? 2 * BN_B : BN_B) : BN_F;
    return (N + bn - 1) / bn;
}

template <int KK, bool LSE>
void launch(const void *hidden, const void *w, int M, int N, int K, int topk, int dtype, int32_t *idx, float *val,
            float *gap, float *lse, void *ws, hipStream_t st) {
    const int ntiles = tiles_for(M, N, K, dtype, KK);
    const Partials p = carve(ws, M, ntiles, KK);
    if (use_big(M, K, dtype)) {
        e3g::GemmParams gp{};
        gp.a[0] = hidden; gp.k[0] = K; gp.nseg = 1;
        gp.b = w; gp.M = M; gp.N = N; gp.K = K; gp.ldc = N;
        constexpr int BM = big_bm(KK);
        gp.mt = (M + BM - 1) / BM; gp.nt = (N + BIG_BN - 1) / BIG_BN;
        if constexpr (KK == 2 && !LSE) {
            if (K / e3g::GBK >= 4) {  // the persistent loop keeps 4 chunks of one tile in flight
                e3g::ctr_zero_kernel<<<1, 64, 0, st>>>(p.ctr);
                lmhead_top2_w8p_kernel<<<std::min(gp.mt * gp.nt, e3_cu_count()), 512, 0, st>>>(gp, ntiles, p);
            } else
                lmhead_top2_w8_kernel<<<gp.mt * gp.nt, 512, 0, st>>>(gp, ntiles, p);
        } else
            lmhead_big_kernel<BM, KK, LSE><<<gp.mt * gp.nt, 256, 0, st>>>(gp, ntiles, p);
    } else if (dtype == EAGLE3_BF16) {
        dim3 grid((M + 63) / 64, ntiles);
        const uint16_t *hp = (const uint16_t *)hidden, *wp = (const uint16_t *)w;
        if (wide_tiles(M, KK, dtype))
            lmhead_bf16_kernel<KK, LSE, true, 8><<<grid, 512, 0, st>>>(hp, wp, M, N, K, ntiles, p);
        else if (grid.x == 1)
            lmhead_bf16_kernel<KK, LSE, true, 4><<<grid, 256, 0, st>>>(hp, wp, M, N, K, ntiles, p);
        else
            lmhead_bf16_kernel<KK, LSE, false, 4><<<grid, 256, 0, st>>>(hp, wp, M, N, K, ntiles, p);
    } else {
        dim3 grid((M + 15) / 16, ntiles);
        lmhead_f32_kernel<KK, LSE><<<grid, 256, 0, st>>>((const float *)hidden, (const float *)w, M, N, K, ntiles, p);
    }
    lmhead_merge_kernel<KK, LSE><<<(M + 3) / 4, 256, 0, st>>>(M, ntiles, p, topk, idx, val, gap, lse);
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
    const int KK = kk_for(topk);
    const int ntiles = tiles_for(M, N, K, dtype, KK);
    const size_t rec = (size_t)M * ntiles;
    return align256(rec * KK * 8) + align256(rec * 4) + align256(rec * 4) + CTR_BYTES;
}

extern "C" int eagle3_lmhead_argmax(const void *hidden, const void *w, int M, int N, int K, int topk, int dtype,
                                    int32_t *idx, float *val, float *gap, float *lse, void *ws, size_t ws_bytes,
                                    void *stream) {
    if (M < 0 || N < 0 || K < 1 || topk < 1) return EAGLE3_ERR_ARG;
    if (topk > 16 || N < 2 || topk > N) return EAGLE3_ERR_UNSUPPORTED;
    if (dtype != EAGLE3_BF16 && dtype != EAGLE3_F32) return EAGLE3_ERR_UNSUPPORTED;
    if (dtype == EAGLE3_BF16 && K % 64 != 0) return EAGLE3_ERR_UNSUPPORTED;
    if (dtype == EAGLE3_BF16 && (uint64_t)M * K * 2 >= (1ull << 32)) return EAGLE3_ERR_UNSUPPORTED;
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
        case 10: launch_kk<10>(want_lse, hidden, w, M, N, K, topk, dtype, idx, val, gap, lse, ws, st); break;
        default: launch_kk<16>(want_lse, hidden, w, M, N, K, topk, dtype, idx, val, gap, lse, ws, st); break;
    }
    E3_LAUNCH_CHECK();
    return EAGLE3_OK;
}

// ------------------------------------------------ entry point that allocates nothing
// For callers that cannot allocate (code under graph capture, tight serving
// loops): the same LM-head argmax with its per-tile records in a file-scope
// device array instead of a caller workspace. Each GPU the library runs on
// holds its own copy of the array until the process ends; every call on that
// GPU reuses it, so calls that overlap on one GPU race. The records are all
// written before they are read, so nothing needs clearing between calls.
static __device__ __align__(256) unsigned char scratch[EAGLE3_LMHEAD_NOALLOC_MAX_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, from hipGetSymbolAddress

// The array's device address on the current device (looked up once per
// device, with that device current). In host code the array's own name is
// not a device address and is never passed to a kernel or a copy.
int scratch_address(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return EAGLE3_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return EAGLE3_ERR_HIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return EAGLE3_OK;
}
}  // namespace

extern "C" int eagle3_lmhead_argmax_noalloc(const void *hidden, const void *w, int M, int N, int K, int topk,
                                            int dtype, int32_t *idx, float *val, float *gap, float *lse,
                                            void *stream) {
    if (M < 0 || N < 0 || K < 1 || topk < 1) return EAGLE3_ERR_ARG;
    if (topk > 16 || N < 2 || topk > N) return EAGLE3_ERR_UNSUPPORTED;
    if (dtype != EAGLE3_BF16 && dtype != EAGLE3_F32) return EAGLE3_ERR_UNSUPPORTED;
    if (M == 0) return EAGLE3_OK;
    // the records this call needs must fit the array (checked before any HIP call)
    if (eagle3_lmhead_workspace(M, N, K, topk, dtype) > EAGLE3_LMHEAD_NOALLOC_MAX_BYTES) return EAGLE3_ERR_WORKSPACE;
    void *ptr = nullptr;
    const int rc = scratch_address(&ptr);
    if (rc != EAGLE3_OK) return rc;
    return eagle3_lmhead_argmax(hidden, w, M, N, K, topk, dtype, idx, val, gap, lse, ptr,
                                EAGLE3_LMHEAD_NOALLOC_MAX_BYTES, stream);
}
