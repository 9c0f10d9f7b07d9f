// bf16 GEMM core shared by the dense layers and the large-batch LM head:
// C = A . B^T over one output tile, A [M, K] (up to three K-segments, each
// optionally row-gathered) and B [N, K], both k-contiguous; fp32 accumulators
// stay in registers for the caller's epilogue.
#pragma once
#include "common.h"

namespace e3g {

typedef __attribute__((address_space(3))) void lds_void_t;

// bf16 GEMM tiles: BM x 256 outputs per 256-thread work-group (BM = 256 or
// 128), waves 2 x 2, each (BM/2) x 128 in 32 x 32 MFMA blocks. K advances in
// chunks of 32 through an NS-stage LDS ring filled by 16-byte
// global_load_lds: NS = 4 keeps three chunks in flight while one is
// multiplied (one work-group per CU); BM = 128 with NS = 3 takes 72 KB, so
// two work-groups share a CU and one's waits are covered by the other's MFMAs.
constexpr int GBN = 256, GBK = 32, GROW = GBK * 2;  // LDS row: 32 bf16 = 64 B
constexpr int GSEG_ALIGN = 64;                                 // segment widths are multiples of this

// NW = 4: waves 2 x 2, each (BM/2) x 128; NW = 8: waves 2 x 4, each
// (BM/2) x 64 (two waves per SIMD share the same ring and tile).
template <int BM, int NS_ = 4, int NW_ = 4>
struct GTile {
    static constexpr int NW = NW_;                      // waves per work-group
    static constexpr int WN = NW / 2;                   // waves along N
    static constexpr int CW = GBN / WN;                 // columns per wave
    static constexpr int STAGE = (BM + GBN) * GROW;    // bytes per ring stage
    static constexpr int LOADS = STAGE / 1024 / NW;    // 1 KB DMA loads per wave per stage
    static constexpr int MB = BM / 64, NB = CW / 32;    // 32 x 32 blocks per wave
    static constexpr int NS = NS_;                      // ring stages
    static constexpr int RING = NS * STAGE;             // ring bytes
};

struct GemmParams {
    const void *a[3];
    const int32_t *a_rows[3];
    int k[3];
    int kofs[3];
    int nseg;
    const void *b;
    const void *res;
    void *c;
    int M, N, K, ldc, a_nrows[3];
    int mt, nt;  // tile counts
};

// 16-byte column of a 64-byte LDS row, XOR-swizzled so that the 32 rows an
// MFMA operand read touches spread over all banks (16 consecutive rows land
// on 16 distinct 16-byte slots of a 256-byte window, 8 rows on 8 slots of 128)
__device__ __forceinline__ int gswz(int row) { return (row ^ (row >> 2)) & 3; }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// wait until at most N LDS reads are outstanding; the fragments are tied to
// the wait so no use of them can be scheduled above it
template <int N, int MB, int NB = 4>
__device__ __forceinline__ void lgkm_wait(u32x4_t *av, u32x4_t *bv) {
    static_assert((MB == 2 || MB == 4) && (NB == 2 || NB == 4), "fragment count");
    if constexpr (NB == 2) {
        static_assert(MB == 4, "fragment count");
        __asm__ volatile("s_waitcnt lgkmcnt(%6)"
                         : "+v"(av[0]), "+v"(av[1]), "+v"(av[2]), "+v"(av[3]), "+v"(bv[0]), "+v"(bv[1])
                         : "i"(N));
    } else if constexpr (MB == 4) {
        __asm__ volatile("s_waitcnt lgkmcnt(%8)"
                         : "+v"(av[0]), "+v"(av[1]), "+v"(av[2]), "+v"(av[3]), "+v"(bv[0]), "+v"(bv[1]),
                           "+v"(bv[2]), "+v"(bv[3])
                         : "i"(N));
    } else {
        __asm__ volatile("s_waitcnt lgkmcnt(%6)"
                         : "+v"(av[0]), "+v"(av[1]), "+v"(bv[0]), "+v"(bv[1]), "+v"(bv[2]), "+v"(bv[3])
                         : "i"(N));
    }
}

// Work-group id -> output tile. Work-groups are dealt to the 8 XCDs in turn;
// give each XCD a contiguous run of tiles, ordered N-fastest within groups of
// G M-tiles, so the tiles one XCD runs together share A rows and B rows in its L2.
// Position t of the tile order -> tile (N-fastest within groups of G M-tiles).
template <int G = 8>
__device__ __forceinline__ void tile_at_order(int t, int MT, int NT, int &mt, int &nt) {
    const int gsz_full = G * NT;
    const int g = t / gsz_full, first = g * G, gs = min(G, MT - first);
    const int u = t - g * gsz_full;
    mt = first + u % gs;
    nt = u / gs;
}

template <int G = 8>
__device__ __forceinline__ void tile_of(int L, int nwg, int MT, int NT, int &mt, int &nt) {
    const int q = nwg >> 3, r = nwg & 7, x = L & 7, j = L >> 3;
    const int t = (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + j;
    const int gsz_full = G * NT;
    const int g = t / gsz_full, first = g * G, gs = min(G, MT - first);
    const int u = t - g * gsz_full;
    mt = first + u % gs;
    nt = u / gs;
}

// Source row of each tile row, per segment (rows past M clamp to M - 1; their
// results are dropped by the epilogue).
// The segment index is a compile-time constant in every access to p: a
// run-time index would place the whole parameter block in private memory.
template <int BM>
__device__ __forceinline__ void fill_arow(const GemmParams &p, int m0, int (*arow)[BM]) {
#pragma unroll
    for (int s = 0; s < 3; ++s) {
        const int32_t *rows = s == 0 ? p.a_rows[0] : s == 1 ? p.a_rows[1] : p.a_rows[2];
        const int nrows = s == 0 ? p.a_nrows[0] : s == 1 ? p.a_nrows[1] : p.a_nrows[2];
        for (int r = threadIdx.x; r < BM; r += blockDim.x) {
            int m = min(m0 + r, p.M - 1);
            if (s < p.nseg && rows) m = min(max(rows[m], 0), nrows - 1);
            arow[s][r] = m;
        }
    }
    __syncthreads();
}

// The K loop of one BM x 256 tile at (m0, n0) over the k chunks c_begin ..
// c_begin + nch - 1 (32 columns each; a split of K, or all of it). ring:
// GTile<BM, NS>::RING
// bytes of LDS (1 KB aligned). On return acc holds the tile: wave (wm, wn) =
// (wave / WN, wave % WN) with CW = 256 / WN columns per wave, block (mb, nb),
// register r of lane (lr, lh) is
// C[m0 + wm BM/2 + 32 mb + 8 (r / 4) + 4 lh + r % 4][n0 + CW wn + 32 nb + lr],
// or with TRANS (the MFMA operands swapped, same loads) its transpose:
// C[m0 + wm BM/2 + 32 mb + lr][n0 + CW wn + 32 nb + 8 (r / 4) + 4 lh + r % 4],
// so a lane's registers hold one row of A's tile.
// The waves run at raised issue priority for the loop (measured on the
// 3904 x 128256 x 4096 LM-head shape with random bf16 data: 3.75 -> 3.53 ms).
__device__ __forceinline__ const uint16_t *e3_uniform_ptr(const uint16_t *q) {
    const uint64_t v = (uint64_t)q;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const uint16_t *)(((uint64_t)hi << 32) | lo);
}

template <int BM, int NS, bool TRANS = false, int NW = 4>
__device__ __forceinline__ void mainloop(const GemmParams &p, int m0, int n0, int c_begin, int nch,
                                         unsigned char *ring, const int (*arow)[BM],
                                         f32x16_t (&acc)[GTile<BM, NS, NW>::MB][GTile<BM, NS, NW>::NB]) {
    using T = GTile<BM, NS, NW>;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int lr = lane & 31, lh = lane >> 5;
    // load j of this wave fills stage block blk = wave * LOADS + j (16 rows of
    // 64 B; A rows first, then B rows); lane -> row 16 blk + lane / 4, slot lane % 4.
    // Source pointers are formed once per A segment; a chunk only adds its k offset.
    const int slot = lane & 3;
    // Each load address is a wave-uniform base (scalar registers) plus a
    // 32-bit per-lane byte offset fixed for the whole loop, so a chunk's loads
    // only add the chunk's k offset to the scalar base. The LDS destination
    // of a load is wave-uniform too (the wave index from readfirstlane).
    const int wave_u = __builtin_amdgcn_readfirstlane(tid >> 6);
    const char *abase = nullptr;  // the current A segment's base (wave-uniform)
    uint32_t voff[T::LOADS];
    int seg = 0;
    // segment fields by constant index only (a run-time index would turn
    // these kernel-argument reads into per-chunk memory loads)
    // wave-uniform copies (readfirstlane): values read through p are not
    // known to be uniform, and a per-lane segment test or loop bound turns
    // the loop control into exec-mask arithmetic
    const int kofs1 = __builtin_amdgcn_readfirstlane(p.nseg > 1 ? p.kofs[1] : 0x7fffffff);
    const int kofs2 = __builtin_amdgcn_readfirstlane(p.nseg > 2 ? p.kofs[2] : 0x7fffffff);
    const bool multi_seg = kofs1 != 0x7fffffff;
    const int kfull = __builtin_amdgcn_readfirstlane(p.K);
    const char *bbase = (const char *)e3_uniform_ptr((const uint16_t *)p.b + (size_t)n0 * kfull);
    auto set_bases = [&](int sg) {
        const uint16_t *aseg = (const uint16_t *)(sg == 0 ? p.a[0] : sg == 1 ? p.a[1] : p.a[2]);
        const int kseg = __builtin_amdgcn_readfirstlane(sg == 0 ? p.k[0] : sg == 1 ? p.k[1] : p.k[2]);
        const int oseg = sg == 0 ? 0 : sg == 1 ? kofs1 : kofs2;
        abase = (const char *)e3_uniform_ptr(aseg - oseg);
#pragma unroll
        for (int j = 0; j < T::LOADS; ++j) {
            const int blk = wave_u * T::LOADS + j;
            const int row = blk * 16 + (lane >> 2);
            if (blk * 16 < BM) {
                voff[j] = (uint32_t)(((size_t)arow[sg][row] * kseg + 8 * (slot ^ gswz(row))) * 2);
            } else {
                const int n = min(n0 + row - BM, p.N - 1);
                voff[j] = (uint32_t)(((size_t)(n - n0) * kfull + 8 * (slot ^ gswz(row))) * 2);
            }
        }
    };
    // the scalar base of load j: A rows (the first BM rows of a stage) or B
    // rows. When BM is a multiple of one wave's rows per stage, all loads of
    // a wave are A rows or all are B rows: one base per wave, no per-load
    // select (which the compiler forms in vector registers)
    constexpr bool WAVE_SIDE = BM % (T::LOADS * 16) == 0;
    auto sbase = [&](int j) {
        if constexpr (WAVE_SIDE) return wave_u * T::LOADS * 16 < BM ? abase : bbase;
        else return (wave_u * T::LOADS + j) * 16 < BM ? abase : bbase;
    };
    set_bases(0);
    // B rows use the full K offset kc; A rows the offset within the segment (kofs folded into the base)
    auto issue = [&](int stage, int kc) {
        const int sg = kc >= kofs2 ? 2 : kc >= kofs1 ? 1 : 0;  // chunks arrive in k order
        if (sg != seg) {
            seg = sg;
            set_bases(seg);
        }
        unsigned char *base = ring + stage * T::STAGE;
#pragma unroll
        for (int j = 0; j < T::LOADS; ++j) {
            const int blk = wave_u * T::LOADS + j;
            __builtin_amdgcn_global_load_lds((const void *)(sbase(j) + (size_t)kc * 2 + voff[j]),
                                             (lds_void_t *)(base + blk * 1024), 16, 0, 0);
        }
    };

#pragma unroll
    for (int i = 0; i < T::MB; ++i)
#pragma unroll
        for (int jj = 0; jj < T::NB; ++jj)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][jj][r] = 0.f;

#pragma unroll
    for (int st = 0; st < T::NS - 1; ++st)
        if (st < nch) issue(st, (c_begin + st) * GBK);
    const int wm = wave / T::WN, wn = wave % T::WN;
    // per-lane LDS byte offsets of the operand rows (sub-step 0 and 1 differ by the column)
    int aoff[T::MB][2], boff[T::NB][2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const int cl = 2 * s + lh;  // both operands take k = 16 s + 8 lh .. +7 of the chunk
#pragma unroll
        for (int mb = 0; mb < T::MB; ++mb) {
            const int row = wm * (BM / 2) + mb * 32 + lr;
            aoff[mb][s] = row * GROW + ((cl ^ gswz(row)) << 4);
        }
#pragma unroll
        for (int nb = 0; nb < T::NB; ++nb) {
            const int row = wn * T::CW + nb * 32 + lr;
            boff[nb][s] = BM * GROW + row * GROW + ((cl ^ gswz(row)) << 4);
        }
    }
    auto wait_chunk = [&](int c) {  // chunk c has landed in LDS for every wave
        const int ahead = min(nch - 1 - c, T::NS - 2);
        if (ahead >= 2) wait_vmcnt<2 * T::LOADS>();
        else if (ahead == 1) wait_vmcnt<T::LOADS>();
        else wait_vmcnt<0>();
        // bare barrier: a fenced one would drain the chunks still in flight
        __builtin_amdgcn_s_barrier();
        __asm__ volatile("" ::: "memory");
    };
    u32x4_t av0[T::MB], bv0[T::NB], av1[T::MB], bv1[T::NB];
    // Fragment reads are issued as inline ds_read_b128: the compiler cannot
    // tell ring slots apart and would otherwise wait for every LDS DMA still
    // in flight before each read. Completion is awaited explicitly (lgkm).
    const uint32_t ring_lds = (uint32_t)(uintptr_t)(lds_void_t *)ring;
    constexpr int NMF = T::MB * T::NB;  // MFMAs per half-chunk
    constexpr int NRD = T::MB + T::NB;  // fragment reads per half-chunk
    static_assert(NRD <= NMF && T::LOADS <= NMF, "one read and one load per MFMA at most");
    auto rd = [&](int slotk, int s, int i, u32x4_t *av, u32x4_t *bv) {
        const uint32_t base = ring_lds + slotk * T::STAGE;
        if (i < T::MB) __asm__ volatile("ds_read_b128 %0, %1" : "=v"(av[i]) : "v"(base + aoff[i][s]));
        else __asm__ volatile("ds_read_b128 %0, %1" : "=v"(bv[i - T::MB]) : "v"(base + boff[i - T::MB][s]));
    };
    auto mf = [&](int j, const u32x4_t *av, const u32x4_t *bv) {
        const int mb = j / T::NB, nb = j % T::NB;
        // the A and B operand formats of the 32 x 32 x 16 MFMA are the same
        // per lane (row or column lr, k = 8 lh .. 8 lh + 7), so swapping the
        // fragments transposes the block
        if constexpr (TRANS)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, bv[nb]),
                                                                  __builtin_bit_cast(bf16x8_t, av[mb]), acc[mb][nb],
                                                                  0, 0, 0);
        else
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, av[mb]),
                                                                  __builtin_bit_cast(bf16x8_t, bv[nb]), acc[mb][nb],
                                                                  0, 0, 0);
    };
    auto dma = [&](int stage, int kc, int j) {
        const int blk = wave_u * T::LOADS + j;
        __builtin_amdgcn_global_load_lds((const void *)(sbase(j) + (size_t)kc * 2 + voff[j]),
                                         (lds_void_t *)(ring + stage * T::STAGE + blk * 1024), 16, 0, 0);
    };
    auto select_seg = [&](int kc) {
        const int sg = kc >= kofs2 ? 2 : kc >= kofs1 ? 1 : 0;  // chunks arrive in k order
        if (sg != seg) {
            seg = sg;
            set_bases(seg);
        }
    };
    // Software pipeline, one wave per SIMD: each instruction between two
    // MFMA groups would leave the matrix pipe idle, so the fragment reads of
    // the next half-chunk and the DMA loads of a later chunk sit between the
    // MFMAs of the current one (scheduling barriers pin that order).
    // A: MFMAs of (c, first half) with the reads of (c, second half) between them.
    auto phase_a = [&](int c) {
        lgkm_wait<0, T::MB, T::NB>(av0, bv0);
        const int sl = c % T::NS;
#pragma unroll
        for (int j = 0; j < NMF; ++j) {
            mf(j, av0, bv0);
            __builtin_amdgcn_sched_barrier(0);
            if (j < NRD) {
                rd(sl, 1, j, av1, bv1);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        lgkm_wait<0, T::MB, T::NB>(av1, bv1);
    };
    // C: MFMAs of (c, second half) with the reads of (c + 1, first half) and,
    // when `refill`, the loads of chunk c + NS into chunk c's slot.
    auto phase_c = [&](int c, bool next, bool refill) {
        const int sl = (c + 1) % T::NS, kc = (c_begin + c + T::NS) * GBK;
        if (refill && multi_seg) select_seg(kc);
        if (next && refill) {
#pragma unroll
            for (int j = 0; j < NMF; ++j) {
                mf(j, av1, bv1);
                __builtin_amdgcn_sched_barrier(0);
                if (j < NRD) {
                    rd(sl, 0, j, av0, bv0);
                    __builtin_amdgcn_sched_barrier(0);
                }
                if (j >= NMF - T::LOADS) {
                    dma(c % T::NS, kc, j - (NMF - T::LOADS));
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        } else if (next) {
#pragma unroll
            for (int j = 0; j < NMF; ++j) {
                mf(j, av1, bv1);
                __builtin_amdgcn_sched_barrier(0);
                if (j < NRD) {
                    rd(sl, 0, j, av0, bv0);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < NMF; ++j) mf(j, av1, bv1);
        }
    };
    __builtin_amdgcn_s_setprio(3);
    if (nch > 0) {
        wait_chunk(0);
        if (T::NS - 1 < nch) issue(T::NS - 1, (c_begin + T::NS - 1) * GBK);
#pragma unroll
        for (int i = 0; i < NRD; ++i) rd(0, 0, i, av0, bv0);
    }
    // steady state: every chunk refills a slot, wait depth is fixed
    const int steady = __builtin_amdgcn_readfirstlane(nch - T::NS);
    for (int c = 0; c < steady; ++c) {
        phase_a(c);
        wait_vmcnt<(T::NS - 2) * T::LOADS>();  // chunk c + 1 has landed (later ones may be in flight)
        __builtin_amdgcn_s_barrier();
        __asm__ volatile("" ::: "memory");
        phase_c(c, true, true);
    }
    for (int c = steady < 0 ? 0 : steady; c < nch; ++c) {
        phase_a(c);
        if (c + 1 < nch) {
            wait_chunk(c + 1);
            phase_c(c, true, false);
        } else {
            phase_c(c, false, false);
        }
    }
    __builtin_amdgcn_s_setprio(0);
}


// Tile-claim counters of the persistent kernels: one per XCD run, 128 bytes
// apart, in a caller's workspace, zeroed by ctr_zero_kernel before a pass.
constexpr int CTR_STRIDE = 32;
constexpr size_t CTR_BYTES = 8 * CTR_STRIDE * sizeof(uint32_t);
static_assert(CTR_BYTES <= EAGLE3_PERSIST_WS_BYTES, "the counters fit the documented workspace");
// a tile claim: a global (not flat) atomic, counted by vmcnt only, so a wait
// for LDS operations does not wait for a claim in flight
__device__ __forceinline__ uint32_t claim_tile(uint32_t *ctr) {
    typedef __attribute__((address_space(1))) uint32_t global_u32;
    return __hip_atomic_fetch_add((global_u32 *)ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <int UNUSED = 0>
__global__ void ctr_zero_kernel(uint32_t *ctr) {
    if (threadIdx.x < 8) ctr[threadIdx.x * CTR_STRIDE] = 0;
}

// barrier over LDS operations only (no wait for vector memory operations)
__device__ __forceinline__ void lds_barrier() {
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
}

// Tile queue of the persistent kernels: the tile order is cut into 8
// runs, one per XCD, each with a claim counter; thread 0 claims for the
// work-group and broadcasts through LDS. first() and advance() are called by
// every thread at points with no load in flight. A work-group claims its
// second tile at the start, unless there are no more tiles than work-groups
// (then each takes one).
struct TileQueue {
    uint32_t *ctr;
    int *tq;              // LDS broadcast slots
    int x, q, r8;         // own run; tiles per run = q (+1 for the first r8 runs)
    int ntiles;           // tiles of the pass
    uint32_t pend;        // thread 0: the claim in flight on the own run
    bool own_left;        // thread 0: the own run may still have tiles
    __device__ __forceinline__ void init(uint32_t *c, int *slots, int ntiles) {
        ctr = c; tq = slots;
        x = blockIdx.x & 7; q = ntiles >> 3; r8 = ntiles & 7; this->ntiles = ntiles;
        pend = 0; own_left = true;
    }
    __device__ __forceinline__ int run_start(int v) const { return v * q + min(v, r8); }
    __device__ __forceinline__ int run_cnt(int v) const { return q + (v < r8 ? 1 : 0); }
    // thread 0: a tile from the runs first_run, first_run + 1, ... (waits for each claim)
    __device__ __forceinline__ int claim(int first_run) {
        for (int d = 0; d < 8; ++d) {
            const int v = (first_run + d) & 7;
            const uint32_t k = claim_tile(ctr + v * CTR_STRIDE);
            if (k < (uint32_t)run_cnt(v)) return run_start(v) + (int)k;
        }
        return -1;
    }
    // the claim for the tile after next, read at the next boundary; the
    // counter's offset is hidden from the compiler, whose rewrite of an atomic
    // on a uniform address would consume the result at once
    __device__ __forceinline__ void issue_pending() {
        int off = x * CTR_STRIDE;
        __asm__ volatile("" : "+v"(off));
        if (own_left) pend = claim_tile(ctr + off);
    }
    __device__ __forceinline__ void first(int &cur, int &nxt) {
        if (threadIdx.x == 0) {
            const int a = claim(x);
            const int b = a < 0 || ntiles <= (int)gridDim.x ? -1 : claim(x);
            own_left = b >= run_start(x) && b < run_start(x) + run_cnt(x);
            tq[0] = a;
            tq[1] = b;
            if (b >= 0) issue_pending();
        }
        lds_barrier();
        cur = tq[0];
        nxt = tq[1];
        lds_barrier();  // the slots are written again at the next boundary
    }
    // nxt holds the new current tile; returns the one after it (-1: none)
    __device__ __forceinline__ void advance(int &nxt) {
        if (threadIdx.x == 0) {
            int t = -1;
            if (own_left && pend < (uint32_t)run_cnt(x)) {
                t = run_start(x) + (int)pend;
            } else {
                own_left = false;
                t = claim((x + 1) & 7);  // the other runs, then the own run again
            }
            if (t >= 0) issue_pending();
            tq[0] = t;
        }
        lds_barrier();
        nxt = tq[0];
        lds_barrier();
    }
};

// Persistent form of the K loop for one A segment without a row gather (the
// many-row LM head, the fused gate/up projection, the plain bf16 product): the work-group runs tile
// after tile as `queue` hands them out and the DMA ring runs on across tile
// boundaries, so the first chunks of a tile are loaded while the previous
// tile finishes and its epilogue(tile, acc) runs. queue.first(cur, nxt)
// gives the first two tiles (-1: none) and queue.advance(nxt) the one after
// the new current tile; both are called by every thread with no load in
// flight and return the same values in every thread. tile_at(tile, m0, n0)
// gives a tile's origin.
// Layout of acc, LDS ring and ordering rule as in mainloop. At a tile
// boundary every wave waits for all of its outstanding vector memory
// operations (the epilogue's stores among them) and meets a barrier before
// the first fragment reads of the next tile, so the partial vmcnt waits
// inside a tile count LDS-DMA loads (and older operations) only. Every wave
// runs every tile, also one whose rows all lie past M (measured: skipping
// such tiles' MFMAs, the upper half of a last tile of at most BM / 2 rows,
// let their work-groups run ahead of the others of their XCD and raised the
// L2 misses of the 3904-row LM head by a third for under 1% of time).
// Requires K / 32 >= NS.
template <int BM, int NS, bool TRANS, int NW, class TileAt, class Queue, class Epi>
__device__ __forceinline__ void mainloop_persistent(const GemmParams &p, TileAt tile_at, Queue &queue, Epi epilogue,
                                                    unsigned char *ring) {
    using T = GTile<BM, NS, NW>;
    static_assert(BM % (T::LOADS * 16) == 0, "a wave's stage rows are all A rows or all B rows");
    static_assert(NS >= 3, "two chunks in flight beyond the one being read");
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int lr = lane & 31, lh = lane >> 5;
    const int wave_u = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kfull = __builtin_amdgcn_readfirstlane(p.K);
    const int nch = kfull / GBK;
    const bool a_side = wave_u * T::LOADS * 16 < BM;
    // the tile being computed and the one after it (-1: none)
    int cur, nxt;
    queue.first(cur, nxt);
    if (cur < 0) return;
    // DMA issue state: chunk of the next load within its tile, that tile's
    // wave-uniform base and the fixed per-lane byte offsets
    int iss_c = 0;
    const char *ibase = nullptr;
    uint32_t voff[T::LOADS];
    auto set_issue_tile = [&](int i) {
        int m0, n0;
        tile_at(i, m0, n0);
        m0 = __builtin_amdgcn_readfirstlane(m0);
        n0 = __builtin_amdgcn_readfirstlane(n0);
        ibase = a_side ? (const char *)e3_uniform_ptr((const uint16_t *)p.a[0] + (size_t)m0 * kfull)
                       : (const char *)e3_uniform_ptr((const uint16_t *)p.b + (size_t)n0 * kfull);
#pragma unroll
        for (int j = 0; j < T::LOADS; ++j) {
            const int row = (wave_u * T::LOADS + j) * 16 + (lane >> 2);
            const int sw = 8 * ((lane & 3) ^ gswz(row));
            if (a_side) voff[j] = (uint32_t)(((size_t)(min(m0 + row, p.M - 1) - m0) * kfull + sw) * 2);
            else voff[j] = (uint32_t)(((size_t)(min(n0 + row - BM, p.N - 1) - n0) * kfull + sw) * 2);
        }
    };
    // move the issue state on to the next tile when this one is done (once
    // per computed tile, during its last NS chunks); after the last tile a
    // virtual one re-reads the current tile's rows: its chunks land in slots
    // nobody reads and are drained at the tile boundary
    auto prep_issue = [&]() {
        if (iss_c == nch) {
            iss_c = 0;
            set_issue_tile(nxt >= 0 ? nxt : cur);
        }
    };
    auto dma = [&](int stage, int j) {
        const int blk = wave_u * T::LOADS + j;
        __builtin_amdgcn_global_load_lds((const void *)(ibase + (size_t)iss_c * (GBK * 2) + voff[j]),
                                         (lds_void_t *)(ring + stage * T::STAGE + blk * 1024), 16, 0, 0);
    };
    auto issue = [&](int stage) {
        prep_issue();
#pragma unroll
        for (int j = 0; j < T::LOADS; ++j) dma(stage, j);
        ++iss_c;
    };
    const int wm = wave / T::WN, wn = wave % T::WN;
    int aoff[T::MB][2], boff[T::NB][2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const int cl = 2 * s + lh;
#pragma unroll
        for (int mb = 0; mb < T::MB; ++mb) {
            const int row = wm * (BM / 2) + mb * 32 + lr;
            aoff[mb][s] = row * GROW + ((cl ^ gswz(row)) << 4);
        }
#pragma unroll
        for (int nb = 0; nb < T::NB; ++nb) {
            const int row = wn * T::CW + nb * 32 + lr;
            boff[nb][s] = BM * GROW + row * GROW + ((cl ^ gswz(row)) << 4);
        }
    }
    auto barrier = [&]() {
        __builtin_amdgcn_s_barrier();
        __asm__ volatile("" ::: "memory");
    };
    u32x4_t av0[T::MB], bv0[T::NB], av1[T::MB], bv1[T::NB];
    const uint32_t ring_lds = (uint32_t)(uintptr_t)(lds_void_t *)ring;
    constexpr int NMF = T::MB * T::NB;
    constexpr int NRD = T::MB + T::NB;
    static_assert(NRD <= NMF && T::LOADS <= NMF, "one read and one load per MFMA at most");
    auto rd = [&](int slotk, int s, int i, u32x4_t *av, u32x4_t *bv) {
        const uint32_t base = ring_lds + slotk * T::STAGE;
        if (i < T::MB) __asm__ volatile("ds_read_b128 %0, %1" : "=v"(av[i]) : "v"(base + aoff[i][s]));
        else __asm__ volatile("ds_read_b128 %0, %1" : "=v"(bv[i - T::MB]) : "v"(base + boff[i - T::MB][s]));
    };
    f32x16_t acc[T::MB][T::NB];
    auto mf = [&](int j, const u32x4_t *av, const u32x4_t *bv) {
        const int mb = j / T::NB, nb = j % T::NB;
        if constexpr (TRANS)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, bv[nb]),
                                                                  __builtin_bit_cast(bf16x8_t, av[mb]), acc[mb][nb],
                                                                  0, 0, 0);
        else
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, av[mb]),
                                                                  __builtin_bit_cast(bf16x8_t, bv[nb]), acc[mb][nb],
                                                                  0, 0, 0);
    };
    // A: MFMAs of (g, first half) with the reads of (g, second half) between them
    auto phase_a = [&](int g) {
        lgkm_wait<0, T::MB, T::NB>(av0, bv0);
        const int sl = g % T::NS;
#pragma unroll
        for (int j = 0; j < NMF; ++j) {
            mf(j, av0, bv0);
            __builtin_amdgcn_sched_barrier(0);
            if (j < NRD) {
                rd(sl, 1, j, av1, bv1);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        lgkm_wait<0, T::MB, T::NB>(av1, bv1);
    };
    // C: MFMAs of (g, second half) with the reads of (g + 1, first half) when
    // NEXT, and the loads of the stream's next chunk into g's slot
    auto phase_c = [&](int g, auto next_c) {
        constexpr bool NEXT = decltype(next_c)::value;
        const int sl = (g + 1) % T::NS, st = g % T::NS;
        prep_issue();
#pragma unroll
        for (int j = 0; j < NMF; ++j) {
            mf(j, av1, bv1);
            __builtin_amdgcn_sched_barrier(0);
            if (NEXT && j < NRD) {
                rd(sl, 0, j, av0, bv0);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (j >= NMF - T::LOADS) {
                dma(st, j - (NMF - T::LOADS));
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        ++iss_c;
    };
    set_issue_tile(cur);
#pragma unroll
    for (int st = 0; st < T::NS - 1; ++st) issue(st);
    wait_vmcnt<(T::NS - 2) * T::LOADS>();  // chunk 0
    barrier();
    issue(T::NS - 1);
#pragma unroll
    for (int i = 0; i < NRD; ++i) rd(0, 0, i, av0, bv0);
    // Every tile runs the same steps; with nch >= NS every chunk waits at
    // full depth and refills a slot.
    int g = 0;
    while (true) {
#pragma unroll
        for (int i = 0; i < T::MB; ++i)
#pragma unroll
            for (int jj = 0; jj < T::NB; ++jj)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][jj][r] = 0.f;
        __builtin_amdgcn_s_setprio(3);
        for (int c = 0; c + 1 < nch; ++c, ++g) {
            phase_a(g);
            wait_vmcnt<(T::NS - 2) * T::LOADS>();
            barrier();
            phase_c(g, std::true_type{});
        }
        // the tile's last chunk: the next tile's chunks keep loading
        phase_a(g);
        barrier();
        phase_c(g, std::false_type{});
        ++g;
        __builtin_amdgcn_s_setprio(0);
        epilogue(cur, acc);
        wait_vmcnt<0>();
        barrier();
        cur = nxt;
        if (cur < 0) break;
        queue.advance(nxt);
#pragma unroll
        for (int i = 0; i < NRD; ++i) rd(g % T::NS, 0, i, av0, bv0);
    }
}

}  // namespace e3g
