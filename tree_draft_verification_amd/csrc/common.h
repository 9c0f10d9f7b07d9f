// Internal helpers of libeagle3.so (gfx950 only). Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "eagle3.h"

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;

#define E3_LAUNCH_CHECK()                                          \
    do {                                                           \
        if (hipGetLastError() != hipSuccess) return EAGLE3_ERR_HIP; \
    } while (0)

// cache-policy operand of a global load: non-temporal (streamed once)
#define E3_CPOL_NT 2

static inline bool e3_aligned16(const void *p) { return (((uintptr_t)p) & 15u) == 0; }
static inline hipStream_t e3_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

// compute units of the current device (queried once per device)
static inline int e3_cu_count() {
    static int cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cache[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev] = n;
    }
    return cache[dev];
}

__device__ __forceinline__ float e3_bf16_to_f32(uint16_t u) { return __uint_as_float(((uint32_t)u) << 16); }

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t e3_f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)0x7fc0;
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2_t;

// two fp32 -> packed bf16 pair (lo in bits 0..15), round to nearest even
// (one v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint32_t e3_pack_bf16x2(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Split two fp32 values into bf16 hi + lo parts (x ~= hi + lo to about 16
// significant bits): hi = bf16(x), lo = bf16(x - hi); x - hi is exact in fp32.
__device__ __forceinline__ void e3_split_bf16x2(float a, float b, uint32_t &hi, uint32_t &lo) {
    hi = e3_pack_bf16x2(a, b);
    const float ha = __uint_as_float(hi << 16), hb = __uint_as_float(hi & 0xffff0000u);
    lo = e3_pack_bf16x2(a - ha, b - hb);
}

// Selection keys. Every selection orders (value, index) pairs by larger
// value first, then lower index. The pair is packed into one 64-bit key whose
// unsigned order is that order: the high word is the float's bits made
// order-preserving (sign bit flipped for positives, all bits for negatives;
// -0 is read as +0), the low word the complemented index. NaN maps to 0, the
// key of an empty slot, so it is never selected.
__device__ __forceinline__ uint64_t e3_key(float v, int i) {
    const uint32_t u = __float_as_uint(v == 0.f ? 0.f : v);
    const bool nan = v != v;
    const uint32_t hi = nan ? 0u : ((u & 0x80000000u) ? ~u : (u | 0x80000000u));
    const uint32_t lo = nan ? 0u : ~(uint32_t)i;
    return ((uint64_t)hi << 32) | lo;
}

// value and index of a key; an empty slot reads as (-inf, INT_MAX)
__device__ __forceinline__ float e3_key_val(uint64_t k) {
    const uint32_t hi = (uint32_t)(k >> 32);
    return k == 0 ? -INFINITY : __uint_as_float((hi & 0x80000000u) ? (hi & 0x7fffffffu) : ~hi);
}
__device__ __forceinline__ int e3_key_idx(uint64_t k) { return k == 0 ? 0x7fffffff : (int)~(uint32_t)k; }

template <int KK>
__device__ __forceinline__ void e3_kinit(uint64_t (&L)[KK]) {
#pragma unroll
    for (int s = 0; s < KK; ++s) L[s] = 0;
}

// insert key k into the descending list L (L[0] best), dropping the last
// entry; branch-free: every slot takes its upper neighbour, k or itself
template <int KK>
__device__ __forceinline__ void e3_kinsert(uint64_t (&L)[KK], uint64_t k) {
    bool g[KK];
#pragma unroll
    for (int s = 0; s < KK; ++s) g[s] = k > L[s];
#pragma unroll
    for (int s = KK - 1; s > 0; --s) L[s] = g[s - 1] ? L[s - 1] : (g[s] ? k : L[s]);
    L[0] = g[0] ? k : L[0];
}

// merge the list held by lane (lane ^ mask) into this lane's list
template <int KK>
__device__ __forceinline__ void e3_kmerge_xor(uint64_t (&L)[KK], int mask) {
    uint64_t o[KK];
#pragma unroll
    for (int s = 0; s < KK; ++s) o[s] = __shfl_xor(L[s], mask);
    // the other list is sorted too: once an entry cannot enter, none after it can
#pragma unroll
    for (int s = 0; s < KK; ++s) {
        if (!(o[s] > L[KK - 1])) break;
        e3_kinsert<KK>(L, o[s]);
    }
}

// log-sum-exp pair (max, sum of exp(x - max)) combination
__device__ __forceinline__ void e3_lse_combine(float &m, float &s, float m2, float s2) {
    float mn = fmaxf(m, m2);
    if (mn == -INFINITY) { m = mn; s = 0.f; return; }
    s = s * __expf(m - mn) + s2 * __expf(m2 - mn);
    m = mn;
}

// sum over a 256-thread work-group (red: 4 floats of LDS); every thread gets the total
__device__ __forceinline__ float e3_block_sum_256(float v, float *red) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (lane == 0) red[wave] = v;
    __syncthreads();
    const float s = red[0] + red[1] + red[2] + red[3];
    __syncthreads();
    return s;
}
