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

// (value, index) order used by every selection: larger value first, then lower index.
__device__ __forceinline__ bool e3_better(float va, int ia, float vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

// insert (v, i) into the sorted list (L[0] best); drops the worst entry.
template <int KK>
__device__ __forceinline__ void e3_topk_insert(float (&lv)[KK], int (&li)[KK], float v, int i) {
#pragma unroll
    for (int s = 0; s < KK; ++s) {
        if (e3_better(v, i, lv[s], li[s])) {
            float tv = lv[s]; int ti = li[s];
            lv[s] = v; li[s] = i;
            v = tv; i = ti;
        }
    }
}

template <int KK>
__device__ __forceinline__ void e3_topk_init(float (&lv)[KK], int (&li)[KK]) {
#pragma unroll
    for (int s = 0; s < KK; ++s) { lv[s] = -INFINITY; li[s] = 0x7fffffff; }
}

// merge the list held by lane (lane ^ mask) into this lane's list
template <int KK>
__device__ __forceinline__ void e3_topk_merge_xor(float (&lv)[KK], int (&li)[KK], int mask) {
    float ov[KK]; int oi[KK];
#pragma unroll
    for (int s = 0; s < KK; ++s) { ov[s] = __shfl_xor(lv[s], mask); oi[s] = __shfl_xor(li[s], mask); }
    // the other list is sorted too: once an entry cannot enter, none after it can
#pragma unroll
    for (int s = 0; s < KK; ++s) {
        if (!e3_better(ov[s], oi[s], lv[KK - 1], li[KK - 1])) break;
        e3_topk_insert<KK>(lv, li, ov[s], oi[s]);
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
