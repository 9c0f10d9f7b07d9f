// RMSNorm over the last dimension: y = x / sqrt(mean(x^2) + eps) * gamma.
// reading: the pages do not name a norm before the LM head; Llama applies an
// RMSNorm there, and without it the synthetic logits would be ~20x flatter.
//
// One 256-thread work-group per row; each thread owns 8 contiguous elements
// per pass (one 16-byte load for bf16, two for fp32). Sums run in fp32.
#include "common.h"

namespace {

template <bool BF16>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const void *__restrict__ x, const void *__restrict__ gamma,
                                                      int K, float eps, void *__restrict__ y) {
    __shared__ float red[4];
    const size_t base = (size_t)blockIdx.x * K;
    float ss = 0.f;
    for (int c = threadIdx.x * 8; c < K; c += 256 * 8) {
        float v[8];
        if (BF16) {
            const u32x4_t raw = *reinterpret_cast<const u32x4_t *>((const uint16_t *)x + base + c);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[2 * i] = __uint_as_float(raw[i] << 16);
                v[2 * i + 1] = __uint_as_float(raw[i] & 0xffff0000u);
            }
        } else {
            const f32x4_t a = *reinterpret_cast<const f32x4_t *>((const float *)x + base + c);
            const f32x4_t b = *reinterpret_cast<const f32x4_t *>((const float *)x + base + c + 4);
#pragma unroll
            for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) ss += v[i] * v[i];
    }
    const float total = e3_block_sum_256(ss, red);
    const float r = 1.0f / sqrtf(total / (float)K + eps);
    for (int c = threadIdx.x * 8; c < K; c += 256 * 8) {
        float v[8], g[8];
        if (BF16) {
            const u32x4_t raw = *reinterpret_cast<const u32x4_t *>((const uint16_t *)x + base + c);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[2 * i] = __uint_as_float(raw[i] << 16);
                v[2 * i + 1] = __uint_as_float(raw[i] & 0xffff0000u);
            }
            if (gamma) {
                const u32x4_t gr = *reinterpret_cast<const u32x4_t *>((const uint16_t *)gamma + c);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    g[2 * i] = __uint_as_float(gr[i] << 16);
                    g[2 * i + 1] = __uint_as_float(gr[i] & 0xffff0000u);
                }
            }
        } else {
            const f32x4_t a = *reinterpret_cast<const f32x4_t *>((const float *)x + base + c);
            const f32x4_t b = *reinterpret_cast<const f32x4_t *>((const float *)x + base + c + 4);
#pragma unroll
            for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
            if (gamma) {
                const f32x4_t ga = *reinterpret_cast<const f32x4_t *>((const float *)gamma + c);
                const f32x4_t gb = *reinterpret_cast<const f32x4_t *>((const float *)gamma + c + 4);
#pragma unroll
                for (int i = 0; i < 4; ++i) { g[i] = ga[i]; g[4 + i] = gb[i]; }
            }
        }
        if (!gamma) {
#pragma unroll
            for (int i = 0; i < 8; ++i) g[i] = 1.f;
        }
        if (BF16) {
            u32x4_t o;
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = e3_pack_bf16x2(v[2 * i] * r * g[2 * i], v[2 * i + 1] * r * g[2 * i + 1]);
            *reinterpret_cast<u32x4_t *>((uint16_t *)y + base + c) = o;
        } else {
            f32x4_t a, b;
#pragma unroll
            for (int i = 0; i < 4; ++i) { a[i] = v[i] * r * g[i]; b[i] = v[4 + i] * r * g[4 + i]; }
            *reinterpret_cast<f32x4_t *>((float *)y + base + c) = a;
            *reinterpret_cast<f32x4_t *>((float *)y + base + c + 4) = b;
        }
    }
}

}  // namespace

extern "C" int eagle3_rmsnorm(const void *x, const void *gamma, int M, int K, float eps, int dtype, void *y,
                              void *stream) {
    if (M < 0 || K < 1 || !(eps >= 0.f)) return EAGLE3_ERR_ARG;
    if (K % 8 != 0) return EAGLE3_ERR_UNSUPPORTED;
    if (dtype != EAGLE3_F32 && dtype != EAGLE3_BF16) return EAGLE3_ERR_UNSUPPORTED;
    if (M == 0) return EAGLE3_OK;
    if (!x || !y) return EAGLE3_ERR_ARG;
    if (!e3_aligned16(x) || !e3_aligned16(y) || (gamma && !e3_aligned16(gamma))) return EAGLE3_ERR_ARG;
    if (dtype == EAGLE3_BF16)
        rmsnorm_kernel<true><<<M, 256, 0, e3_stream(stream)>>>(x, gamma, K, eps, y);
    else
        rmsnorm_kernel<false><<<M, 256, 0, e3_stream(stream)>>>(x, gamma, K, eps, y);
    E3_LAUNCH_CHECK();
    return EAGLE3_OK;
}
