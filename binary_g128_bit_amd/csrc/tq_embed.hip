// Token-embedding rows from packed ternary / binary g128 weights, gfx950.
//
// out[i][k] = s[id_i][k / 128] * t[id_i][k] as FP16.  Every weight matrix of
// the model is stored ternary, the embedding table included (aitrends.kr,
// "Ternary-Bonsai-27B-mlx-2bit", section on what sets the build apart), and a
// weight is w = s_g * t with one FP16 scale per 128 weights (thakicloud.github.io,
// "Bonsai 27B: ternary and 1-bit quantization", "How the compression works").
// With t in {-1, 0, +1} the product is exact in FP16, so the row can feed the
// FP16 activation input of the matmul with no rounding.
//
// One thread per code dword (16 ternary or 32 binary weights).  A code pair is
// moved to bits [10,12) of each half (ternary c = t + 1, giving c * 2^-14) or
// bit 10 (binary b = (t + 1) / 2, giving b * 2^-14), mapped to t exactly with
// one packed FP16 fma (c * 2^-14 * 2^14 - 1, or b * 2^-14 * 2^15 - 1) and
// multiplied by the broadcast scale with one packed FP16 multiply, which keeps
// IEEE semantics for signed zeros and subnormal scales.  Lanes take
// consecutive dwords of a row, so a wave reads 256 contiguous code bytes and
// writes 2 or 4 KiB of contiguous output.
#include <hip/hip_runtime.h>

#include "tq_internal.h"

namespace tq {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t scaled_pair(uint32_t v, half2_t mul, half2_t s2) {
    const half2_t one = {(_Float16)1.0f, (_Float16)1.0f};
    half2_t t = __builtin_bit_cast(half2_t, v) * mul - one;
    return __builtin_bit_cast(uint32_t, t * s2);
}

// upr = code dwords per row; total = rows in this launch * upr (< 2^31).
template <int VARIANT>
__global__ __launch_bounds__(kThreads) void embed_kernel(const uint32_t *__restrict__ codes,
                                                         const uint16_t *__restrict__ scales,
                                                         const int32_t *__restrict__ ids,
                                                         uint16_t *__restrict__ out,
                                                         uint32_t total, uint32_t upr, int64_t N,
                                                         int64_t G) {
    constexpr int W = VARIANT == TQ_TERNARY ? 16 : 32;  // weights per code dword
    constexpr int NV = W / 8;                           // 16-byte stores per thread
    const uint32_t g = blockIdx.x * kThreads + threadIdx.x;
    if (g >= total) return;
    const uint32_t i = g / upr;
    const uint32_t u = g - i * upr;
    const int64_t id = ids[i];
    u32x4 *dst = reinterpret_cast<u32x4 *>(out + (int64_t)i * upr * W + (int64_t)u * W);
    if (id < 0 || id >= N) {
        const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int v = 0; v < NV; ++v) dst[v] = z;
        return;
    }
    const uint32_t d = codes[id * upr + u];
    const uint32_t sb = scales[id * G + (int64_t)u * W / 128];
    const half2_t s2 = __builtin_bit_cast(half2_t, sb | (sb << 16));
    uint32_t o[W / 2];
    if constexpr (VARIANT == TQ_TERNARY) {
        const half2_t mul = {(_Float16)16384.0f, (_Float16)16384.0f};
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            const uint32_t x = d >> (4 * p);
            o[p] = scaled_pair(((x & 3u) << 10) | ((x & 0xCu) << 24), mul, s2);
        }
    } else {
        const half2_t mul = {(_Float16)32768.0f, (_Float16)32768.0f};
#pragma unroll
        for (int p = 0; p < 16; ++p) {
            const uint32_t x = d >> (2 * p);
            o[p] = scaled_pair(((x & 1u) << 10) | ((x & 2u) << 25), mul, s2);
        }
    }
#pragma unroll
    for (int v = 0; v < NV; ++v) dst[v] = u32x4{o[4 * v], o[4 * v + 1], o[4 * v + 2], o[4 * v + 3]};
}

}  // namespace

int32_t embed_enqueue(const uint8_t *codes, const uint16_t *scales, const int32_t *ids,
                      uint16_t *out, int64_t n_ids, int64_t N, int64_t K, int32_t variant,
                      hipStream_t stream) {
    const int64_t W = variant == TQ_TERNARY ? 16 : 32;
    const int64_t upr = K / W;
    const int64_t G = K / kGroup;
    // rows per launch so that every flat thread index fits in 31 bits
    const int64_t chunk = ((int64_t(1) << 31) - kThreads) / upr;
    for (int64_t i0 = 0; i0 < n_ids; i0 += chunk) {
        const int64_t rows = n_ids - i0 < chunk ? n_ids - i0 : chunk;
        const uint32_t total = (uint32_t)(rows * upr);
        const dim3 grid((total + kThreads - 1) / kThreads);
        const uint32_t *c = reinterpret_cast<const uint32_t *>(codes);
        if (variant == TQ_TERNARY)
            hipLaunchKernelGGL((embed_kernel<TQ_TERNARY>), grid, dim3(kThreads), 0, stream, c,
                               scales, ids + i0, out + i0 * K, total, (uint32_t)upr, N, G);
        else
            hipLaunchKernelGGL((embed_kernel<TQ_BINARY>), grid, dim3(kThreads), 0, stream, c,
                               scales, ids + i0, out + i0 * K, total, (uint32_t)upr, N, G);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return fail(TQ_ERR_HIP, "embedding launch failed: %s", hipGetErrorString(e));
    }
    return TQ_OK;
}

}  // namespace tq
