// Measurement aid, not part of the matmul: a plain streaming read of a device
// buffer, the ceiling a bandwidth-bound kernel of the same size is measured
// against.  Every 16-byte unit is loaded once (non-temporal, like the GEMV's
// code stream), folded into an XOR, and the result is stored only when it
// equals a value no real buffer produces in practice, so the loads cannot be
// dropped and the kernel writes nothing in practice.
#include <hip/hip_runtime.h>

#include "tq_internal.h"

namespace tq {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

int probe_cus() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        return 256;
    return n;
}

// Grid-stride loop with four 16-byte loads in flight per thread.
__global__ __launch_bounds__(512) void stream_read_kernel(const u32x4 *__restrict__ p, size_t n16,
                                                          uint32_t *__restrict__ sink) {
    u32x4 acc = {0u, 0u, 0u, 0u};
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4 a = __builtin_nontemporal_load(p + i);
        const u32x4 b = __builtin_nontemporal_load(p + i + stride);
        const u32x4 c = __builtin_nontemporal_load(p + i + 2 * stride);
        const u32x4 d = __builtin_nontemporal_load(p + i + 3 * stride);
        acc ^= a ^ b ^ c ^ d;
    }
    for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(p + i);
    const uint32_t v = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    if (v == 0x9E3779B9u) sink[0] = v;
}

}  // namespace
}  // namespace tq

extern "C" int32_t tq_stream_read(const void *buf, size_t bytes, uint32_t *sink, int32_t blocks_per_cu,
                                  void *stream) {
    tq::clear_error();
    if (!buf || !sink) return tq::fail(TQ_ERR_NULL, "NULL pointer argument");
    if (bytes == 0 || bytes % 16) return tq::fail(TQ_ERR_SHAPE, "bytes=%zu must be a positive multiple of 16", bytes);
    if (blocks_per_cu < 1 || blocks_per_cu > 8)
        return tq::fail(TQ_ERR_SHAPE, "blocks_per_cu=%d outside [1, 8]", blocks_per_cu);
    if (!tq::aligned(buf, 16) || !tq::aligned(sink, 4))
        return tq::fail(TQ_ERR_ALIGN, "buffer must be 16-byte aligned, sink 4-byte");
    hipLaunchKernelGGL(tq::stream_read_kernel, dim3(tq::probe_cus() * blocks_per_cu), dim3(512), 0,
                       static_cast<hipStream_t>(stream), static_cast<const tq::u32x4 *>(buf), bytes / 16,
                       sink);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return tq::fail(TQ_ERR_HIP, "stream read launch: %s", hipGetErrorString(e));
    return TQ_OK;
}
