// Small-batch GEMM over packed ternary / binary g128 weights (gfx950).
// Y[m][n] = sum_g s[n][g] * sum_j t[n][128g+j] * X[m][128g+j].
// First version: one GEMV launch per activation row.
#include <hip/hip_runtime.h>

#include "tq_internal.h"

namespace tq {
int32_t gemv_enqueue(const uint8_t *codes, const uint16_t *scales, const uint16_t *x, float *y,
                     int64_t N, int64_t K, int32_t variant, hipStream_t stream);

int32_t gemm_enqueue(const uint8_t *codes, const uint16_t *scales, const uint16_t *X, float *Y,
                     int64_t M, int64_t N, int64_t K, int32_t variant, hipStream_t stream) {
    for (int64_t m = 0; m < M; ++m)
        if (int32_t rc = gemv_enqueue(codes, scales, X + m * K, Y + m * N, N, K, variant, stream))
            return rc;
    return TQ_OK;
}
}  // namespace tq
