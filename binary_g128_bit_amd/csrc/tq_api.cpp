// C ABI entry points for the device matmuls: argument validation (host only,
// before any HIP call) and dispatch to the kernels.  The operation is the
// pages' w_i = s_g * t_i product with one FP16 scale per 128 weights
// (thakicloud.github.io, "Bonsai 27B: ternary and 1-bit quantization",
// "How the compression works"), evaluated from the packed slots.
#include <hip/hip_runtime_api.h>

#include "tq_internal.h"

namespace tq {
int32_t gemv_enqueue(const uint8_t *codes, const uint16_t *scales, const uint16_t *x, float *y,
                     int64_t N, int64_t K, int32_t variant, hipStream_t stream);
int32_t gemm_enqueue(const uint8_t *codes, const uint16_t *scales, const uint16_t *X, float *Y,
                     int64_t M, int64_t N, int64_t K, int32_t variant, hipStream_t stream);
int32_t gemv5_enqueue(const uint8_t *codes, const uint16_t *scales, const uint16_t *x, float *y,
                      int64_t N, int64_t K, hipStream_t stream);
int32_t gemv_affine_enqueue(const uint8_t *codes, const uint16_t *scales, const uint16_t *biases,
                            const uint16_t *x, float *y, int64_t N, int64_t K, hipStream_t stream);
int32_t embed_enqueue(const uint8_t *codes, const uint16_t *scales, const int32_t *ids,
                      uint16_t *out, int64_t n_ids, int64_t N, int64_t K, int32_t variant,
                      hipStream_t stream);

namespace {
int32_t check_device_args(const void *codes, const void *scales, const void *x, const void *y,
                          int64_t M, int64_t N, int64_t K, int32_t group, int32_t variant) {
    if (!codes || !scales || !x || !y) return fail(TQ_ERR_NULL, "NULL pointer argument");
    if (int32_t rc = check_shape(M, N, K, group, variant)) return rc;
    if (!aligned(codes, 16)) return fail(TQ_ERR_ALIGN, "codes must be 16-byte aligned");
    if (!aligned(x, 16)) return fail(TQ_ERR_ALIGN, "activations must be 16-byte aligned");
    if (!aligned(scales, 2)) return fail(TQ_ERR_ALIGN, "scales must be 2-byte aligned");
    if (!aligned(y, 4)) return fail(TQ_ERR_ALIGN, "output must be 4-byte aligned");
    return TQ_OK;
}
}  // namespace
}  // namespace tq

extern "C" {

int32_t tq_gemv(const uint8_t *codes, const uint16_t *scales, const uint16_t *x, float *y,
                int64_t N, int64_t K, int32_t group, int32_t variant, void *stream) {
    tq::clear_error();
    if (int32_t rc = tq::check_device_args(codes, scales, x, y, 1, N, K, group, variant)) return rc;
    if (variant == TQ_AFFINE2)
        return tq::fail(TQ_ERR_VARIANT, "TQ_AFFINE2 weights need biases: use tq_gemv_affine");
    if (variant == TQ_TERNARY5)
        return tq::gemv5_enqueue(codes, scales, x, y, N, K, static_cast<hipStream_t>(stream));
    return tq::gemv_enqueue(codes, scales, x, y, N, K, variant,
                            static_cast<hipStream_t>(stream));
}

int32_t tq_gemm(const uint8_t *codes, const uint16_t *scales, const uint16_t *X, float *Y,
                int64_t M, int64_t N, int64_t K, int32_t group, int32_t variant, void *stream) {
    tq::clear_error();
    if (int32_t rc = tq::check_device_args(codes, scales, X, Y, M, N, K, group, variant)) return rc;
    if (variant == TQ_AFFINE2)
        return tq::fail(TQ_ERR_VARIANT, "TQ_AFFINE2 weights need biases: use tq_gemv_affine");
    if (variant == TQ_TERNARY5) {
        if (M != 1)
            return tq::fail(TQ_ERR_VARIANT, "TQ_TERNARY5 has a GEMV only (M = 1), got M=%lld",
                            (long long)M);
        return tq::gemv5_enqueue(codes, scales, X, Y, N, K, static_cast<hipStream_t>(stream));
    }
    if (M == 1)
        return tq::gemv_enqueue(codes, scales, X, Y, N, K, variant,
                                static_cast<hipStream_t>(stream));
    return tq::gemm_enqueue(codes, scales, X, Y, M, N, K, variant,
                            static_cast<hipStream_t>(stream));
}

int32_t tq_embed(const uint8_t *codes, const uint16_t *scales, const int32_t *ids, uint16_t *out,
                 int64_t n_ids, int64_t N, int64_t K, int32_t group, int32_t variant,
                 void *stream) {
    tq::clear_error();
    if (int32_t rc = tq::check_shape(1, N, K, group, variant)) return rc;
    if (variant == TQ_TERNARY5 || variant == TQ_AFFINE2)
        return tq::fail(TQ_ERR_VARIANT, "tq_embed takes TQ_TERNARY or TQ_BINARY tables");
    if (n_ids < 0 || n_ids > tq::kMaxN)
        return tq::fail(TQ_ERR_SHAPE, "n_ids=%lld outside [0, 2^31)", (long long)n_ids);
    if (n_ids == 0) return TQ_OK;
    if (!codes || !scales || !ids || !out) return tq::fail(TQ_ERR_NULL, "NULL pointer argument");
    if (!tq::aligned(codes, 4)) return tq::fail(TQ_ERR_ALIGN, "codes must be 4-byte aligned");
    if (!tq::aligned(scales, 2)) return tq::fail(TQ_ERR_ALIGN, "scales must be 2-byte aligned");
    if (!tq::aligned(ids, 4)) return tq::fail(TQ_ERR_ALIGN, "ids must be 4-byte aligned");
    if (!tq::aligned(out, 16)) return tq::fail(TQ_ERR_ALIGN, "output must be 16-byte aligned");
    return tq::embed_enqueue(codes, scales, ids, out, n_ids, N, K, variant,
                             static_cast<hipStream_t>(stream));
}

int32_t tq_gemv_affine(const uint8_t *codes, const uint16_t *scales, const uint16_t *biases,
                       const uint16_t *x, float *y, int64_t N, int64_t K, int32_t group,
                       void *stream) {
    tq::clear_error();
    if (!biases) return tq::fail(TQ_ERR_NULL, "NULL pointer argument");
    if (int32_t rc = tq::check_device_args(codes, scales, x, y, 1, N, K, group, TQ_AFFINE2))
        return rc;
    if (!tq::aligned(biases, 2)) return tq::fail(TQ_ERR_ALIGN, "biases must be 2-byte aligned");
    return tq::gemv_affine_enqueue(codes, scales, biases, x, y, N, K,
                                   static_cast<hipStream_t>(stream));
}

}  // extern "C"
