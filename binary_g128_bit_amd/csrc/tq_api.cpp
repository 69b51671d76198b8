// C ABI entry points for the device matmuls: argument validation (host only,
// before any HIP call) and dispatch to the kernels.  The operation is the
// pages' w_i = s_g * t_i product with one FP16 scale per 128 weights
// (thakicloud.github.io, "Bonsai 27B: ternary and 1-bit quantization",
// "How the compression works"), evaluated from the packed slots.
#include <hip/hip_runtime_api.h>

#include <cstdlib>
#include <cstring>

#include "tq_internal.h"

namespace tq {
int32_t gemv_enqueue(const uint8_t *codes, const uint16_t *scales, const uint16_t *x, float *y,
                     int64_t N, int64_t K, int32_t variant, hipStream_t stream);
int32_t gemm_enqueue(const uint8_t *codes, const uint16_t *scales, const uint16_t *X, float *Y,
                     int64_t M, int64_t N, int64_t K, int32_t variant, hipStream_t stream);
int32_t gemm_quad_enqueue(const uint8_t *codes, const uint16_t *scales, const uint16_t *X, float *Y,
                          int64_t M, int64_t N, int64_t K, int32_t variant, hipStream_t stream, bool *handled);
int32_t gemm_split_enqueue(const uint8_t *codes, const uint16_t *scales, const uint16_t *X, float *Y,
                           int64_t M, int64_t N, int64_t K, int32_t variant, float *ws, size_t ws_bytes,
                           hipStream_t stream, bool *handled);
size_t gemm_split_ws_bytes(int64_t M, int64_t N, int64_t K, int32_t variant);
int32_t gemm_mcol_enqueue(const uint8_t *codes, const uint16_t *scales, const uint16_t *X, float *Y,
                          int64_t M, int64_t N, int64_t K, int32_t variant, hipStream_t stream,
                          bool *handled);
int32_t gemv5_enqueue(const uint8_t *codes, const uint16_t *scales, const uint16_t *x, float *y,
                      int64_t N, int64_t K, hipStream_t stream);
int32_t gemv_affine_enqueue(const uint8_t *codes, const uint16_t *scales, const uint16_t *biases,
                            const uint16_t *x, float *y, int64_t N, int64_t K, hipStream_t stream);
int64_t attn_chunk(int64_t T, int64_t n_kv);
int32_t kv_append_enqueue(const uint16_t *k, const uint16_t *v, int64_t n_tok, int64_t pos, int64_t H,
                          int64_t TC, uint8_t *kc, uint16_t *ks, uint8_t *vc, uint16_t *vs,
                          hipStream_t stream);
int32_t attn_decode_enqueue(const uint16_t *q, const uint8_t *kc, const uint16_t *ks,
                            const uint8_t *vc, const uint16_t *vs, int64_t T, int64_t TC,
                            int64_t n_q, int64_t n_kv, float *out, float *ws, hipStream_t stream);
size_t attn_scratch_bytes();
int32_t attn_scratch(float **out);
int32_t embed_enqueue(const uint8_t *codes, const uint16_t *scales, const int32_t *ids,
                      uint16_t *out, int64_t n_ids, int64_t N, int64_t K, int32_t variant,
                      hipStream_t stream);

namespace {
// Kernel choice for small batches, read once per process from TQ_GEMM_QUAD:
// "off" never takes the 4-row MFMA kernel (tq_gemm_quad.hip), "all" sends it
// M = 1 as well, and the default sends it M >= 2 (it declines what it does
// not fit; M = 9 and up).  Measured (same box), ternary M = 2 against the
// two-row VALU kernel: 9.6 / 15.0 / 11.2 us against 11.4 / 16.4 / 11.7 on
// 17408 x 5120, 34816 x 5120 and 5120 x 17408, 87 against 100 us on the
// 248320-row head; M = 1 stays with the GEMV (8.2 against 9.8 us).
int quad_mode() {
    static const int mode = [] {
        const char *v = getenv("TQ_GEMM_QUAD");
        if (v && strcmp(v, "off") == 0) return 0;
        if (v && strcmp(v, "all") == 0) return 2;
        return 1;
    }();
    return mode;
}

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
constexpr int64_t kMaxTC = (int64_t(1) << 31) - 32;

int32_t check_kv(int64_t n_kv, int64_t t_cap) {
    if (n_kv < 1 || n_kv > 64) return fail(TQ_ERR_SHAPE, "n_kv=%lld outside [1, 64]", (long long)n_kv);
    if (t_cap < 32 || t_cap % 32 || t_cap > kMaxTC)
        return fail(TQ_ERR_SHAPE, "t_cap=%lld must be a positive multiple of 32 below 2^31",
                    (long long)t_cap);
    return TQ_OK;
}

size_t attn_ws_bytes(int64_t T, int64_t n_q, int64_t n_kv) {
    const int64_t chunk = attn_chunk(T, n_kv);
    return size_t((T + chunk - 1) / chunk) * size_t(n_q) * (256 + 2) * sizeof(float);
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
    return tq_gemm_ws(codes, scales, X, Y, M, N, K, group, variant, nullptr, 0, stream);
}

size_t tq_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t group, int32_t variant) {
    if (tq::check_shape(M, N, K, group, variant) != TQ_OK) {
        tq::clear_error();
        return 0;
    }
    return tq::gemm_split_ws_bytes(M, N, K, variant);
}

int32_t tq_gemm_ws(const uint8_t *codes, const uint16_t *scales, const uint16_t *X, float *Y,
                   int64_t M, int64_t N, int64_t K, int32_t group, int32_t variant, void *workspace,
                   size_t workspace_bytes, void *stream) {
    tq::clear_error();
    if (int32_t rc = tq::check_device_args(codes, scales, X, Y, M, N, K, group, variant)) return rc;
    if (workspace && !tq::aligned(workspace, 16))
        return tq::fail(TQ_ERR_ALIGN, "workspace must be 16-byte aligned");
    if (!workspace) workspace_bytes = 0;
    if (variant == TQ_AFFINE2)
        return tq::fail(TQ_ERR_VARIANT, "TQ_AFFINE2 weights need biases: use tq_gemv_affine");
    if (variant == TQ_TERNARY5) {
        if (M != 1)
            return tq::fail(TQ_ERR_VARIANT, "TQ_TERNARY5 has a GEMV only (M = 1), got M=%lld",
                            (long long)M);
        return tq::gemv5_enqueue(codes, scales, X, Y, N, K, static_cast<hipStream_t>(stream));
    }
    bool handled = false;
    if (tq::quad_mode() == 2 || (tq::quad_mode() == 1 && M >= 2)) {
        const int32_t rq = tq::gemm_quad_enqueue(codes, scales, X, Y, M, N, K, variant,
                                                 static_cast<hipStream_t>(stream), &handled);
        if (handled || rq != TQ_OK) return rq;
    }
    if (M >= 5 && M <= 64) {
        const int32_t rs = tq::gemm_split_enqueue(codes, scales, X, Y, M, N, K, variant,
                                                  static_cast<float *>(workspace), workspace_bytes,
                                                  static_cast<hipStream_t>(stream), &handled);
        if (handled || rs != TQ_OK) return rs;
    }
    if (M == 1)
        return tq::gemv_enqueue(codes, scales, X, Y, N, K, variant,
                                static_cast<hipStream_t>(stream));
    const int32_t rc = tq::gemm_mcol_enqueue(codes, scales, X, Y, M, N, K, variant,
                                             static_cast<hipStream_t>(stream), &handled);
    if (handled || rc != TQ_OK) return rc;
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

size_t tq_kv_bytes(int64_t n_kv, int64_t t_cap, int32_t part) {
    if (n_kv < 1 || n_kv > 64 || t_cap < 32 || t_cap % 32 || t_cap > tq::kMaxTC) return 0;
    switch (part) {
        case TQ_KV_K_CODES:
        case TQ_KV_V_CODES: return size_t(n_kv) * size_t(t_cap) * 128;
        case TQ_KV_K_SCALES:
        case TQ_KV_V_SCALES: return size_t(n_kv) * size_t(t_cap) * 16;
        default: return 0;
    }
}

int32_t tq_kv_append(const uint16_t *k, const uint16_t *v, int64_t n_tok, int64_t pos, int64_t n_kv,
                     int64_t t_cap, uint8_t *kc, uint16_t *ks, uint8_t *vc, uint16_t *vs,
                     void *stream) {
    tq::clear_error();
    if (int32_t rc = tq::check_kv(n_kv, t_cap)) return rc;
    if (n_tok < 0 || pos < 0 || pos + n_tok > t_cap)
        return tq::fail(TQ_ERR_SHAPE, "tokens [%lld, %lld) outside the capacity %lld", (long long)pos,
                        (long long)(pos + n_tok), (long long)t_cap);
    if (n_tok * n_kv > (int64_t(1) << 31) - 1)
        return tq::fail(TQ_ERR_SHAPE, "n_tok * n_kv above 2^31 - 1");
    if (n_tok == 0) return TQ_OK;
    if (!k || !v || !kc || !ks || !vc || !vs) return tq::fail(TQ_ERR_NULL, "NULL pointer argument");
    if (!tq::aligned(k, 2) || !tq::aligned(v, 2)) return tq::fail(TQ_ERR_ALIGN, "k and v must be 2-byte aligned");
    if (!tq::aligned(kc, 16) || !tq::aligned(ks, 16) || !tq::aligned(vc, 16) || !tq::aligned(vs, 16))
        return tq::fail(TQ_ERR_ALIGN, "cache arrays must be 16-byte aligned");
    return tq::kv_append_enqueue(k, v, n_tok, pos, n_kv, t_cap, kc, ks, vc, vs,
                                 static_cast<hipStream_t>(stream));
}

size_t tq_attn_workspace_bytes(int64_t T, int64_t n_q, int64_t n_kv) {
    if (T < 1 || T > tq::kMaxTC || n_kv < 1 || n_kv > 64 || n_q < n_kv || n_q % n_kv || n_q / n_kv > 16)
        return 0;
    return tq::attn_ws_bytes(T, n_q, n_kv);
}

}  // extern "C"

namespace tq {
namespace {
// Shape, pointer and alignment checks shared by the two attention entry points
// (the workspace pointer is checked by the one that takes it).
int32_t check_attn(const uint16_t *q, const uint8_t *kc, const uint16_t *ks, const uint8_t *vc,
                   const uint16_t *vs, int64_t T, int64_t n_q, int64_t n_kv, int64_t t_cap,
                   const float *out) {
    if (int32_t rc = check_kv(n_kv, t_cap)) return rc;
    if (n_q < n_kv || n_q % n_kv || n_q / n_kv > 16)
        return fail(TQ_ERR_SHAPE, "n_q=%lld must be a multiple of n_kv=%lld, at most 16 times it",
                    (long long)n_q, (long long)n_kv);
    if (T < 1 || T > t_cap)
        return fail(TQ_ERR_SHAPE, "T=%lld outside [1, t_cap=%lld]", (long long)T, (long long)t_cap);
    if (!q || !kc || !ks || !vc || !vs || !out) return fail(TQ_ERR_NULL, "NULL pointer argument");
    if (!aligned(q, 16) || !aligned(kc, 16) || !aligned(ks, 16) || !aligned(vc, 16) ||
        !aligned(vs, 16) || !aligned(out, 4))
        return fail(TQ_ERR_ALIGN, "q and cache must be 16-byte aligned, out 4-byte");
    return TQ_OK;
}
}  // namespace
}  // namespace tq

extern "C" {

int32_t tq_attn_decode(const uint16_t *q, const uint8_t *kc, const uint16_t *ks, const uint8_t *vc,
                       const uint16_t *vs, int64_t T, int64_t n_q, int64_t n_kv, int64_t t_cap,
                       float *out, void *workspace, size_t workspace_bytes, void *stream) {
    tq::clear_error();
    if (int32_t rc = tq::check_attn(q, kc, ks, vc, vs, T, n_q, n_kv, t_cap, out)) return rc;
    if (!workspace) return tq::fail(TQ_ERR_NULL, "NULL pointer argument");
    if (!tq::aligned(workspace, 16)) return tq::fail(TQ_ERR_ALIGN, "workspace must be 16-byte aligned");
    const size_t need = tq::attn_ws_bytes(T, n_q, n_kv);
    if (workspace_bytes < need)
        return tq::fail(TQ_ERR_SHAPE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
    return tq::attn_decode_enqueue(q, kc, ks, vc, vs, T, t_cap, n_q, n_kv, out,
                                   static_cast<float *>(workspace), static_cast<hipStream_t>(stream));
}

int32_t tq_attn_decode_noalloc(const uint16_t *q, const uint8_t *kc, const uint16_t *ks,
                               const uint8_t *vc, const uint16_t *vs, int64_t T, int64_t n_q,
                               int64_t n_kv, int64_t t_cap, float *out, void *stream) {
    tq::clear_error();
    if (int32_t rc = tq::check_attn(q, kc, ks, vc, vs, T, n_q, n_kv, t_cap, out)) return rc;
    const size_t need = tq::attn_ws_bytes(T, n_q, n_kv);
    if (need > tq::attn_scratch_bytes())
        return tq::fail(TQ_ERR_SHAPE,
                        "T=%lld n_q=%lld n_kv=%lld needs %zu bytes of scratch, above the %zu this "
                        "entry point holds; use tq_attn_decode with a workspace",
                        (long long)T, (long long)n_q, (long long)n_kv, need, tq::attn_scratch_bytes());
    float *ws = nullptr;
    if (int32_t rc = tq::attn_scratch(&ws)) return rc;
    return tq::attn_decode_enqueue(q, kc, ks, vc, vs, T, t_cap, n_q, n_kv, out, ws,
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
