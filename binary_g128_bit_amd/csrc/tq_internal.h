// Internal helpers shared by the library's translation units: the calling
// thread's error record and argument validation.  Not part of the C ABI.
#pragma once

#include <cstdint>
#include <cstdio>

#include "tq.h"

namespace tq {

// Record an error for tq_last_error(); returns `code` so callers can write
// `return fail(TQ_ERR_SHAPE, "...")`.
int32_t fail(int32_t code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int32_t fail_at(int32_t code, int64_t index, const char *fmt, ...)
    __attribute__((format(printf, 3, 4)));
void clear_error();

constexpr int32_t kGroup = 128;
constexpr int64_t kMaxK = 65536;
constexpr int64_t kMaxN = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxM = 65536;

// Shape / group / variant checks common to every entry point (after the
// caller has checked its pointers).
inline int32_t check_shape(int64_t M, int64_t N, int64_t K, int32_t group, int32_t variant) {
    if (M < 1 || M > kMaxM)
        return fail(TQ_ERR_SHAPE, "M=%lld outside [1, %lld]", (long long)M, (long long)kMaxM);
    if (N < 1 || N > kMaxN)
        return fail(TQ_ERR_SHAPE, "N=%lld outside [1, 2^31)", (long long)N);
    if (K < kGroup || K % kGroup != 0)
        return fail(TQ_ERR_SHAPE, "K=%lld must be a positive multiple of 128", (long long)K);
    if (K > kMaxK)
        return fail(TQ_ERR_SHAPE, "K=%lld above the supported maximum %lld", (long long)K,
                    (long long)kMaxK);
    if (group != kGroup)
        return fail(TQ_ERR_GROUP, "group=%d; only 128 is supported", group);
    if (variant != TQ_TERNARY && variant != TQ_BINARY && variant != TQ_TERNARY5 &&
        variant != TQ_AFFINE2)
        return fail(TQ_ERR_VARIANT,
                    "variant=%d is not TQ_TERNARY (0), TQ_BINARY (1), TQ_TERNARY5 (2) or "
                    "TQ_AFFINE2 (3)", variant);
    return TQ_OK;
}

// Bytes of one row of five-trit codes: 26 per group, padded to 16.
inline int64_t ternary5_row_bytes(int64_t K) { return (26 * (K / kGroup) + 15) / 16 * 16; }

inline bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

}  // namespace tq
