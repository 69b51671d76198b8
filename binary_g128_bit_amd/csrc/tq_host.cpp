// Host side of the library: error record, size queries, and the packer /
// unpacker for the slot layout declared in include/tq.h (ternary code
// c = t + 1 in LSB-first 2-bit slots, binary bit b = (t + 1)/2 LSB-first).
// The slots themselves follow the pages' storage of each trit in a 2-bit
// slot (aitrends.kr, "Ternary-Bonsai-27B-mlx-2bit", section "Technical
// features") and the 1-bit build's {-1, +1} set (thakicloud.github.io,
// "Bonsai 27B: ternary and 1-bit quantization", "How the compression works").
// The affine levels (TQ_AFFINE2) use the same slots with q in {0..3}.
// The five-trit storage (TQ_TERNARY5) is the native ternary packing the
// model card names as the next step: 26 bytes per 128-weight group, byte b
// the base-3 number of trits 5b..5b+4 (least significant digit first).
#include <cstdarg>
#include <cstring>
#include <string>

#include "tq_internal.h"

namespace tq {
namespace {
thread_local char g_msg[512] = "";
thread_local int64_t g_index = -1;

void vset(const char *fmt, va_list ap) { vsnprintf(g_msg, sizeof g_msg, fmt, ap); }
}  // namespace

int32_t fail(int32_t code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vset(fmt, ap);
    va_end(ap);
    g_index = -1;
    return code;
}

int32_t fail_at(int32_t code, int64_t index, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vset(fmt, ap);
    va_end(ap);
    g_index = index;
    return code;
}

void clear_error() {
    g_msg[0] = '\0';
    g_index = -1;
}

namespace {

// One packed ternary byte from four trits, or -1 if any trit is outside
// {-1,0,+1}.  Trit i of the quad goes to bits [2i, 2i+2) as i-th code t+1.
inline int tern_byte(const int8_t *q) {
    uint32_t v = 0;
    for (int i = 0; i < 4; ++i) {
        int c = int(q[i]) + 1;
        if (static_cast<unsigned>(c) > 2u) return -1 - i;
        v |= uint32_t(c) << (2 * i);
    }
    return int(v);
}

// One packed binary byte from eight signs, or -1-i for the first bad one.
inline int bin_byte(const int8_t *o) {
    uint32_t v = 0;
    for (int i = 0; i < 8; ++i) {
        if (o[i] == 1)
            v |= 1u << i;
        else if (o[i] != -1)
            return -1 - i;
    }
    return int(v);
}

// Base-3 digits of every byte value: digits[v][i] for i < 5; ok[v] when v < 3^5.
struct Base3Table {
    int8_t trit[256][5];
    bool below243[256];
    Base3Table() {
        for (int v = 0; v < 256; ++v) {
            int r = v;
            for (int i = 0; i < 5; ++i) {
                trit[v][i] = int8_t(r % 3 - 1);
                r /= 3;
            }
            below243[v] = r == 0;
        }
    }
};
const Base3Table &base3() {
    static const Base3Table table;
    return table;
}

// Five-trit bytes of one row: n trits per byte (5, or 3 for the last byte of
// a group) folded most significant first, c = t + 1, then zero padding.  A
// trit outside {-1,0,+1} returns TQ_ERR_VALUE with its index in the row.
int32_t pack_row5(const int8_t *t, int64_t K, uint8_t *out, int64_t *bad_k) {
    for (int64_t k = 0; k < K; ++k)
        if (static_cast<unsigned>(int(t[k]) + 1) > 2u) {
            *bad_k = k;
            return TQ_ERR_VALUE;
        }
    const int64_t G = K / kGroup, rb = ternary5_row_bytes(K);
    for (int64_t g = 0; g < G; ++g) {
        const int8_t *tg = t + g * kGroup;
        for (int b = 0; b < 26; ++b) {
            int v = 0;
            for (int i = (b < 25 ? 5 : 3) - 1; i >= 0; --i) v = 3 * v + int(tg[5 * b + i]) + 1;
            out[g * 26 + b] = uint8_t(v);
        }
    }
    for (int64_t i = G * 26; i < rb; ++i) out[i] = 0;
    return TQ_OK;
}

int32_t check_host(const void *a, const void *b, int64_t N, int64_t K, int32_t group,
                   int32_t variant) {
    if (!a || !b) return fail(TQ_ERR_NULL, "NULL pointer argument");
    return check_shape(1, N, K, group, variant);
}

}  // namespace
}  // namespace tq

extern "C" {

size_t tq_codes_bytes(int64_t N, int64_t K, int32_t variant) {
    if (N < 1 || K < tq::kGroup || K % tq::kGroup) return 0;
    if (variant == TQ_TERNARY || variant == TQ_AFFINE2) return size_t(N) * size_t(K / 4);
    if (variant == TQ_BINARY) return size_t(N) * size_t(K / 8);
    if (variant == TQ_TERNARY5) return size_t(N) * size_t(tq::ternary5_row_bytes(K));
    return 0;
}

size_t tq_scales_count(int64_t N, int64_t K, int32_t group) {
    if (N < 1 || group != tq::kGroup || K < group || K % group) return 0;
    return size_t(N) * size_t(K / group);
}

int32_t tq_pack(const int8_t *t, int64_t N, int64_t K, int32_t group, int32_t variant,
                uint8_t *codes) {
    tq::clear_error();
    if (int32_t rc = tq::check_host(t, codes, N, K, group, variant)) return rc;
    if (variant == TQ_TERNARY5) {
        const int64_t rb = tq::ternary5_row_bytes(K);
        for (int64_t n = 0; n < N; ++n) {
            int64_t k = -1;
            if (tq::pack_row5(t + n * K, K, codes + n * rb, &k) != TQ_OK) {
                const int64_t idx = n * K + k;
                return tq::fail_at(TQ_ERR_VALUE, idx, "t[%lld] = %d is outside {-1,0,+1}",
                                   (long long)idx, int(t[idx]));
            }
        }
        return TQ_OK;
    }
    if (variant == TQ_AFFINE2) {
        const int64_t nbytes = N * (K / 4);
        for (int64_t i = 0; i < nbytes; ++i) {
            uint32_t v = 0;
            for (int s = 0; s < 4; ++s) {
                const int q = t[i * 4 + s];
                if (static_cast<unsigned>(q) > 3u) {
                    const int64_t idx = i * 4 + s;
                    return tq::fail_at(TQ_ERR_VALUE, idx, "q[%lld] = %d is outside {0,1,2,3}",
                                       (long long)idx, q);
                }
                v |= uint32_t(q) << (2 * s);
            }
            codes[i] = uint8_t(v);
        }
        return TQ_OK;
    }
    const int64_t per = variant == TQ_TERNARY ? 4 : 8;
    const int64_t nbytes = N * (K / per);
    for (int64_t i = 0; i < nbytes; ++i) {
        const int8_t *src = t + i * per;
        int b = variant == TQ_TERNARY ? tq::tern_byte(src) : tq::bin_byte(src);
        if (b < 0) {
            int64_t idx = i * per + (-1 - b);
            return tq::fail_at(TQ_ERR_VALUE, idx, "t[%lld] = %d is outside the %s set",
                               (long long)idx, int(t[idx]),
                               variant == TQ_TERNARY ? "{-1,0,+1}" : "{-1,+1}");
        }
        codes[i] = uint8_t(b);
    }
    return TQ_OK;
}

int32_t tq_unpack(const uint8_t *codes, int64_t N, int64_t K, int32_t group, int32_t variant,
                  int8_t *t) {
    tq::clear_error();
    if (int32_t rc = tq::check_host(codes, t, N, K, group, variant)) return rc;
    if (variant == TQ_TERNARY5) {
        const tq::Base3Table &tb = tq::base3();
        const int64_t G = K / tq::kGroup, rb = tq::ternary5_row_bytes(K);
        for (int64_t n = 0; n < N; ++n)
            for (int64_t g = 0; g < G; ++g)
                for (int b = 0; b < 26; ++b) {
                    const uint8_t v = codes[n * rb + g * 26 + b];
                    // the last byte of a group holds three trits: digits 3, 4 must be 0
                    const bool ok = b < 25 ? tb.below243[v] : v < 27;
                    const int64_t idx = n * K + g * tq::kGroup + 5 * b;
                    if (!ok)
                        return tq::fail_at(TQ_ERR_CODE, idx,
                                           "invalid five-trit byte %u at weight %lld (row %lld, k %lld)",
                                           unsigned(v), (long long)idx, (long long)n,
                                           (long long)(idx - n * K));
                    const int nt = b < 25 ? 5 : 3;
                    for (int i = 0; i < nt; ++i) t[idx + i] = tb.trit[v][i];
                }
        return TQ_OK;
    }
    if (variant == TQ_AFFINE2) {
        const int64_t nbytes = N * (K / 4);
        for (int64_t i = 0; i < nbytes; ++i)
            for (int s = 0; s < 4; ++s) t[i * 4 + s] = int8_t((codes[i] >> (2 * s)) & 3u);
        return TQ_OK;
    }
    if (variant == TQ_TERNARY) {
        const int64_t nbytes = N * (K / 4);
        for (int64_t i = 0; i < nbytes; ++i) {
            uint32_t b = codes[i];
            // a slot holds 3 iff both of its bits are set
            uint32_t both = b & (b >> 1) & 0x55u;
            if (both) {
                int slot = __builtin_ctz(both) / 2;
                int64_t idx = i * 4 + slot;
                return tq::fail_at(TQ_ERR_CODE, idx, "invalid code 3 at weight %lld (row %lld, k %lld)",
                                   (long long)idx, (long long)(idx / K), (long long)(idx % K));
            }
            for (int s = 0; s < 4; ++s) t[i * 4 + s] = int8_t(int((b >> (2 * s)) & 3u) - 1);
        }
    } else {
        const int64_t nbytes = N * (K / 8);
        for (int64_t i = 0; i < nbytes; ++i) {
            uint32_t b = codes[i];
            for (int s = 0; s < 8; ++s) t[i * 8 + s] = ((b >> s) & 1u) ? int8_t(1) : int8_t(-1);
        }
    }
    return TQ_OK;
}

const char *tq_last_error(void) { return tq::g_msg; }

int64_t tq_last_error_index(void) { return tq::g_index; }

const char *tq_version(void) { return "tq 0.1.0 (gfx950)"; }

}  // extern "C"
