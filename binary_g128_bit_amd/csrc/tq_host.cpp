// Host side of the library: error record, size queries, and the packer /
// unpacker for the slot layout declared in include/tq.h (ternary code
// c = t + 1 in LSB-first 2-bit slots, binary bit b = (t + 1)/2 LSB-first).
// The slots themselves follow the pages' storage of each trit in a 2-bit
// slot (aitrends.kr, "Ternary-Bonsai-27B-mlx-2bit", section "Technical
// features") and the 1-bit build's {-1, +1} set (thakicloud.github.io,
// "Bonsai 27B: ternary and 1-bit quantization", "How the compression works").
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
    if (variant == TQ_TERNARY) return size_t(N) * size_t(K / 4);
    if (variant == TQ_BINARY) return size_t(N) * size_t(K / 8);
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
