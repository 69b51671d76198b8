// Small-batch GEMM over packed ternary / binary g128 weights on the gfx950
// matrix cores.
//
// Y[m][n] = sum_g s[n][g] * sum_{j<128} t[n][128g+j] * X[m][128g+j]
// (w_i = s_g * t_i, one FP16 scale per 128 weights along K: thakicloud.github.io,
// "Bonsai 27B: ternary and 1-bit quantization", "How the compression works";
// the packed slots are read directly and the scale is applied in the matmul:
// aitrends.kr, "Ternary-Bonsai-27B-mlx-2bit", "Technical features").  Every
// weight is shared by all M activation rows, so the decode is paid once per
// weight and the multiply-adds go to v_mfma_f32_16x16x32_f16 with 16
// activation rows as the A operand and 16 weight rows as the B operand.
//
// MFMA operand layout (16x16x32 f16): lane l supplies row l % 16 of A and
// column l % 16 of B, eight K values each, lane group q = l / 16 taking the
// K slice [8q, 8q + 8); lane l receives D[4q + i][l % 16], i < 4.  The K
// order inside an instruction is free as long as A and B agree, so lane group
// q works on weights [32q, 32q + 32) of every 128-weight group, in the order
// the decode produces them, and its activations are permuted to match.
//
// Decode (exact; one VALU op per two weights, plus shifts).  Each weight
// becomes an FP16 value that is linear in its code, with a fixed offset per
// slot position:
//   ternary E: code c in bits [10,12) of a half (exponent LSBs) is c * 2^-14;
//   ternary M: code c in bits [8,10) under exponent field 3 is
//              2^-12 + c * 2^-14 (offset 4 units of 2^-14);
//   binary:    bit b at position 11 is b * 2^-13; bit b at position p <= 10
//              under exponent field 12 - p is 2^(-3-p) + b * 2^-13 (offset
//              2^(10-p) units of 2^-13).
// The offsets and the shift t = c - 1 (ternary) or t = 2b - 1 (binary) are
// removed by starting each group's accumulation from C = -sum_k w_k x_k, with
// w_k = (1 + off_k) * 2^-14 (ternary) or (2 off_k + 1) * 2^-14 (binary), so
// that D = 2^-14 * sum_k t_k x_k.  C does not depend on the weight row: four
// MFMAs against a constant B operand give it per activation tile and group,
// shared by all weight tiles.  FP16 products are exact in FP32; each group's
// D is multiplied by its FP32 scale once, and totals by 2^14 at the end.
//
// Memory.  A wave owns NT tiles of 16 weight rows and a contiguous range of
// groups; the KW waves of a workgroup split K and add their partial sums in a
// fixed order through LDS, so results do not depend on timing.  Codes are read
// with 16-byte loads, eight lanes per 128-byte row segment (4 ternary or 8
// binary groups), written to the wave's LDS tile and read back in the MFMA
// layout: loading that layout directly reads 32 bytes per row per instruction,
// which streams from HBM at well under half the rate.  Two kernels share this
// structure: gemm_kernel loads each group's activations (small, L2-resident)
// straight into registers one group ahead and holds up to 64 activation rows
// per wave; gemm_stage_kernel (M <= 8) issues all loads of a stage in one
// batch and stages the activations in LDS (see its comment).  For wide
// batches gemm_tile_kernel instead decodes each weight once per workgroup into
// LDS as exact FP16 s * t and runs 32x32x16 MFMAs across all groups (see its
// comment).  Two-row batches take a VALU kernel in tq_gemv.hip.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "tq_internal.h"

namespace tq {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kPitch = 144;  // LDS bytes per staged code row: 128 + 16 of skew

// FP16 bits of -(v * 2^-14) for an integer 1 <= v < 2048 (exact).
constexpr uint32_t neg_units(int v) {
    int e = 0;
    while ((2 << e) <= v) ++e;
    return 0x8000u | (uint32_t)((e + 1) << 10) | (uint32_t)((v - (1 << e)) << (10 - e));
}
constexpr uint32_t pair(uint32_t h) { return h | (h << 16); }

template <int VARIANT>
struct Fmt;

// Ternary: 32 code bytes per row and group.  A lane's 32 weights are two code
// dwords; each gives 8 pairs (weight p in the low half, p + 8 in the high
// half) in the order E5 M4 E3 M2 E1 M0 E7 M6 (copies d, d << 4, d << 8, d >> 4).
template <>
struct Fmt<TQ_TERNARY> {
    static constexpr int kGroupBytes = 32, kStageGroups = 4, kHiOffset = 8;
    static constexpr int kOrder[8] = {5, 4, 3, 2, 1, 0, 7, 6};
    // weight index (of the lane's 32) in the low half of pair q
    static constexpr int lo(int q) { return 16 * (q / 8) + kOrder[q % 8]; }
    // correction weight of pair q: E slots (1 + 0), M slots (1 + 4)
    static constexpr int wt(int q) { return q % 2 ? 5 : 1; }
    static constexpr uint32_t corr(int q) { return pair(neg_units(wt(q))); }
};

// Binary: 16 code bytes per row and group.  A lane's 32 weights are one code
// dword giving 16 pairs (bit p low, bit p + 16 high): copy d yields p = 11..6,
// copy d << 6 yields p = 5..0 and copy d >> 4 yields p = 15..12 at slots 11..6.
template <>
struct Fmt<TQ_BINARY> {
    static constexpr int kGroupBytes = 16, kStageGroups = 8, kHiOffset = 16;
    static constexpr int kSlot[16] = {11, 10, 9, 8, 7, 6, 11, 10, 9, 8, 7, 6, 11, 10, 9, 8};
    static constexpr int kLo[16] = {11, 10, 9, 8, 7, 6, 5, 4, 3, 2, 1, 0, 15, 14, 13, 12};
    static constexpr int lo(int q) { return kLo[q]; }
    // slot offset in units of 2^-13: 0 at bit 11, 2^(10 - p) at bit p <= 10
    static constexpr int off(int s) { return s == 11 ? 0 : 1 << (10 - s); }
    static constexpr int wt(int q) { return 2 * off(kSlot[q]) + 1; }
    static constexpr uint32_t corr(int q) { return pair(neg_units(wt(q))); }
};

// Constants of v_and_or_b32 stay in VGPRs (gfx9 VOP3 takes no literal and
// reads at most one SGPR).
__device__ __forceinline__ uint32_t vreg(uint32_t v) {
    asm volatile("" : "+v"(v));
    return v;
}

template <int VARIANT>
struct Decoder;

template <>
struct Decoder<TQ_TERNARY> {
    uint32_t mm, e3;
    __device__ __forceinline__ Decoder() : mm(vreg(0x03000300u)), e3(vreg(0x0C000C00u)) {}
    // d[0]: codes of weights 0..15 of the lane's 32, d[1]: weights 16..31
    __device__ __forceinline__ void operator()(const uint32_t *d, uint32_t (&w)[16]) const {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t c[4] = {d[h], d[h] << 4, d[h] << 8, d[h] >> 4};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                w[8 * h + 2 * i] = c[i] & 0x0C000C00u;    // E: c * 2^-14
                w[8 * h + 2 * i + 1] = (c[i] & mm) | e3;  // M: 2^-12 + c * 2^-14
            }
        }
    }
};

template <>
struct Decoder<TQ_BINARY> {
    uint32_t e2, e3, e4, e5, e6;
    __device__ __forceinline__ Decoder()
        : e2(vreg(0x08000800u)), e3(vreg(0x0C000C00u)), e4(vreg(0x10001000u)),
          e5(vreg(0x14001400u)), e6(vreg(0x18001800u)) {}
    // slots 11..11-n+1 of copy c into w[0..n)
    template <int n>
    __device__ __forceinline__ void slots(uint32_t c, uint32_t *w) const {
        w[0] = c & 0x08000800u;                   // bit 11: b * 2^-13
        w[1] = (c & 0x04000400u) | e2;            // bit 10: 2^-13 + b * 2^-13
        w[2] = (c & 0x02000200u) | e3;            // bit 9:  2^-12 + b * 2^-13
        w[3] = (c & 0x01000100u) | e4;            // bit 8:  2^-11 + b * 2^-13
        if (n > 4) w[4] = (c & 0x00800080u) | e5; // bit 7:  2^-10 + b * 2^-13
        if (n > 5) w[5] = (c & 0x00400040u) | e6; // bit 6:  2^-9  + b * 2^-13
    }
    __device__ __forceinline__ void operator()(const uint32_t *d, uint32_t (&w)[16]) const {
        slots<6>(d[0], w);
        slots<6>(d[0] << 6, w + 6);
        slots<4>(d[0] >> 4, w + 12);
    }
};

__device__ __forceinline__ half8 as_half8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    const u32x4 v = {a, b, c, d};
    return __builtin_bit_cast(half8, v);
}

__device__ __forceinline__ f32x4 mfma(half8 a, half8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// FP16 pair of -wt(q), the integer that turns pair q's slot value v into t:
// t = v * 2^14 - wt(q) (ternary wt = offset + 1: 1 or 5; binary 2 offset + 1).
// neg_units(w) is -w * 2^-14; 14 more in the exponent field makes it -w.
template <int VARIANT>
constexpr uint32_t tile_bias(int q) {
    return pair(neg_units(Fmt<VARIANT>::wt(q)) + (14u << 10));
}
static_assert(pair(neg_units(1) + (14u << 10)) == 0xBC00BC00u, "-1 in FP16");
static_assert(pair(neg_units(5) + (14u << 10)) == 0xC500C500u, "-5 in FP16");
static_assert(pair(neg_units(33) + (14u << 10)) == 0xD020D020u, "-33 in FP16");

// The decode's 16 slot pairs as exact FP16 s * t (t is ternary or +-1, so
// s * t is an FP16 value): t = v * 2^14 - wt(q), then t * s, each exact.
template <int VARIANT>
__device__ __forceinline__ void exact_st(uint32_t (&w)[16], uint32_t s2, uint32_t two14) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int qq = 0; qq < 16; ++qq) {
        const h2 t = __builtin_bit_cast(h2, w[qq]) * __builtin_bit_cast(h2, two14) +
                     __builtin_bit_cast(h2, tile_bias<VARIANT>(qq));
        w[qq] = __builtin_bit_cast(uint32_t, t * __builtin_bit_cast(h2, s2));
    }
}

// Pair q of the lane's 32 activations: low half = activation lo(q), high
// half = activation lo(q) + kHiOffset (xw holds them as 16 dwords).
template <int VARIANT>
__device__ __forceinline__ void permute_x(const u32x4 (&xr)[4], uint32_t (&xa)[16]) {
    using F = Fmt<VARIANT>;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int lo = F::lo(q), hi = lo + F::kHiOffset;
        const uint32_t wlo = xr[lo / 8][(lo / 2) % 4], whi = xr[hi / 8][(hi / 2) % 4];
        // v_perm_b32: bytes 0-3 select from the second source, 4-7 from the first
        const uint32_t sel = (lo % 2 ? 0x0302u : 0x0100u) | (hi % 2 ? 0x07060000u : 0x05040000u);
        xa[q] = __builtin_amdgcn_perm(whi, wlo, sel);
    }
}

template <int NT, int MT, int KW>
constexpr size_t gemm_lds_bytes() {
    constexpr size_t stage = (size_t)KW * 16 * NT * kPitch;
    constexpr size_t red = (size_t)KW * NT * MT * 256 * sizeof(float);
    return stage > red ? stage : red;
}

template <int VARIANT, int NT, int MT, int KW>
__global__ __launch_bounds__(64 * KW) void gemm_kernel(const uint8_t *__restrict__ codes,
                                                       const uint16_t *__restrict__ scales,
                                                       const uint16_t *__restrict__ X,
                                                       float *__restrict__ Y, int M, int N, int K) {
    using F = Fmt<VARIANT>;
    constexpr int SG = F::kStageGroups, GB = F::kGroupBytes;
    constexpr int ROWS = 16 * NT, LOADS = ROWS / 8, SPL = SG / 4;
    __shared__ __attribute__((aligned(16))) uint8_t smem[gemm_lds_bytes<NT, MT, KW>()];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l16 = lane & 15, q = lane >> 4;
    const int G = K >> 7;
    const size_t RB = (size_t)G * GB;  // code bytes per weight row
    const int n0 = blockIdx.x * ROWS, m0 = blockIdx.y * 16 * MT;
    const int g_begin = (int)((int64_t)wave * G / KW), g_end = (int)((int64_t)(wave + 1) * G / KW);
    uint8_t *lds = smem + wave * ROWS * kPitch;

    f32x4 acc[NT][MT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int u = 0; u < MT; ++u) acc[t][u] = (f32x4){0.f, 0.f, 0.f, 0.f};

    if (g_begin < g_end) {
        const Decoder<VARIANT> dec;
        const half8 cb[4] = {as_half8(F::corr(0), F::corr(1), F::corr(2), F::corr(3)),
                             as_half8(F::corr(4), F::corr(5), F::corr(6), F::corr(7)),
                             as_half8(F::corr(8), F::corr(9), F::corr(10), F::corr(11)),
                             as_half8(F::corr(12), F::corr(13), F::corr(14), F::corr(15))};
        // staging loads: load i covers rows 8i .. 8i + 7 of the wave's tile
        const uint8_t *cp[LOADS];
#pragma unroll
        for (int i = 0; i < LOADS; ++i)
            cp[i] = codes + (size_t)min(n0 + 8 * i + (lane >> 3), N - 1) * RB;
        const int col = 16 * (lane & 7);
        const uint16_t *xp[MT];
#pragma unroll
        for (int u = 0; u < MT; ++u)
            xp[u] = X + (size_t)min(m0 + 16 * u + l16, M - 1) * K + 32 * q;
        const uint16_t *sp[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) sp[t] = scales + (size_t)min(n0 + 16 * t + l16, N - 1) * G;
        const int last = g_begin + (g_end - 1 - g_begin) / SG * SG;  // first group of the last stage

        u32x4 cr[LOADS];
        float sc[NT][SPL];
        u32x4 xr[MT][4];
        // stage gs: code bytes of groups [gs, gs + SG) (clamped into the wave's
        // range) and the scales of group gs + q + 4k held by lane group q
        auto load_stage = [&](int gs) __attribute__((always_inline)) {
            const int c = min(col, min(SG, g_end - gs) * GB - 16);
#pragma unroll
            for (int i = 0; i < LOADS; ++i)
                cr[i] = __builtin_nontemporal_load(
                    reinterpret_cast<const u32x4 *>(cp[i] + (size_t)gs * GB + c));
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int k = 0; k < SPL; ++k)
                    sc[t][k] = (float)__builtin_bit_cast(_Float16, sp[t][min(gs + q + 4 * k, g_end - 1)]);
        };
        auto load_x = [&](int g) __attribute__((always_inline)) {
#pragma unroll
            for (int u = 0; u < MT; ++u)
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    xr[u][k] = *reinterpret_cast<const u32x4 *>(xp[u] + (size_t)g * 128 + 8 * k);
        };

        load_stage(g_begin);
        load_x(g_begin);
        for (int gs = g_begin;; gs += SG) {
#pragma unroll
            for (int i = 0; i < LOADS; ++i)
                *reinterpret_cast<u32x4 *>(lds + (8 * i + (lane >> 3)) * kPitch + col) = cr[i];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            float scur[NT][SPL];
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int k = 0; k < SPL; ++k) scur[t][k] = sc[t][k];
            load_stage(min(gs + SG, last));
            const int ng = min(SG, g_end - gs);
#pragma unroll
            for (int gl = 0; gl < SG; ++gl) {
                u32x4 xc[MT][4];
#pragma unroll
                for (int u = 0; u < MT; ++u)
#pragma unroll
                    for (int k = 0; k < 4; ++k) xc[u][k] = xr[u][k];
                load_x(min(gs + gl + 1, g_end - 1));
                if (gl < ng) {
                    uint32_t xa[MT][16];
                    f32x4 cor[MT];
#pragma unroll
                    for (int u = 0; u < MT; ++u) {
                        permute_x<VARIANT>(xc[u], xa[u]);
                        cor[u] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            cor[u] = mfma(as_half8(xa[u][4 * j], xa[u][4 * j + 1], xa[u][4 * j + 2],
                                                   xa[u][4 * j + 3]),
                                          cb[j], cor[u]);
                    }
#pragma unroll
                    for (int t = 0; t < NT; ++t) {
                        const uint8_t *row = lds + (16 * t + l16) * kPitch + gl * GB;
                        uint32_t d[2];
                        if (VARIANT == TQ_TERNARY) {
                            const u32x2 v = *reinterpret_cast<const u32x2 *>(row + 8 * q);
                            d[0] = v.x;
                            d[1] = v.y;
                        } else {
                            d[0] = *reinterpret_cast<const uint32_t *>(row + 4 * q);
                            d[1] = 0;
                        }
                        uint32_t w[16];
                        dec(d, w);
                        const float s = __shfl(scur[t][gl / 4], l16 + 16 * (gl % 4));
#pragma unroll
                        for (int u = 0; u < MT; ++u) {
                            f32x4 D = cor[u];
#pragma unroll
                            for (int j = 0; j < 4; ++j)
                                D = mfma(as_half8(xa[u][4 * j], xa[u][4 * j + 1], xa[u][4 * j + 2],
                                                  xa[u][4 * j + 3]),
                                         as_half8(w[4 * j], w[4 * j + 1], w[4 * j + 2], w[4 * j + 3]),
                                         D);
#pragma unroll
                            for (int i = 0; i < 4; ++i) acc[t][u][i] = __builtin_fmaf(s, D[i], acc[t][u][i]);
                        }
                    }
                }
            }
            if (gs >= last) break;
        }
    }

    // fixed-order sum of the KW partials; the staging area is reused
    __syncthreads();
    float *red = reinterpret_cast<float *>(smem);
    constexpr int E = NT * MT * 256;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int u = 0; u < MT; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) red[wave * E + ((t * MT + u) * 4 + i) * 64 + lane] = acc[t][u][i];
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 64 * KW) {
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < KW; ++w) s += red[w * E + e];
        const int le = e & 63, i = (e >> 6) & 3, tu = e >> 8;
        const int m = m0 + 16 * (tu % MT) + 4 * (le >> 4) + i;
        const int n = n0 + 16 * (tu / MT) + (le & 15);
        if (m < M && n < N) Y[(size_t)m * N + n] = s * 16384.0f;
    }
}

// Stage-pipelined variant for up to 16 activation rows.  A stage is SG groups
// of K: the codes of the wave's 16*NT weight rows (128- or 64-byte row
// segments), the activations of MR rows over the same groups and their
// scales.  Loads are issued in a fixed order, one batch per stage: the next
// stage's activations, then the codes and scales PC stages ahead (a ring of
// PC register sets).  Loads complete in order, so waiting for a stage's
// activations only forces code batches issued at least two stages earlier,
// and every wave keeps about PC stages of codes in flight.  At the start of
// a stage the wave writes its codes (transposed) and activations (permuted
// into MFMA A-operand order) into its own LDS area and computes the stage
// from there.  MR = 4 stages four activation rows (M <= 4): lanes of rows
// 4..15 read row 3, whose duplicate outputs are never stored.
template <int VARIANT, int MR>
struct StageFmt {
    using F = Fmt<VARIANT>;
    // 128-byte code rows per stage where the activation tile stays small
    static constexpr int SG = (VARIANT == TQ_BINARY && MR <= 4) ? 8 : 4;
    static constexpr int ROW_BYTES = SG * F::kGroupBytes;      // 128 or 64
    static constexpr int LPRW = ROW_BYTES / 16;                // lanes per code row
    static constexpr int XITEMS = MR * SG * 4;                 // 32-activation items per stage
    static constexpr int XPL = (XITEMS + 63) / 64;             // items per lane
    static constexpr int XBYTES = SG * 16 * MR * 16;           // LDS activation tile
};

template <int VARIANT, int NT, int MR, int KW>
constexpr size_t stage_lds_bytes() {
    using SF = StageFmt<VARIANT, MR>;
    constexpr size_t per_wave = (size_t)16 * NT * kPitch + SF::XBYTES;
    constexpr size_t red = (size_t)KW * NT * 256 * sizeof(float);
    return KW * per_wave > red ? KW * per_wave : red;
}

template <int VARIANT, int NT, int MR, int KW, int PC>
__global__ __launch_bounds__(64 * KW) void gemm_stage_kernel(const uint8_t *__restrict__ codes,
                                                             const uint16_t *__restrict__ scales,
                                                             const uint16_t *__restrict__ X,
                                                             float *__restrict__ Y, int M, int N,
                                                             int K) {
    using F = Fmt<VARIANT>;
    using SF = StageFmt<VARIANT, MR>;
    constexpr int SG = SF::SG, GB = F::kGroupBytes, SPL = SG / 4;
    constexpr int ROWS = 16 * NT, RPI = 64 / SF::LPRW, LOADS = ROWS / RPI;
    constexpr int PER_WAVE = ROWS * kPitch + SF::XBYTES;
    __shared__ __attribute__((aligned(16))) uint8_t smem[stage_lds_bytes<VARIANT, NT, MR, KW>()];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l16 = lane & 15, q = lane >> 4;
    const int G = K >> 7;
    const size_t RB = (size_t)G * GB;
    const int n0 = blockIdx.x * ROWS, m0 = blockIdx.y * 16;
    const int g_begin = (int)((int64_t)wave * G / KW), g_end = (int)((int64_t)(wave + 1) * G / KW);
    uint8_t *lds_c = smem + wave * PER_WAVE;
    u32x4 *lds_x = reinterpret_cast<u32x4 *>(lds_c + ROWS * kPitch);

    f32x4 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = (f32x4){0.f, 0.f, 0.f, 0.f};

    if (g_begin < g_end) {
        const Decoder<VARIANT> dec;
        const half8 cb[4] = {as_half8(F::corr(0), F::corr(1), F::corr(2), F::corr(3)),
                             as_half8(F::corr(4), F::corr(5), F::corr(6), F::corr(7)),
                             as_half8(F::corr(8), F::corr(9), F::corr(10), F::corr(11)),
                             as_half8(F::corr(12), F::corr(13), F::corr(14), F::corr(15))};
        const uint8_t *cp[LOADS];
#pragma unroll
        for (int i = 0; i < LOADS; ++i)
            cp[i] = codes + (size_t)min(n0 + RPI * i + lane / SF::LPRW, N - 1) * RB;
        const int col = 16 * (lane % SF::LPRW);
        const uint16_t *sp[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) sp[t] = scales + (size_t)min(n0 + 16 * t + l16, N - 1) * G;
        // activation items of this lane: item = lane + 64 k -> (row, group, quarter)
        const uint16_t *xrow[SF::XPL];
        int xg[SF::XPL], xq[SF::XPL], xm[SF::XPL];
#pragma unroll
        for (int k = 0; k < SF::XPL; ++k) {
            const int it = min(lane + 64 * k, SF::XITEMS - 1);
            xq[k] = it & 3;
            xg[k] = (it >> 2) % SG;
            xm[k] = it / (4 * SG);
            xrow[k] = X + (size_t)min(m0 + xm[k], M - 1) * K + 32 * xq[k];
        }
        const int last = g_begin + (g_end - 1 - g_begin) / SG * SG;
        // lane (row l16, quarter q) reads activation row min(l16, MR - 1)
        const int xr_m = min(l16, MR - 1);

        u32x4 cr[PC][LOADS];
        float sc[PC][NT][SPL];
        u32x4 xv[SF::XPL][4];
        // codes and scales of the stage starting at group gs into ring set p
        auto load_codes = [&](int p, int gs) __attribute__((always_inline)) {
            gs = min(gs, last);
            const int c = min(col, min(SG, g_end - gs) * GB - 16);
#pragma unroll
            for (int i = 0; i < LOADS; ++i)
                cr[p][i] = __builtin_nontemporal_load(
                    reinterpret_cast<const u32x4 *>(cp[i] + (size_t)gs * GB + c));
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int k = 0; k < SPL; ++k)
                    sc[p][t][k] =
                        (float)__builtin_bit_cast(_Float16, sp[t][min(gs + q + 4 * k, g_end - 1)]);
        };
        auto load_x = [&](int gs) __attribute__((always_inline)) {
            gs = min(gs, last);
#pragma unroll
            for (int k = 0; k < SF::XPL; ++k) {
                const uint16_t *src = xrow[k] + (size_t)min(gs + xg[k], g_end - 1) * 128;
#pragma unroll
                for (int v = 0; v < 4; ++v) xv[k][v] = *reinterpret_cast<const u32x4 *>(src + 8 * v);
            }
        };
        // a full stage is computed without branches so that the independent
        // MFMA chains of its groups and tiles can be interleaved
        auto compute = [&](auto full, const float (&scur)[NT][SPL], int gs) __attribute__((always_inline)) {
            const int ng = min(SG, g_end - gs);
#pragma unroll
            for (int gl = 0; gl < SG; ++gl) {
                if (decltype(full)::value || gl < ng) {
                    u32x4 xa4[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) xa4[j] = lds_x[((gl * 4 + j) * 4 + q) * MR + xr_m];
                    f32x4 cor = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        cor = mfma(as_half8(xa4[j][0], xa4[j][1], xa4[j][2], xa4[j][3]), cb[j], cor);
#pragma unroll
                    for (int t = 0; t < NT; ++t) {
                        const uint8_t *row = lds_c + (16 * t + l16) * kPitch + gl * GB;
                        uint32_t d[2];
                        if (VARIANT == TQ_TERNARY) {
                            const u32x2 v = *reinterpret_cast<const u32x2 *>(row + 8 * q);
                            d[0] = v.x;
                            d[1] = v.y;
                        } else {
                            d[0] = *reinterpret_cast<const uint32_t *>(row + 4 * q);
                            d[1] = 0;
                        }
                        uint32_t w[16];
                        dec(d, w);
                        const float s = __shfl(scur[t][gl / 4], l16 + 16 * (gl % 4));
                        f32x4 D = cor;
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            D = mfma(as_half8(xa4[j][0], xa4[j][1], xa4[j][2], xa4[j][3]),
                                     as_half8(w[4 * j], w[4 * j + 1], w[4 * j + 2], w[4 * j + 3]), D);
#pragma unroll
                        for (int i = 0; i < 4; ++i) acc[t][i] = __builtin_fmaf(s, D[i], acc[t][i]);
                    }
                }
            }
        };

        // prologue: codes of stage 0, activations of stage 0, codes of stages 1..PC-1
        load_codes(0, g_begin);
        load_x(g_begin);
#pragma unroll
        for (int p = 1; p < PC; ++p) load_codes(p, g_begin + p * SG);
        for (int gs = g_begin;;) {
#pragma unroll
            for (int p = 0; p < PC; ++p) {
#pragma unroll
                for (int i = 0; i < LOADS; ++i)
                    *reinterpret_cast<u32x4 *>(lds_c + (RPI * i + lane / SF::LPRW) * kPitch + col) =
                        cr[p][i];
#pragma unroll
                for (int k = 0; k < SF::XPL; ++k) {
                    if (SF::XITEMS % 64 != 0 && lane + 64 * k >= SF::XITEMS) continue;
                    uint32_t xa[16];
                    permute_x<VARIANT>(xv[k], xa);
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        lds_x[((xg[k] * 4 + j) * 4 + xq[k]) * MR + xm[k]] =
                            (u32x4){xa[4 * j], xa[4 * j + 1], xa[4 * j + 2], xa[4 * j + 3]};
                }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                // this stage's scales leave ring set p before it is refilled
                float scur[NT][SPL];
#pragma unroll
                for (int t = 0; t < NT; ++t)
#pragma unroll
                    for (int k = 0; k < SPL; ++k) scur[t][k] = sc[p][t][k];
                load_x(gs + SG);
                load_codes(p, gs + PC * SG);
                if (gs + SG <= g_end)
                    compute(std::true_type{}, scur, gs);
                else
                    compute(std::false_type{}, scur, gs);
                if (gs >= last) goto done;
                gs += SG;
            }
        }
    done:;
    }

    __syncthreads();
    float *red = reinterpret_cast<float *>(smem);
    constexpr int E = NT * 256;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave * E + (t * 4 + i) * 64 + lane] = acc[t][i];
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 64 * KW) {
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < KW; ++w) s += red[w * E + e];
        const int le = e & 63, i = (e >> 6) & 3, t = e >> 8;
        const int m = m0 + 4 * (le >> 4) + i;
        const int n = n0 + 16 * t + (le & 15);
        if (m < M && n < N) Y[(size_t)m * N + n] = s * 16384.0f;
    }
}

// Tiled variant for wide batches (M >= 64).  A workgroup owns a BM x BN
// output tile.  Per group of K it decodes the BN weight rows once into LDS as
// exact FP16 s * t (t is ternary, so s * t is an FP16 value: the slot value v
// of the decode above becomes t with one packed FMA, v * 2^14 - wt(q), and
// t * s with one packed multiply), and stages the BM activation rows beside
// them, permuted into the decode's pair order (permute_x), so that both MFMA
// operands read the same K order.  With the scale inside B the accumulators
// run across all groups: no correction MFMAs and no per-group scale FMAs.
// The eight waves specialise: four consumers run the MFMAs of group g from
// one LDS buffer (2 x 2 waves of (BM/2) x (BN/2), v_mfma_f32_32x32x16_f16)
// while four producers load, decode and stage group g + 1 into the other, one
// barrier per group; a producer and a consumer share each SIMD, so the decode
// and the MFMAs overlap (with all eight waves doing both in turn, the phases
// ran one after the other and the kernel was slower than the per-group one).
// Producers load group g + 2 into registers as they finish g + 1.
constexpr int kTilePitch = 272;  // LDS bytes per staged row: 256 + 16 of skew

template <int BM, int BN>
constexpr size_t tile_lds_bytes() {
    return (size_t)2 * (BM + BN) * kTilePitch;
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int VARIANT, int BM, int BN>
__global__ __launch_bounds__(512) void gemm_tile_kernel(const uint8_t *__restrict__ codes,
                                                        const uint16_t *__restrict__ scales,
                                                        const uint16_t *__restrict__ X,
                                                        float *__restrict__ Y, int M, int N, int K) {
    using F = Fmt<VARIANT>;
    constexpr int GB = F::kGroupBytes;
    constexpr int WM = BM / 2, WN = BN / 2;      // consumer wave tile
    static_assert(WM % 32 == 0 && WN % 32 == 0, "consumer tiles are 32 x 32 MFMA tiles");
    // producer work: ternary rows take two threads (16 code bytes each, two
    // 32-weight chunks), binary rows one (16 bytes, four chunks)
    constexpr int CPT = VARIANT == TQ_TERNARY ? 2 : 4;   // chunks decoded per thread
    constexpr int WTHREADS = BN * 4 / CPT;               // producer threads decoding weights
    constexpr int XTHREADS = BM * 2;                     // producer threads staging activations
    static_assert(WTHREADS <= 256 && XTHREADS <= 256, "one staging item per producer thread");
    __shared__ __attribute__((aligned(16))) uint8_t smem[tile_lds_bytes<BM, BN>()];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const bool producer = wave >= 4;
    const int G = K >> 7;
    const size_t RB = (size_t)G * GB;
    const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;

    if (producer) {
        const int tid = threadIdx.x - 256;
        const bool w_role = tid < WTHREADS, x_role = tid < XTHREADS;
        const int w_row = tid / (4 / CPT), w_part = tid % (4 / CPT);  // 16-byte part of the row's group
        const int x_row = tid >> 1, x_part = tid & 1;                 // 64-activation half of the row's group
        const uint8_t *wsrc = codes + (size_t)min(n0 + min(w_row, BN - 1), N - 1) * RB + 16 * w_part;
        const uint16_t *ssrc = scales + (size_t)min(n0 + min(w_row, BN - 1), N - 1) * G;
        const uint16_t *xsrc = X + (size_t)min(m0 + min(x_row, BM - 1), M - 1) * K + 64 * x_part;
        u32x4 wc;          // 16 code bytes
        uint32_t sbits;    // the row's scale
        u32x4 xr[2][4];    // 64 activations (two 32-activation chunks)
        auto load = [&](int g) __attribute__((always_inline)) {
            wc = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(wsrc + (size_t)g * GB));
            sbits = ssrc[g];
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    xr[c][k] = *reinterpret_cast<const u32x4 *>(xsrc + (size_t)g * 128 + 32 * c + 8 * k);
        };
        const Decoder<VARIANT> dec;
        const uint32_t two14 = vreg(0x74007400u);  // FP16 16384, both halves
        auto stage = [&](int b) __attribute__((always_inline)) {
            uint8_t *ws = smem + (size_t)b * (BM + BN) * kTilePitch;
            uint8_t *xs = ws + (size_t)BN * kTilePitch;
            if (w_role) {
                const uint32_t s2 = (sbits & 0xFFFFu) | (sbits << 16);
#pragma unroll
                for (int c = 0; c < CPT; ++c) {
                    uint32_t d[2];
                    if (VARIANT == TQ_TERNARY) {
                        d[0] = wc[2 * c];
                        d[1] = wc[2 * c + 1];
                    } else {
                        d[0] = wc[c];
                        d[1] = 0;
                    }
                    uint32_t w[16];
                    dec(d, w);
                    exact_st<VARIANT>(w, s2, two14);
                    const int chunk = CPT * w_part + c;  // 32-weight chunk of the group
                    u32x4 *dst = reinterpret_cast<u32x4 *>(ws + (size_t)w_row * kTilePitch + 64 * chunk);
#pragma unroll
                    for (int k = 0; k < 4; ++k) dst[k] = u32x4{w[4 * k], w[4 * k + 1], w[4 * k + 2], w[4 * k + 3]};
                }
            }
            if (x_role) {
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    uint32_t xa[16];
                    permute_x<VARIANT>(xr[c], xa);
                    u32x4 *dst = reinterpret_cast<u32x4 *>(xs + (size_t)x_row * kTilePitch + 64 * (2 * x_part + c));
#pragma unroll
                    for (int k = 0; k < 4; ++k) dst[k] = u32x4{xa[4 * k], xa[4 * k + 1], xa[4 * k + 2], xa[4 * k + 3]};
                }
            }
        };
        load(0);
        stage(0);
        load(min(1, G - 1));
        __syncthreads();
        for (int g = 0; g < G; ++g) {
            // the other buffer was last read before the previous barrier
            if (g + 1 < G) {
                stage((g + 1) & 1);
                load(min(g + 2, G - 1));
            }
            __syncthreads();
        }
    } else {
        // v_mfma_f32_32x32x16_f16: lane l supplies A row / B column l % 32 and
        // the K half l / 32 of each 16-wide slice; D element i of lane l is
        // row 8 (i / 4) + 4 (l / 32) + i % 4, column l % 32
        constexpr int UM = WM / 32, UN = WN / 32;
        const int wm = wave >> 1, wn = wave & 1;
        const int l32 = lane & 31, h2 = lane >> 5;
        f32x16 acc[UM][UN];
#pragma unroll
        for (int a = 0; a < UM; ++a)
#pragma unroll
            for (int b = 0; b < UN; ++b)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;
        __syncthreads();
        for (int g = 0; g < G; ++g) {
            const uint8_t *ws = smem + (size_t)(g & 1) * (BM + BN) * kTilePitch;
            const uint8_t *xs = ws + (size_t)BN * kTilePitch;
#pragma unroll
            for (int j = 0; j < 8; ++j) {  // 16-wide K slice of the group
                half8 av[UM], bv[UN];
#pragma unroll
                for (int a = 0; a < UM; ++a)
                    av[a] = *reinterpret_cast<const half8 *>(
                        xs + (size_t)(wm * WM + 32 * a + l32) * kTilePitch + 32 * j + 16 * h2);
#pragma unroll
                for (int b = 0; b < UN; ++b)
                    bv[b] = *reinterpret_cast<const half8 *>(
                        ws + (size_t)(wn * WN + 32 * b + l32) * kTilePitch + 32 * j + 16 * h2);
#pragma unroll
                for (int a = 0; a < UM; ++a)
#pragma unroll
                    for (int b = 0; b < UN; ++b)
                        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[a], bv[b], acc[a][b], 0, 0, 0);
            }
            __syncthreads();
        }
#pragma unroll
        for (int a = 0; a < UM; ++a)
#pragma unroll
            for (int b = 0; b < UN; ++b)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int m = m0 + wm * WM + 32 * a + 8 * (i / 4) + 4 * h2 + i % 4;
                    const int n = n0 + wn * WN + 32 * b + l32;
                    if (m < M && n < N) Y[(size_t)m * N + n] = acc[a][b][i];
                }
    }
}

template <int VARIANT, int BM, int BN>
hipError_t launch_tile(const uint8_t *codes, const uint16_t *scales, const uint16_t *X, float *Y,
                       int M, int N, int K, hipStream_t stream) {
    const dim3 grid((N + BN - 1) / BN, (M + BM - 1) / BM);
    hipLaunchKernelGGL((gemm_tile_kernel<VARIANT, BM, BN>), grid, dim3(512), 0, stream, codes, scales,
                       X, Y, M, N, K);
    return hipGetLastError();
}

template <int VARIANT, int NT, int MR, int KW, int PC>
hipError_t launch_stage(const uint8_t *codes, const uint16_t *scales, const uint16_t *X, float *Y,
                        int M, int N, int K, hipStream_t stream) {
    const dim3 grid((N + 16 * NT - 1) / (16 * NT), (M + 15) / 16);
    hipLaunchKernelGGL((gemm_stage_kernel<VARIANT, NT, MR, KW, PC>), grid, dim3(64 * KW), 0, stream,
                       codes, scales, X, Y, M, N, K);
    return hipGetLastError();
}

template <int VARIANT, int NT, int MT, int KW>
hipError_t launch(const uint8_t *codes, const uint16_t *scales, const uint16_t *X, float *Y, int M,
                  int N, int K, hipStream_t stream) {
    const dim3 grid((N + 16 * NT - 1) / (16 * NT), (M + 16 * MT - 1) / (16 * MT));
    hipLaunchKernelGGL((gemm_kernel<VARIANT, NT, MT, KW>), grid, dim3(64 * KW), 0, stream, codes,
                       scales, X, Y, M, N, K);
    return hipGetLastError();
}

// Configurations measured on the MLP shapes (17408 x 5120 and 5120 x 17408):
// M >= 128 with at least 128 output tiles of 128 x 128 takes the tiled kernel
// (M = 128 / 512 on 17408 x 5120: 67 / 189 us against 81 / 213 for the
// per-group kernel; 5120 x 17408 at M = 512: 204 against 225; with fewer
// tiles, 5120 x 17408 at M = 256 is 205 against 135),
// M <= 4 takes the stage-pipelined kernel with four staged activation rows,
// M <= 8 the same kernel with eight while N <= 65536 (18.0 / 19.5 us at M = 8
// against 21.4 / 21.0 for the per-group kernel; on the 248320-row LM head it
// took 166 us against 116: its waves live for 2.5 stages only, and sixteen
// staged rows are slower than the per-group kernel at M = 16); wider batches
// and taller matrices take the per-group kernel, with
// taller weight tiles and a two-way K split when N leaves enough workgroups
// (N >= 8192), else shorter tiles and a four-way split.
template <int VARIANT>
hipError_t dispatch(const uint8_t *codes, const uint16_t *scales, const uint16_t *X, float *Y,
                    int M, int N, int K, hipStream_t s) {
    const bool tall = N >= 8192;
    // the tiled kernel needs a grid of about half the CUs to pay off
    if (M >= 128 && (int64_t)((N + 127) / 128) * ((M + 127) / 128) >= 128)
        return launch_tile<VARIANT, 128, 128>(codes, scales, X, Y, M, N, K, s);
    if (M <= 4) return launch_stage<VARIANT, 2, 4, 4, 1>(codes, scales, X, Y, M, N, K, s);
    if (M <= 8 && N <= 65536) return launch_stage<VARIANT, 2, 8, 4, 1>(codes, scales, X, Y, M, N, K, s);
    if (M <= 16)
        return tall ? launch<VARIANT, 4, 1, 2>(codes, scales, X, Y, M, N, K, s)
                    : launch<VARIANT, 2, 1, 4>(codes, scales, X, Y, M, N, K, s);
    if (M <= 32) return launch<VARIANT, 4, 2, 4>(codes, scales, X, Y, M, N, K, s);
    return tall ? launch<VARIANT, 4, 4, 2>(codes, scales, X, Y, M, N, K, s)
                : launch<VARIANT, 4, 2, 4>(codes, scales, X, Y, M, N, K, s);
}

}  // namespace

int32_t gemm_enqueue(const uint8_t *codes, const uint16_t *scales, const uint16_t *X, float *Y,
                     int64_t M, int64_t N, int64_t K, int32_t variant, hipStream_t stream) {
    const hipError_t e =
        variant == TQ_TERNARY
            ? dispatch<TQ_TERNARY>(codes, scales, X, Y, (int)M, (int)N, (int)K, stream)
            : dispatch<TQ_BINARY>(codes, scales, X, Y, (int)M, (int)N, (int)K, stream);
    if (e != hipSuccess) return fail(TQ_ERR_HIP, "GEMM launch failed: %s", hipGetErrorString(e));
    return TQ_OK;
}

}  // namespace tq
