// Batch-1 decode GEMV over packed ternary / binary g128 weights, gfx950.
//
// y[n] = sum_g s[n][g] * sum_{j<128} t[n][128g+j] * x[128g+j]
// (w_i = s_g * t_i with one FP16 scale per 128 weights: thakicloud.github.io,
// "Bonsai 27B: ternary and 1-bit quantization", "How the compression works";
// the packed slots are consumed directly and the scale is applied inside the
// matmul: aitrends.kr, "Ternary-Bonsai-27B-mlx-2bit", "Technical features").
//
// Decode.  v_dot2_f32_f16 is accurate to a few ulp of its largest operand
// when fed normal FP16 values, so every code is turned into a normal FP16
// whose value is linear in the code, without a per-weight normalising op.
// Ternary uses three slot kinds, all in units of 2^-14:
//   E:   a 2-bit code moved to bits [10,12) of a half (the exponent LSBs, the
//        rest zero) is the FP16 c * 2^-14, exactly (0 for c = 0);
//   M4:  a code at bits [8,10) under exponent field 3 is 2^-12 + c * 2^-14;
//   M16: a code at bits [6,8) under exponent field 5 is 2^-10 + c * 2^-14.
// One copy of a code dword serves an E, an M4 and an M16 pair (slot p in the
// low half, p + 8 in the high half): d gives slots 5, 4, 3, d << 6 gives
// 2, 1, 0 and d >> 4 gives 7, 6, so one mask op per pair and two shifts
// decode 16 weights (the shifts taken on two code dwords at once as 64-bit
// shifts: one per dword and copy kind per pair of dwords).  Per 16-byte chunk the slot offsets (4 and 16 units) and
// sum x (t = c - 1) are removed by seeding the chunk's accumulator with
// -(sum x + 4 S_M4 + 16 S_M16) * 2^-14, a constant computed while x is staged
// (S_M4 and S_M16 sum x over those slots), and the row total is scaled by
// 2^14 once.  Rounding stays proportional to the terms summed (the largest
// offset is 16 code units), so a row of zero trits leaves only a small
// residue of order 2^-20 * sum |s * x|.  The 1-bit variant reads bit b at
// position 11 as b * 2^-13 and at position q <= 10 under exponent field
// 12 - q as 2^(-3-q) + b * 2^-13 (offsets 1 .. 16 units of 2^-13); copies d,
// d << 6 and d >> 4 cover a dword's 16 pairs through bits 11..6, and the seed
// -(sum over pairs of (2 offset + 1) x) * 2^-14 leaves 2^-14 (2 sum b*x -
// sum x) = 2^-14 sum t*x.
//
// Work split.  A wave owns 64/LPR row slots of LPR lanes each; lane j of a
// slot takes the chunks j, j+LPR, j+2*LPR, ... of its rows (a chunk is 16
// code bytes; in the register kernel 64 weights: 16 bytes of 2-bit slots or 8
// bytes of binary bits).  Workgroups are persistent, one per CU with eight
// waves, and walk a contiguous range of row blocks round-robin over their
// waves.  Each lane issues its share of the x loads (L2-resident) and its
// first block's code and scale loads before x is permuted into LDS; later
// blocks are loaded while earlier ones are computed.  Per-row partial sums
// are reduced across the LPR lanes with DPP moves (quad_perm,
// row_half_mirror, row_mirror) and swizzles beyond 16.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr size_t kMaxLds = 163840;  // bytes of LDS one gfx950 workgroup may use

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c,
                                  false);
}

// Masks used with v_and_or_b32 stay in VGPRs: gfx9 VOP3 encodings take no
// literal and read one SGPR at most, which then holds the exponent constant.
struct Masks {
    uint32_t m8, m6, m4, b10, b9, b8, b7, b6;
    __device__ __forceinline__ Masks()
        : m8(0x03000300u), m6(0x00C000C0u), m4(0x00300030u), b10(0x04000400u), b9(0x02000200u),
          b8(0x01000100u), b7(0x00800080u), b6(0x00400040u) {
        asm volatile("" : "+v"(m8));
        asm volatile("" : "+v"(m4));
        asm volatile("" : "+v"(m6));
        asm volatile("" : "+v"(b10));
        asm volatile("" : "+v"(b9));
        asm volatile("" : "+v"(b8));
        asm volatile("" : "+v"(b7));
        asm volatile("" : "+v"(b6));
    }
};

typedef uint64_t u64;


// 32 ternary codes (dwords d0, d1) against pairs xp[p] = (x[p], x[p+8]) of
// each dword's 16 weights, accumulated into a in units of 2^-14.
__device__ __forceinline__ void tern_acc32(uint32_t d0, uint32_t d1, const uint32_t *xp0,
                                           const uint32_t *xp1, float &a, const Masks &k) {
    const uint32_t dd[2] = {d0, d1};
    const uint32_t *xps[2] = {xp0, xp1};
    uint32_t l6[2], s4[2];
    shifts64<6, 4>(d0, d1, l6, s4);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t *xp = xps[h];
        const uint32_t c0 = dd[h], c6 = l6[h], r4 = s4[h];
        a = dot2(c0 & 0x0C000C00u, xp[5], a);              // E   slot 5
        a = dot2((c0 & k.m8) | 0x0C000C00u, xp[4], a);     // M4  slot 4
        a = dot2((c0 & k.m6) | 0x14001400u, xp[3], a);     // M16 slot 3
        a = dot2(c6 & 0x0C000C00u, xp[2], a);              // E   slot 2
        a = dot2((c6 & k.m8) | 0x0C000C00u, xp[1], a);     // M4  slot 1
        a = dot2((c6 & k.m6) | 0x14001400u, xp[0], a);     // M16 slot 0
        a = dot2(r4 & 0x0C000C00u, xp[7], a);              // E   slot 7
        a = dot2((r4 & k.m8) | 0x0C000C00u, xp[6], a);     // M4  slot 6
    }
}

// 16 ternary codes (dword d) against its pairs xp[p] = (x[p], x[p+8]),
// accumulated into a in units of 2^-14 (one dword of tern_acc32).
__device__ __forceinline__ void tern_acc16(uint32_t d, const uint32_t *xp, float &a, const Masks &k) {
    const uint32_t c6 = d << 6, r4 = d >> 4;
    a = dot2(d & 0x0C000C00u, xp[5], a);               // E   slot 5
    a = dot2((d & k.m8) | 0x0C000C00u, xp[4], a);      // M4  slot 4
    a = dot2((d & k.m6) | 0x14001400u, xp[3], a);      // M16 slot 3
    a = dot2(c6 & 0x0C000C00u, xp[2], a);              // E   slot 2
    a = dot2((c6 & k.m8) | 0x0C000C00u, xp[1], a);     // M4  slot 1
    a = dot2((c6 & k.m6) | 0x14001400u, xp[0], a);     // M16 slot 0
    a = dot2(r4 & 0x0C000C00u, xp[7], a);              // E   slot 7
    a = dot2((r4 & k.m8) | 0x0C000C00u, xp[6], a);     // M4  slot 6
}

// 32 affine levels q in {0..3} (dwords d0, d1) against pairs xp[p] =
// (x[p], x[p+8]), accumulated into a in units of 2^-14.  Level 3 rules out the
// E slot (exponent field 3 is 4 units, not 3), so three mantissa slots serve
// a copy: M4 at bits [8,10) (exponent 3, 2^-12 + q 2^-14), M16 at [6,8)
// (exponent 5, 2^-10 + q 2^-14) and M64 at [4,6) (exponent 7, 2^-8 + q 2^-14).
// Copies d (slots 4, 3, 2), d << 6 (1, 0) and d >> 6 (7, 6, 5).
__device__ __forceinline__ void aff_acc32(uint32_t d0, uint32_t d1, const uint32_t *xp0,
                                          const uint32_t *xp1, float &a, const Masks &k) {
    const uint32_t dd[2] = {d0, d1};
    const uint32_t *xps[2] = {xp0, xp1};
    uint32_t l6[2], s6[2];
    shifts64<6, 6>(d0, d1, l6, s6);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t *xp = xps[h];
        const uint32_t c0 = dd[h], c6 = l6[h], r6 = s6[h];
        a = dot2((c0 & k.m8) | 0x0C000C00u, xp[4], a);     // M4  slot 4
        a = dot2((c0 & k.m6) | 0x14001400u, xp[3], a);     // M16 slot 3
        a = dot2((c0 & k.m4) | 0x1C001C00u, xp[2], a);     // M64 slot 2
        a = dot2((c6 & k.m8) | 0x0C000C00u, xp[1], a);     // M4  slot 1
        a = dot2((c6 & k.m6) | 0x14001400u, xp[0], a);     // M16 slot 0
        a = dot2((r6 & k.m8) | 0x0C000C00u, xp[7], a);     // M4  slot 7
        a = dot2((r6 & k.m6) | 0x14001400u, xp[6], a);     // M16 slot 6
        a = dot2((r6 & k.m4) | 0x1C001C00u, xp[5], a);     // M64 slot 5
    }
}

// 16 affine levels (dword d) against its pairs xp[p] = (x[p], x[p+8]),
// accumulated into a in units of 2^-14 (one dword of aff_acc32).
__device__ __forceinline__ void aff_acc16(uint32_t d, const uint32_t *xp, float &a, const Masks &k) {
    const uint32_t c6 = d << 6, r6 = d >> 6;
    a = dot2((d & k.m8) | 0x0C000C00u, xp[4], a);      // M4  slot 4
    a = dot2((d & k.m6) | 0x14001400u, xp[3], a);      // M16 slot 3
    a = dot2((d & k.m4) | 0x1C001C00u, xp[2], a);      // M64 slot 2
    a = dot2((c6 & k.m8) | 0x0C000C00u, xp[1], a);     // M4  slot 1
    a = dot2((c6 & k.m6) | 0x14001400u, xp[0], a);     // M16 slot 0
    a = dot2((r6 & k.m8) | 0x0C000C00u, xp[7], a);     // M4  slot 7
    a = dot2((r6 & k.m6) | 0x14001400u, xp[6], a);     // M16 slot 6
    a = dot2((r6 & k.m4) | 0x1C001C00u, xp[5], a);     // M64 slot 5
}

// 64 binary bits (dwords d0, d1) against pairs xp[p] = (x[p], x[p+16]) of
// each dword's 32 weights, accumulated into a: bit b at position 11 is
// b * 2^-13 and at position q <= 10 under exponent field 12 - q it is
// 2^(-3-q) + b * 2^-13.  Copy d reads bits 11..6 (slots 11..6), d << 6 reads
// bits 5..0 and d >> 4 bits 15..12, each through slots 11.. downwards.
__device__ __forceinline__ void bin_slots(uint32_t c, const uint32_t *xp, int p0, int n, float &a,
                                          const Masks &k) {
    a = dot2(c & 0x08000800u, xp[p0], a);                          // bit 11
    a = dot2((c & k.b10) | 0x08000800u, xp[p0 - 1], a);            // bit 10, offset 1
    a = dot2((c & k.b9) | 0x0C000C00u, xp[p0 - 2], a);             // bit 9,  offset 2
    a = dot2((c & k.b8) | 0x10001000u, xp[p0 - 3], a);             // bit 8,  offset 4
    if (n > 4) a = dot2((c & k.b7) | 0x14001400u, xp[p0 - 4], a);  // bit 7,  offset 8
    if (n > 5) a = dot2((c & k.b6) | 0x18001800u, xp[p0 - 5], a);  // bit 6,  offset 16
}

__device__ __forceinline__ void bin_acc64(uint32_t d0, uint32_t d1, const uint32_t *xp0,
                                          const uint32_t *xp1, float &a, const Masks &k) {
    const uint32_t dd[2] = {d0, d1};
    const uint32_t *xps[2] = {xp0, xp1};
    uint32_t l6[2], s4[2];
    shifts64<6, 4>(d0, d1, l6, s4);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        bin_slots(dd[h], xps[h], 11, 6, a, k);
        bin_slots(l6[h], xps[h], 5, 6, a, k);
        bin_slots(s4[h], xps[h], 15, 4, a, k);
    }
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                                 0xF, 0xF, false));
}

// v + (v of the lane W = 16 or 32 away, within 2W-lane groups): a
// v_permlane16/32_swap of v with itself leaves the lane's own value in one
// result and its partner's in the other, so their sum is what a lane-xor
// shuffle gives, on the VALU instead of through the LDS crossbar.
template <int W>
__device__ __forceinline__ float swap_sum(float v) {
    const uint32_t u = __builtin_bit_cast(uint32_t, v);
    const auto e = W == 16 ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                           : __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __builtin_bit_cast(float, (uint32_t)e[0]) + __builtin_bit_cast(float, (uint32_t)e[1]);
}

// Sum over aligned segments of LPR lanes; every lane of a segment gets the sum.
template <int LPR>
__device__ __forceinline__ float seg_sum(float v) {
    if (LPR >= 2) v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
    if (LPR >= 4) v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
    if (LPR >= 8) v += dpp_f<0x141>(v);  // row_half_mirror
    if (LPR >= 16) v += dpp_f<0x140>(v); // row_mirror
    if (LPR >= 32) v = swap_sum<16>(v);
    if (LPR >= 64) v = swap_sum<32>(v);
    return v;
}

// x staging.  Ternary unit: 16 weights -> 8 pairs (p, p+8); binary unit:
// 32 weights -> 16 pairs (p, p+16).  UPC consecutive units make one chunk:
// four for a 16-byte code chunk (64 ternary or 128 binary weights), two for
// the register kernel's 8-byte binary chunk (64 weights).  In LDS every chunk has a
// slot of CHUNK_DW dwords: its pairs, then its constant (a float), then pad,
// so chunk c of a row sits at c * CHUNK_DW and the compute loop addresses
// every chunk with an immediate offset.  Slots past the last real chunk (a
// ragged row shape) hold zeros, which makes their contribution exactly 0.
template <int VARIANT, int UPC = 4>
struct XUnit {
    static constexpr int UNIT = VARIANT == TQ_BINARY ? 32 : 16;
    static constexpr int PAIRS = UPC * UNIT / 2;      // pair dwords per chunk of UPC units
    static constexpr int CHUNK_DW = PAIRS + 4;        // 36 or 68: 16-byte aligned, bank-spread
    static constexpr int V4 = UNIT / 8;               // 16-byte loads per unit
    u32x4 v[V4];

    // FP16 pair (w, w) weighting pair p in the chunk constant
    static __device__ __forceinline__ uint32_t zweight(int p) {
        if constexpr (VARIANT == TQ_AFFINE2) {
            // the slot offsets alone (no t = c - 1 shift): M16 slots 0, 3, 6;
            // M4 slots 1, 4, 7; M64 slots 2, 5
            return (p == 0 || p == 3 || p == 6) ? 0x4C004C00u : (p == 2 || p == 5) ? 0x54005400u
                                                                                   : 0x44004400u;  // 16 : 64 : 4
        } else if constexpr (VARIANT == TQ_TERNARY) {
            // E slots 2, 5, 7; M4 slots 1, 4, 6; M16 slots 0, 3
            return (p == 0 || p == 3) ? 0x4C404C40u : (p == 1 || p == 4 || p == 6) ? 0x45004500u
                                                                                    : 0x3C003C00u;  // 17 : 5 : 1
        } else {
            // pair p is read by the slot at bit 11 - (p + 4) % 6 for p <= 11 (copies d
            // and d << 6) or 11 - (15 - p) for p >= 12 (copy d >> 4); weight 2 off + 1
            constexpr uint32_t w[16] = {0x50205020u, 0x4C404C40u, 0x48804880u, 0x45004500u,
                                        0x42004200u, 0x3C003C00u, 0x50205020u, 0x4C404C40u,
                                        0x48804880u, 0x45004500u, 0x42004200u, 0x3C003C00u,
                                        0x48804880u, 0x45004500u, 0x42004200u, 0x3C003C00u};
            return w[p];  // 33 17 9 5 3 1 | 33 17 9 5 3 1 | 9 5 3 1
        }
    }

    // accumulator unit 2^-14 for both variants (binary codes carry b in units of
    // 2^-13, which folds the 2 of t = 2b - 1)
    static constexpr float kSeedScale = 6.103515625e-05f;
    static constexpr float kRowScale = 16384.0f;

    __device__ __forceinline__ void load(const uint16_t *__restrict__ x, int u) {
        const u32x4 *src = reinterpret_cast<const u32x4 *>(x + (size_t)u * UNIT);
#pragma unroll
        for (int i = 0; i < V4; ++i) v[i] = src[i];
    }

    // Writes unit u (zeros when !real) into its chunk slot; the lane holding a
    // chunk's first unit writes the chunk constant.  The UPC units of a chunk
    // are UPC aligned consecutive lanes, so the constant reduces with seg_sum.
    __device__ __forceinline__ void store(uint32_t *xs, int u, bool real) const {
        uint32_t xp[UNIT / 2];
        // low halves x[0..UNIT/2), high halves x[UNIT/2..UNIT)
#pragma unroll
        for (int i = 0; i < UNIT / 4; ++i) {
            const uint32_t l = v[i / 4][i % 4], h = v[V4 / 2 + i / 4][i % 4];
            xp[2 * i] = real ? (l & 0xFFFFu) | (h << 16) : 0u;
            xp[2 * i + 1] = real ? (l >> 16) | (h & 0xFFFF0000u) : 0u;
        }
        // seed: -(sum over the pairs of w_p * (x[p] + x[p+UNIT/2])) * 2^-14 with
        // w = 1 + offset (ternary: 1, 5, 17) or 2 offset + 1 (binary: 1 .. 33)
        float z = 0.0f;
#pragma unroll
        for (int i = 0; i < UNIT / 2; ++i) z = dot2(xp[i], zweight(i), z);
        uint32_t *slot = xs + (u / UPC) * CHUNK_DW;
        uint32_t *dst = slot + (u % UPC) * (UNIT / 2);
#pragma unroll
        for (int i = 0; i < UNIT / 8; ++i)
            reinterpret_cast<u32x4 *>(dst)[i] = u32x4{xp[4 * i], xp[4 * i + 1], xp[4 * i + 2], xp[4 * i + 3]};
        z = seg_sum<UPC>(z) * -kSeedScale;
        if (u % UPC == 0) slot[PAIRS] = __builtin_bit_cast(uint32_t, z);
        if constexpr (VARIANT == TQ_AFFINE2) {
            // the chunk's plain sum of x, in the accumulator unit, for the bias
            float zs = 0.0f;
#pragma unroll
            for (int i = 0; i < UNIT / 2; ++i) zs = dot2(xp[i], 0x3C003C00u, zs);
            zs = seg_sum<UPC>(zs) * kSeedScale;
            if (u % UPC == 0) slot[PAIRS + 1] = __builtin_bit_cast(uint32_t, zs);
        }
    }
};

// Decode and dot one 16-byte chunk position for RPL rows and fold it into
// their accumulators: acc[r] += s[r] * (sum of row r's chunk products, in the
// accumulator unit).  xg is the chunk's LDS slot, read once for all RPL rows.
template <int VARIANT, int RPL>
__device__ __forceinline__ void chunk_dot(const u32x4 (&c)[RPL], const uint32_t *xg,
                                          const uint32_t (&sbits)[RPL], float (&acc)[RPL],
                                          const Masks &km) {
    using XU = XUnit<VARIANT>;
    const float seed = __builtin_bit_cast(float, xg[XU::PAIRS]);
    float aE[RPL], aM[RPL];
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
        aE[r] = 0.0f;
        aM[r] = seed;
    }
#pragma unroll
    for (int d = 0; d < 4; d += 2) {
        if constexpr (VARIANT == TQ_TERNARY) {
            const u32x4 q0 = reinterpret_cast<const u32x4 *>(xg + 8 * d)[0];
            const u32x4 q1 = reinterpret_cast<const u32x4 *>(xg + 8 * d)[1];
            const u32x4 q2 = reinterpret_cast<const u32x4 *>(xg + 8 * d)[2];
            const u32x4 q3 = reinterpret_cast<const u32x4 *>(xg + 8 * d)[3];
            const uint32_t xp0[8] = {q0[0], q0[1], q0[2], q0[3], q1[0], q1[1], q1[2], q1[3]};
            const uint32_t xp1[8] = {q2[0], q2[1], q2[2], q2[3], q3[0], q3[1], q3[2], q3[3]};
#pragma unroll
            for (int r = 0; r < RPL; ++r) tern_acc32(c[r][d], c[r][d + 1], xp0, xp1, aM[r], km);
        } else {
            uint32_t xp0[16], xp1[16];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const u32x4 qa = reinterpret_cast<const u32x4 *>(xg + 16 * d)[v];
                const u32x4 qb = reinterpret_cast<const u32x4 *>(xg + 16 * d + 16)[v];
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    xp0[4 * v + w] = qa[w];
                    xp1[4 * v + w] = qb[w];
                }
            }
#pragma unroll
            for (int r = 0; r < RPL; ++r) bin_acc64(c[r][d], c[r][d + 1], xp0, xp1, aM[r], km);
        }
    }
#pragma unroll
    for (int r = 0; r < RPL; ++r)
        acc[r] = __builtin_fmaf((float)__builtin_bit_cast(_Float16, (uint16_t)sbits[r]), aE[r] + aM[r],
                                acc[r]);
}

// Registers a lane keeps per chunk column: 32 pair dwords and the seed, plus
// the chunk's sum of x for affine levels.  A register-kernel chunk is 64
// weights for every variant: 16 code bytes of 2-bit slots (four 16-weight
// units) or 8 bytes of binary bits (two 32-weight units).
template <int VARIANT>
struct XReg {
    static constexpr int N = VARIANT == TQ_AFFINE2 ? 34 : 33;
    static constexpr int UPC = VARIANT == TQ_BINARY ? 2 : 4;        // units per chunk
    static constexpr int CB = VARIANT == TQ_BINARY ? 8 : 16;        // code bytes per chunk
    using Unit = XUnit<VARIANT, UPC>;
    using Code = typename std::conditional<VARIANT == TQ_BINARY, u32x2, u32x4>::type;
};

__device__ __forceinline__ float half_bits(uint32_t bits) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

// chunk_dot with the chunk's pairs and constants held in registers (one
// row): xr[0..32) are the pairs of the chunk's units, xr[32] the seed.
// Affine levels add the group's bias times xr[33], the chunk's sum of x in
// the accumulator unit (w = s q + b: s * sum q x + b * sum x).
template <int VARIANT>
__device__ __forceinline__ void chunk_dot_reg(const typename XReg<VARIANT>::Code &c,
                                              const uint32_t (&xr)[XReg<VARIANT>::N],
                                              uint32_t sbits, uint32_t bbits, float &acc,
                                              const Masks &km) {
    float a = __builtin_bit_cast(float, xr[32]);
    if constexpr (VARIANT == TQ_BINARY) {
        bin_acc64(c[0], c[1], xr, xr + 16, a, km);
        acc = __builtin_fmaf(half_bits(sbits), a, acc);
    } else if constexpr (VARIANT == TQ_AFFINE2) {
        aff_acc32(c[0], c[1], xr, xr + 8, a, km);
        aff_acc32(c[2], c[3], xr + 16, xr + 24, a, km);
        acc = __builtin_fmaf(half_bits(sbits), a, acc);
        acc = __builtin_fmaf(half_bits(bbits), __builtin_bit_cast(float, xr[33]), acc);
    } else {
        tern_acc32(c[0], c[1], xr, xr + 8, a, km);
        tern_acc32(c[2], c[3], xr + 16, xr + 24, a, km);
        acc = __builtin_fmaf(half_bits(sbits), a, acc);
    }
}

// One row block = RPL * 64/LPR consecutive rows handled by one wave: LPR lanes
// per row, lane (seg, j) takes rows seg, seg + 64/LPR, ... of the block and in
// each the 16-byte chunks j, j+LPR, ..., so consecutive lanes read consecutive
// 16 bytes.  When LPR*NU exceeds the chunks of a row (RAGGED), chunk and scale
// indices are clamped into the row; those slots' x is zero, so they contribute
// nothing.  Otherwise every chunk is the row base plus a compile-time offset.
// Scales are loaded first and kept zero-extended, one per register.
template <int VARIANT, int LPR, int NU, int RPL, bool RAGGED>
__device__ __forceinline__ void load_block(const uint8_t *__restrict__ codes,
                                           const uint16_t *__restrict__ scales, const int (&row)[RPL],
                                           int j, int CPR, int G, u32x4 (&c)[NU][RPL],
                                           uint32_t (&s)[NU][RPL]) {
    constexpr int CPG = VARIANT == TQ_BINARY ? 1 : 2;  // 16-byte chunks per group
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
        const uint16_t *sp = scales + (size_t)row[r] * G;
#pragma unroll
        for (int i = 0; i < NU; ++i)
            s[i][r] = RAGGED ? sp[min(j + i * LPR, CPR - 1) / CPG] : sp[j / CPG + i * (LPR / CPG)];
    }
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
        const u32x4 *rp = reinterpret_cast<const u32x4 *>(codes + (size_t)row[r] * CPR * 16);
#pragma unroll
        for (int i = 0; i < NU; ++i)
            c[i][r] = __builtin_nontemporal_load(rp + (RAGGED ? min(j + i * LPR, CPR - 1) : j + i * LPR));
    }
}

// This lane's share of a block: per row, the sum over its chunks reduced over
// the row's LPR lanes, times the accumulator's power-of-two unit.  The
// scheduling barrier keeps one chunk's activations live at a time.
template <int VARIANT, int LPR, int NU, int RPL>
__device__ __forceinline__ void block_dot(const u32x4 (&c)[NU][RPL], const uint32_t (&s)[NU][RPL],
                                          const uint32_t *xj, const Masks &km, float (&out)[RPL]) {
    float acc[RPL];
#pragma unroll
    for (int r = 0; r < RPL; ++r) acc[r] = 0.0f;
#pragma unroll
    for (int i = 0; i < NU; ++i) {
        chunk_dot<VARIANT, RPL>(c[i], xj + i * LPR * XUnit<VARIANT>::CHUNK_DW, s[i], acc, km);
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int r = 0; r < RPL; ++r) out[r] = seg_sum<LPR>(acc[r]) * XUnit<VARIANT>::kRowScale;
}

// Persistent GEMV.  Each workgroup stages x once, then its waves walk the
// workgroup's contiguous range of row blocks round-robin, prefetching the
// next block while decoding the current one (two register sets, ping-pong).
template <int VARIANT, int LPR, int NU, int RPL, int WAVES, bool RAGGED>
__global__ __launch_bounds__(64 * WAVES) void gemv_kernel(const uint8_t *__restrict__ codes,
                                                          const uint16_t *__restrict__ scales,
                                                          const uint16_t *__restrict__ x,
                                                          float *__restrict__ y, int N, int K) {
    extern __shared__ uint32_t xs[];
    using XU = XUnit<VARIANT>;
    constexpr int THREADS = 64 * WAVES;
    constexpr int RS = 64 / LPR;                        // rows per wave slot
    constexpr int RB = RS * RPL;                        // rows per block
    constexpr int CAP = LPR * NU;                       // chunk slots per row
    constexpr int XMAX = (CAP * 4 + THREADS - 1) / THREADS;
    const int G = K >> 7, CPR = G * (VARIANT == TQ_BINARY ? 1 : 2);
    const int nunits = CPR * 4;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int seg = lane / LPR, j = lane % LPR;
    const int nblocks = (N + RB - 1) / RB;
    const int b_begin = (int)(((long long)blockIdx.x * nblocks) / gridDim.x);
    const int b_end = (int)(((long long)(blockIdx.x + 1) * nblocks) / gridDim.x);
    const Masks km;
    auto rows_of = [&](int bb, int (&row)[RPL]) {
#pragma unroll
        for (int r = 0; r < RPL; ++r) row[r] = min(bb * RB + r * RS + seg, N - 1);
    };

    // 1. x loads for staging, then the first block's codes and scales
    XU xu[XMAX];
#pragma unroll
    for (int k = 0; k < XMAX; ++k)
        xu[k].load(x, min(min((int)threadIdx.x + k * THREADS, CAP * 4 - 1), nunits - 1));
    __builtin_amdgcn_sched_barrier(0);
    // every wave's x loads ahead of any wave's code loads (a barrier, no
    // wait for data), as in the register kernel: 0.06-0.09 us less per
    // launch on 5120 x 24576 than a per-wave wait for x, 0.16 us less than
    // issuing them together
    __builtin_amdgcn_s_barrier();
    u32x4 ca[NU][RPL], cb[NU][RPL];
    uint32_t sa[NU][RPL], sb[NU][RPL];
    int b = b_begin + wave;
    int row[RPL];
    rows_of(min(b, b_end - 1), row);
    load_block<VARIANT, LPR, NU, RPL, RAGGED>(codes, scales, row, j, CPR, G, ca, sa);
    __builtin_amdgcn_sched_barrier(0);

    // 2. permuted x and chunk constants into LDS (zero slots past the row).
    // Threads past the last slot redo the last unit (identical data; only the
    // first unit of a chunk writes its constant): an unconditional store keeps
    // the x loads from being sunk below the code stream.
#pragma unroll
    for (int k = 0; k < XMAX; ++k) {
        const int u = min((int)threadIdx.x + k * THREADS, CAP * 4 - 1);
        xu[k].store(xs, u, u < nunits);
    }
    __syncthreads();

    // 3. ping-pong over this wave's blocks
    const uint32_t *xj = xs + j * XU::CHUNK_DW;
    float out[RPL];
    for (; b < b_end; b += 2 * WAVES) {
        const int b2 = b + WAVES;
        if (b2 < b_end) {
            rows_of(b2, row);
            load_block<VARIANT, LPR, NU, RPL, RAGGED>(codes, scales, row, j, CPR, G, cb, sb);
        }
        block_dot<VARIANT, LPR, NU, RPL>(ca, sa, xj, km, out);
#pragma unroll
        for (int r = 0; r < RPL; ++r) {
            const int rr = b * RB + r * RS + seg;
            if (j == 0 && rr < N) y[rr] = out[r];
        }
        if (b2 >= b_end) break;
        const int b3 = b2 + WAVES;
        if (b3 < b_end) {
            rows_of(b3, row);
            load_block<VARIANT, LPR, NU, RPL, RAGGED>(codes, scales, row, j, CPR, G, ca, sa);
        }
        block_dot<VARIANT, LPR, NU, RPL>(cb, sb, xj, km, out);
#pragma unroll
        for (int r = 0; r < RPL; ++r) {
            const int rr = b2 * RB + r * RS + seg;
            if (j == 0 && rr < N) y[rr] = out[r];
        }
    }
}

// Group biases of a block (affine levels), indexed like the scales in
// load_block (two chunks per group).
template <int LPR, int NU, bool RAGGED>
__device__ __forceinline__ void load_bias(const uint16_t *__restrict__ biases, int row, int j, int CPR,
                                          int G, uint32_t (&bv)[NU][1]) {
    const uint16_t *bp = biases + (size_t)row * G;
#pragma unroll
    for (int i = 0; i < NU; ++i)
        bv[i][0] = RAGGED ? bp[min(j + i * LPR, CPR - 1) / 2] : bp[j / 2 + i * (LPR / 2)];
}

// Ternary, binary and affine 2-bit GEMV, one row per lane segment, with the
// lane's activations in registers.  Lane j of a row segment only ever reads chunk
// columns j, j + LPR, ..., so after the workgroup has staged x into LDS once
// (permuted, with the chunk constants), each lane copies its NU chunk slots
// into VGPRs and the block loop reads no LDS at all.
//
// Two block loops.  PIPE (scales, and affine biases, readable as aligned
// dwords; binary chunks are 8 code bytes, two 32-weight units): one register
// set, each chunk refilled with the wave's next block as soon as it is
// consumed, a block's compute ahead of its use.  Every load is unconditional
// (clamped to the range's last block, mostly a cache hit), so the load order
// is the same on every path and the compiler's wait before each chunk is for
// that chunk only.  Only the first block is requested before the loop: a
// second one there (two register sets) doubled the burst every wave waits
// behind at the start and measured 10 % slower on the MLP shapes.  Scales
// and biases come from the aligned dword that holds them (a genuine 32-bit
// value: 16-bit registers are packed in pairs, and the packing waits for both
// loads).  Otherwise a plain ping-pong of two register sets, each loaded whole
// one block ahead.
template <int VARIANT, int LPR, int NU, int WAVES, bool RAGGED, bool PIPE, int TW = 0>
__global__ __launch_bounds__(64 * WAVES) void gemv_xreg_kernel(const uint8_t *__restrict__ codes,
                                                               const uint16_t *__restrict__ scales,
                                                               const uint16_t *__restrict__ biases,
                                                               const uint16_t *__restrict__ x,
                                                               float *__restrict__ y, int N, int K) {
    extern __shared__ uint32_t xs[];
    using XU = typename XReg<VARIANT>::Unit;
    using Code = typename XReg<VARIANT>::Code;
    constexpr bool AFF = VARIANT == TQ_AFFINE2;
    static_assert(PIPE || VARIANT != TQ_BINARY, "binary codes take the pipelined loop only");
    // TW (tail weights per lane, 16 or 32): a row is NU full chunk columns of
    // the LPR lanes plus LPR TW / 64 chunks more, which the lanes take TW
    // weights each in a tail slot (one or two code dwords of 2-bit codes or
    // affine levels; one 1-bit dword, on lanes j < LPR TW / 32), where a
    // clamped extra chunk column would leave most of its lanes decoding nothing
    constexpr bool TAIL = TW != 0;
    static_assert(TW == 0 || TW == 16 || TW == 32, "a tail slot takes 16 or 32 weights per lane");
    static_assert(!TAIL || (PIPE && !RAGGED && (LPR * NU) % 8 == 0),
                  "the tail slot is an exact, pipelined layout with an even scale dword start");
    constexpr int XN = XReg<VARIANT>::N;
    constexpr int UPC = XReg<VARIANT>::UPC, CB = XReg<VARIANT>::CB;
    constexpr int THREADS = 64 * WAVES;
    constexpr int RS = 64 / LPR;  // rows per block (one per lane segment)
    constexpr int CAP = LPR * NU + LPR * TW / 64;  // staged chunk slots
    constexpr int XMAX = (CAP * UPC + THREADS - 1) / THREADS;
    const int G = K >> 7, CPR = 2 * G;  // 64-weight chunks per row
    const int nunits = CPR * UPC;
    const int lane = threadIdx.x & 63;
    // wave-uniform (scalar) block bookkeeping: the loops branch on SGPRs
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int seg = lane / LPR, j = lane % LPR;
    const int nblocks = (N + RS - 1) / RS;
    const int b_begin = (int)(((long long)blockIdx.x * nblocks) / gridDim.x);
    const int b_end = (int)(((long long)(blockIdx.x + 1) * nblocks) / gridDim.x);
    const Masks km;

    XU xu[XMAX];
#pragma unroll
    for (int k = 0; k < XMAX; ++k)
        xu[k].load(x, min(min((int)threadIdx.x + k * THREADS, CAP * UPC - 1), nunits - 1));
    __builtin_amdgcn_sched_barrier(0);

    // x staged into LDS (permuted, with the chunk constants) once per
    // workgroup, then chunk slot i of this lane copied into registers
    auto stage_lds = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < XMAX; ++k) {
            const int u = min((int)threadIdx.x + k * THREADS, CAP * UPC - 1);
            xu[k].store(xs, u, u < nunits);
        }
        __syncthreads();
    };
    auto fill = [&](uint32_t (&xr)[NU][XN], int i) __attribute__((always_inline)) {
        const uint32_t *slot = xs + (j + i * LPR) * XU::CHUNK_DW;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const u32x4 v = reinterpret_cast<const u32x4 *>(slot)[q];
            xr[i][4 * q] = v[0];
            xr[i][4 * q + 1] = v[1];
            xr[i][4 * q + 2] = v[2];
            xr[i][4 * q + 3] = v[3];
        }
        xr[i][32] = slot[32];
        if constexpr (AFF) xr[i][33] = slot[33];
    };
    auto stage_x = [&](uint32_t (&xr)[NU][XN]) __attribute__((always_inline)) {
        stage_lds();
#pragma unroll
        for (int i = 0; i < NU; ++i) fill(xr, i);
    };
    uint32_t xr[NU][XN];

    if constexpr (PIPE) {
        const int blast = b_end - 1;
        const int b0 = b_begin + wave;
        const int nb = b0 < b_end ? (b_end - b0 + WAVES - 1) / WAVES : 0;  // this wave's blocks
        // chunk columns of this lane (clamped into the row when ragged) and
        // the half of the scale dword that holds each chunk's group scale
        int col[NU];
        uint32_t hsh[NU];
#pragma unroll
        for (int i = 0; i < NU; ++i) {
            col[i] = RAGGED ? min(j + i * LPR, CPR - 1) : j + i * LPR;
            hsh[i] = ((uint32_t)(col[i] >> 1) & 1u) * 16u;
        }
        const uint32_t *sc32 = reinterpret_cast<const uint32_t *>(scales);
        const uint32_t *bi32 = reinterpret_cast<const uint32_t *>(biases);
        // Bases of the row this lane segment loads: the same for all NU
        // chunks of a block, so they are formed once per block and each chunk
        // adds its column (this loop runs with an even group count, so every
        // row's scales start on a dword and chunk col's scale dword is
        // col / 4 into the row).
        const Code *crow = nullptr;
        const uint32_t *srow = nullptr, *brow = nullptr;
        auto set_row = [&](int bb) __attribute__((always_inline)) {
            const int r = min(min(bb, blast) * RS + seg, N - 1);
            crow = reinterpret_cast<const Code *>(codes + (size_t)r * CPR * CB);
            srow = sc32 + (size_t)r * (G >> 1);
            if constexpr (AFF) brow = bi32 + (size_t)r * (G >> 1);
        };
        auto load_chunk = [&](int i, Code (&c)[NU], uint32_t (&sv)[NU], uint32_t (&bv)[NU])
                              __attribute__((always_inline)) {
            // unclamped columns are j + i LPR: constant offsets from the
            // lane's first chunk, which the loads take as immediates
            const int sc = RAGGED ? col[i] >> 2 : (j >> 2) + i * (LPR >> 2);
            sv[i] = srow[sc];
            if constexpr (AFF) bv[i] = brow[sc];
            c[i] = __builtin_nontemporal_load(crow + (RAGGED ? col[i] : j + i * LPR));
        };
        Code ca[NU];
        uint32_t sa[NU], ba[NU];
        // tail slot (TW): lane j takes UL units (UL code dwords of UW weights)
        // from unit UL j of the row's last LPR TW / 64 chunks; their group is
        // LPR NU / 2 + UW UL j / 128, in scale dword LPR NU / 4 + UW UL j / 256
        // at half (UW UL j / 128) & 1 (LPR NU is a multiple of 8).  1-bit
        // lanes j >= TU load the last unit and hold zero activations.
        constexpr int UW = XU::UNIT, TP = UW / 2;        // weights and pair dwords per unit
        constexpr int UL = TW > UW ? TW / UW : 1;        // units per lane
        constexpr int TU = TW ? LPR * TW / UW / UL : 1;  // lanes with tail units
        constexpr int CDW = CB / 4;                      // code dwords per chunk
        using TCode = typename std::conditional<UL == 2, u32x2, uint32_t>::type;
        const int jt = min(j, TU - 1);
        TCode ct{};
        uint32_t st = 0, bt = 0, xt[UL * TP + 2];
        const uint32_t hsh_t = ((uint32_t)(jt * UL * UW / 128) & 1u) * 16u;
        auto load_tail = [&]() __attribute__((always_inline)) {
            if constexpr (TAIL) {
                st = srow[(LPR * NU) / 4 + jt * UL * UW / 256];
                if constexpr (AFF) bt = brow[(LPR * NU) / 4 + jt * UL * UW / 256];
                ct = __builtin_nontemporal_load(
                    reinterpret_cast<const TCode *>(reinterpret_cast<const uint32_t *>(crow) + LPR * NU * CDW) + jt);
            }
        };
        // the units' pairs from their chunk slot and their own seed (the
        // chunk constant covers all the units of a chunk)
        auto fill_tail = [&]() __attribute__((always_inline)) {
            if constexpr (TAIL) {
                const int u0 = jt * UL;
                const uint32_t *slot = xs + (LPR * NU + u0 / UPC) * XU::CHUNK_DW + (u0 % UPC) * TP;
                float z = 0.0f;
#pragma unroll
                for (int q = 0; q < UL * TP / 4; ++q) {
                    const u32x4 v = reinterpret_cast<const u32x4 *>(slot)[q];
#pragma unroll
                    for (int p = 0; p < 4; ++p) xt[4 * q + p] = j < TU ? v[p] : 0u;
                }
#pragma unroll
                for (int p = 0; p < UL * TP; ++p) z = dot2(xt[p], XU::zweight(p % TP), z);
                xt[UL * TP] = __builtin_bit_cast(uint32_t, z * -XU::kSeedScale);
                if constexpr (AFF) {  // the units' plain sum of x, in the accumulator unit
                    float zs = 0.0f;
#pragma unroll
                    for (int p = 0; p < UL * TP; ++p) zs = dot2(xt[p], 0x3C003C00u, zs);
                    xt[UL * TP + 1] = __builtin_bit_cast(uint32_t, zs * XU::kSeedScale);
                }
            }
        };
        // Every wave of the workgroup issues its x loads before any wave
        // issues code loads (a barrier, no wait for data): issued per wave,
        // the x loads of later waves queued behind earlier waves' first-block
        // code bursts and x reached the registers about 2.9 us into the fused
        // MLP launch.  The first block then copies chunk slot i + 1 from LDS
        // while chunk i computes, instead of all 165 registers before the
        // loop (about 340 KB of LDS reads per CU, 1.3 us at 128 B per clock).
        __builtin_amdgcn_s_barrier();
        set_row(b0);
#pragma unroll
        for (int i = 0; i < NU; ++i) load_chunk(i, ca, sa, ba);
        load_tail();
        __builtin_amdgcn_sched_barrier(0);
        stage_lds();
        fill(xr, 0);

        auto block = [&](auto refill, auto first, Code (&c)[NU], uint32_t (&sv)[NU], uint32_t (&bv)[NU], int bb,
                         int bn) __attribute__((always_inline)) {
            float acc = 0.0f;
            if constexpr (decltype(refill)::value) set_row(bn);
#pragma unroll
            for (int i = 0; i < NU; ++i) {
                if constexpr (decltype(first)::value) {
                    if (i + 1 < NU) fill(xr, i + 1);
                    else fill_tail();
                }
                chunk_dot_reg<VARIANT>(c[i], xr[i], sv[i] >> hsh[i], AFF ? bv[i] >> hsh[i] : 0u, acc, km);
                if constexpr (decltype(refill)::value) load_chunk(i, c, sv, bv);
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (TAIL) {
                float a = __builtin_bit_cast(float, xt[UL * TP]);
                if constexpr (UL == 2) {
                    if constexpr (AFF) aff_acc32(ct[0], ct[1], xt, xt + TP, a, km);
                    else tern_acc32(ct[0], ct[1], xt, xt + TP, a, km);
                } else if constexpr (VARIANT == TQ_TERNARY) {
                    tern_acc16(ct, xt, a, km);
                } else if constexpr (AFF) {
                    aff_acc16(ct, xt, a, km);
                } else {
                    bin_slots(ct, xt, 11, 6, a, km);
                    bin_slots(ct << 6, xt, 5, 6, a, km);
                    bin_slots(ct >> 4, xt, 15, 4, a, km);
                }
                acc = __builtin_fmaf(half_bits(st >> hsh_t), a, acc);
                if constexpr (AFF)
                    acc = __builtin_fmaf(half_bits(bt >> hsh_t), __builtin_bit_cast(float, xt[UL * TP + 1]), acc);
                if constexpr (decltype(refill)::value) load_tail();
                __builtin_amdgcn_sched_barrier(0);
            }
            const float out = seg_sum<LPR>(acc) * XU::kRowScale;
            const int rr = bb * RS + seg;
            if (j == 0 && rr < N) y[rr] = out;
        };
        using Refill = std::integral_constant<bool, true>;
        using Last = std::integral_constant<bool, false>;
        using First = std::integral_constant<bool, true>;
        using Later = std::integral_constant<bool, false>;
        int k = 0;
        if (nb > 1) {
            block(Refill{}, First{}, ca, sa, ba, b0, b0 + WAVES);
            k = 1;
        } else if (nb == 1) {
            block(Last{}, First{}, ca, sa, ba, b0, 0);
            k = 1;
        }
        for (; k + 1 < nb; ++k) block(Refill{}, Later{}, ca, sa, ba, b0 + k * WAVES, b0 + (k + 1) * WAVES);
        if (k < nb) block(Last{}, Later{}, ca, sa, ba, b0 + k * WAVES, 0);
    } else if constexpr (VARIANT != TQ_BINARY) {
        u32x4 ca[NU][1], cb[NU][1];
        uint32_t sa[NU][1], sb[NU][1];
        uint32_t ba[NU][1] = {}, bb_[NU][1] = {};
        int b = b_begin + wave;
        int row[1] = {min(min(b, b_end - 1) * RS + seg, N - 1)};
        if constexpr (AFF) load_bias<LPR, NU, RAGGED>(biases, row[0], j, CPR, G, ba);
        load_block<VARIANT, LPR, NU, 1, RAGGED>(codes, scales, row, j, CPR, G, ca, sa);
        __builtin_amdgcn_sched_barrier(0);
        stage_x(xr);

        auto block = [&](const u32x4 (&c)[NU][1], const uint32_t (&sv)[NU][1],
                         const uint32_t (&bv)[NU][1], int bb) __attribute__((always_inline)) {
            float acc = 0.0f;
#pragma unroll
            for (int i = 0; i < NU; ++i) {
                chunk_dot_reg<VARIANT>(c[i][0], xr[i], sv[i][0], bv[i][0], acc, km);
                __builtin_amdgcn_sched_barrier(0);
            }
            const float out = seg_sum<LPR>(acc) * XU::kRowScale;
            const int rr = bb * RS + seg;
            if (j == 0 && rr < N) y[rr] = out;
        };
        for (; b < b_end; b += 2 * WAVES) {
            const int b2 = b + WAVES;
            if (b2 < b_end) {
                row[0] = b2 * RS + seg < N ? b2 * RS + seg : N - 1;
                if constexpr (AFF) load_bias<LPR, NU, RAGGED>(biases, row[0], j, CPR, G, bb_);
                load_block<VARIANT, LPR, NU, 1, RAGGED>(codes, scales, row, j, CPR, G, cb, sb);
            }
            block(ca, sa, ba, b);
            if (b2 >= b_end) break;
            const int b3 = b2 + WAVES;
            if (b3 < b_end) {
                row[0] = b3 * RS + seg < N ? b3 * RS + seg : N - 1;
                if constexpr (AFF) load_bias<LPR, NU, RAGGED>(biases, row[0], j, CPR, G, ba);
                load_block<VARIANT, LPR, NU, 1, RAGGED>(codes, scales, row, j, CPR, G, ca, sa);
            }
            block(cb, sb, bb_, b2);
        }
    }
}

struct Config {
    int lpr, nu;
};

// Lanes-per-row x chunks-per-lane shapes, smallest capacity first.
constexpr Config kConfigs[] = {{8, 1},  {16, 1}, {8, 2},  {16, 2}, {16, 3}, {8, 5},
                               {16, 4}, {16, 5}, {32, 3}, {16, 6}, {32, 4}, {32, 5},
                               {32, 6}, {64, 4}, {64, 5}, {64, 6}, {64, 8}, {64, 12},
                               {64, 16}};

// The shape with the least capacity that covers CPR chunks; among equal
// capacities the one with fewer chunks per lane.
Config pick(int cpr) {
    Config best{0, 0};
    for (const Config &c : kConfigs) {
        const int cap = c.lpr * c.nu;
        if (cap < cpr) continue;
        if (!best.lpr || cap < best.lpr * best.nu || (cap == best.lpr * best.nu && c.nu < best.nu))
            best = c;
    }
    return best;
}

// Rows per lane and waves per workgroup.  One row per lane and eight waves
// (two per SIMD) give each wave several blocks to pipeline; fewer, larger
// blocks per wave (two rows per lane, twelve waves) leave the first blocks'
// latency exposed and measured slower on every shape.
template <int NU>
struct Tiling {
    static constexpr int RPL = 1;
    static constexpr int WAVES = 8;
};

template <int VARIANT, int LPR, int NU>
constexpr size_t lds_bytes() {
    return (size_t)LPR * NU * XUnit<VARIANT>::CHUNK_DW * sizeof(uint32_t);
}

// Compute units of the current device, cached per device.
int device_cus() {
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cache[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cache[dev] = n;
    }
    return cache[dev];
}

template <int VARIANT, int LPR, int NU>
hipError_t launch(const uint8_t *codes, const uint16_t *scales, const uint16_t *x, float *y, int N,
                  int K, hipStream_t stream) {
    constexpr int RPL = Tiling<NU>::RPL, WAVES = Tiling<NU>::WAVES;
    constexpr int rows_per_block = (64 / LPR) * RPL;
    const int nblocks = (N + rows_per_block - 1) / rows_per_block;
    // one workgroup per CU, but never more workgroups than waves' worth of blocks
    const int grid = max(1, min(device_cus(), (nblocks + WAVES - 1) / WAVES));
    constexpr size_t lds = lds_bytes<VARIANT, LPR, NU>();
    const int cpr = (K / 128) * (VARIANT == TQ_TERNARY ? 2 : 1);
    if (cpr == LPR * NU)
        hipLaunchKernelGGL((gemv_kernel<VARIANT, LPR, NU, RPL, WAVES, false>), dim3(grid),
                           dim3(64 * WAVES), lds, stream, codes, scales, x, y, N, K);
    else
        hipLaunchKernelGGL((gemv_kernel<VARIANT, LPR, NU, RPL, WAVES, true>), dim3(grid),
                           dim3(64 * WAVES), lds, stream, codes, scales, x, y, N, K);
    return hipGetLastError();
}

template <int VARIANT>
hipError_t dispatch(const Config &c, const uint8_t *codes, const uint16_t *scales,
                    const uint16_t *x, float *y, int N, int K, hipStream_t s, size_t *lds) {
#define TQ_CASE(L, U)                                                       \
    if (c.lpr == L && c.nu == U) {                                          \
        *lds = lds_bytes<VARIANT, L, U>();                                  \
        if (*lds > kMaxLds) return hipErrorInvalidValue;                    \
        return launch<VARIANT, L, U>(codes, scales, x, y, N, K, s);        \
    }
    TQ_CASE(8, 1) TQ_CASE(16, 1) TQ_CASE(8, 2) TQ_CASE(16, 2) TQ_CASE(16, 3) TQ_CASE(8, 5)
    TQ_CASE(16, 4) TQ_CASE(16, 5) TQ_CASE(32, 3) TQ_CASE(16, 6) TQ_CASE(32, 4) TQ_CASE(32, 5)
    TQ_CASE(32, 6) TQ_CASE(64, 4) TQ_CASE(64, 5) TQ_CASE(64, 6) TQ_CASE(64, 8) TQ_CASE(64, 12)
    TQ_CASE(64, 16)
#undef TQ_CASE
    return hipErrorInvalidValue;
}

}  // namespace

namespace {

// Register-resident activations: (LPR, NU) with NU <= kXregMaxNU, the least
// capacity LPR * NU that covers CPR chunks, ties to fewer chunks per lane;
// {0, 0} when no shape fits.
constexpr int kXregMaxNU = 5;
constexpr int kXregWaves = 8;

Config pick_xreg(int cpr) {
    Config best{0, 0};
    for (int lpr : {8, 16, 32, 64})
        for (int nu = 1; nu <= kXregMaxNU; ++nu) {
            const int cap = lpr * nu;
            if (cap < cpr) continue;
            if (!best.lpr || cap < best.lpr * best.nu || (cap == best.lpr * best.nu && nu < best.nu))
                best = Config{lpr, nu};
        }
    return best;
}

template <int VARIANT, int LPR, int NU, int TW = 0>
constexpr size_t lds_bytes_xreg() {
    return (size_t)(LPR * NU + LPR * TW / 64) * XReg<VARIANT>::Unit::CHUNK_DW * sizeof(uint32_t);
}

// A row of exactly LPR NU full chunk columns plus LPR TW / 64 chunks (TW = 16
// or 32 weights per lane: one or two dwords of 2-bit codes or affine levels,
// or one 1-bit dword on the first LPR TW / 32 lanes): codes on the pipelined
// loop take the tail slot instead of an extra, mostly clamped, chunk column.
template <int VARIANT, int LPR, int NU, int TW = 16>
hipError_t launch_xreg_tail(const uint8_t *codes, const uint16_t *scales, const uint16_t *biases,
                            const uint16_t *x, float *y, int N, hipStream_t stream) {
    constexpr int RS = 64 / LPR;
    constexpr int K = (LPR * NU + LPR * TW / 64) * 64;
    const int nblocks = (N + RS - 1) / RS;
    const int grid = max(1, min(device_cus(), (nblocks + kXregWaves - 1) / kXregWaves));
    constexpr size_t lds = lds_bytes_xreg<VARIANT, LPR, NU, TW>();
    hipLaunchKernelGGL((gemv_xreg_kernel<VARIANT, LPR, NU, kXregWaves, false, true, TW>), dim3(grid),
                       dim3(64 * kXregWaves), lds, stream, codes, scales, biases, x, y, N, K);
    return hipGetLastError();
}

template <int VARIANT, int LPR, int NU>
hipError_t launch_xreg(const uint8_t *codes, const uint16_t *scales, const uint16_t *biases,
                       const uint16_t *x, float *y, int N, int K, hipStream_t stream) {
    constexpr int RS = 64 / LPR;
    const int nblocks = (N + RS - 1) / RS;
    const int grid = max(1, min(device_cus(), (nblocks + kXregWaves - 1) / kXregWaves));
    constexpr size_t lds = lds_bytes_xreg<VARIANT, LPR, NU>();
    const bool exact = (K / 128) * 2 == LPR * NU;
    // the pipelined loop reads each scale from its aligned dword: an even
    // group count keeps every row's scales dword aligned
    const bool pipe = (K / 128) % 2 == 0 && (reinterpret_cast<uintptr_t>(scales) & 3) == 0 &&
                      (VARIANT != TQ_AFFINE2 || (reinterpret_cast<uintptr_t>(biases) & 3) == 0);
#define TQ_XL(R, P)                                                                               \
    hipLaunchKernelGGL((gemv_xreg_kernel<VARIANT, LPR, NU, kXregWaves, R, P>), dim3(grid),         \
                       dim3(64 * kXregWaves), lds, stream, codes, scales, biases, x, y, N, K)
    if constexpr (NU >= 2) {
        if (pipe && K == (LPR * (NU - 1) + LPR / 4) * 64)
            return launch_xreg_tail<VARIANT, LPR, NU - 1, 16>(codes, scales, biases, x, y, N, stream);
        if (pipe && K == (LPR * (NU - 1) + LPR / 2) * 64)
            return launch_xreg_tail<VARIANT, LPR, NU - 1, 32>(codes, scales, biases, x, y, N, stream);
    }
    // Few rows: a shape with several rows per wave block leaves at least half
    // the waves without a block, where one row per block over 64 lanes (full
    // columns plus the tail slot) gives every wave work: 1024 x 5120
    // 4.06 -> 2.93 us, 2048 x 5120 4.17 -> 3.12, 4096 x 5120 4.43 -> 3.95,
    // 2048 x 9216 4.55 -> 3.71.  From 6144 rows (three quarters of the waves
    // busy) the 64-lane rows, with their longer row sums, measured slower.
    // At most one block per wave on 16 lanes per row (5120-wide rows: 4096 to
    // 8192 rows): 32 lanes per row (two full columns and a 32-weight tail)
    // halve the activation registers and give waves two blocks.  Two runs,
    // same process: 2-bit 4100 x 5120 4.47 -> 3.84 us, 5120 x 5120 4.64 ->
    // 4.22, 6144 x 5120 4.75 -> 4.31, 8192 x 5120 within 1 %; affine 6144
    // and 8192 rows 5.06 -> 4.42 and 5.22 -> 4.97; 1-bit 6144 rows 4.37 ->
    // 4.12 but 8192 rows (exactly one block per wave) 4.46 -> 4.81, so 1-bit
    // codes stop below one block per wave.  12288 rows measured 0.5 us slower.
    if constexpr (LPR == 16) {
        const int nb = (N + RS - 1) / RS, waves = kXregWaves * device_cus();
        if (pipe && K == (32 * 2 + 16) * 64 && nb > waves / 2 &&
            (VARIANT == TQ_BINARY ? nb < waves : nb <= waves))
            return launch_xreg_tail<VARIANT, 32, 2, 32>(codes, scales, biases, x, y, N, stream);
    }
    if constexpr (LPR < 64) {
        if (pipe && (N + RS - 1) / RS <= kXregWaves / 2 * device_cus()) {
            switch (K) {
#define TQ_XT(n, tw) \
    case (64 * n + tw) * 64: return launch_xreg_tail<VARIANT, 64, n, tw>(codes, scales, biases, x, y, N, stream);
                TQ_XT(1, 16) TQ_XT(2, 16) TQ_XT(3, 16) TQ_XT(1, 32) TQ_XT(2, 32) TQ_XT(3, 32)
#undef TQ_XT
                default: break;
            }
        }
    }
    if constexpr (VARIANT == TQ_TERNARY) {
        if (pipe && exact) TQ_XL(false, true);
        else if (pipe) TQ_XL(true, true);
        else TQ_XL(true, false);
    } else if constexpr (VARIANT == TQ_BINARY) {
        if (!pipe) return hipErrorInvalidValue;  // the caller checks: never taken
        if (exact) TQ_XL(false, true);
        else TQ_XL(true, true);
    } else {
        if (pipe && exact) TQ_XL(false, true);
        else if (pipe) TQ_XL(true, true);
        else TQ_XL(true, false);
    }
#undef TQ_XL
    return hipGetLastError();
}

template <int VARIANT>
hipError_t dispatch_xreg(const Config &c, const uint8_t *codes, const uint16_t *scales,
                         const uint16_t *biases, const uint16_t *x, float *y, int N, int K,
                         hipStream_t s) {
#define TQ_XCASE(L)                                                                            \
    if (c.lpr == L) switch (c.nu) {                                                            \
        case 1: return launch_xreg<VARIANT, L, 1>(codes, scales, biases, x, y, N, K, s);       \
        case 2: return launch_xreg<VARIANT, L, 2>(codes, scales, biases, x, y, N, K, s);       \
        case 3: return launch_xreg<VARIANT, L, 3>(codes, scales, biases, x, y, N, K, s);       \
        case 4: return launch_xreg<VARIANT, L, 4>(codes, scales, biases, x, y, N, K, s);       \
        case 5: return launch_xreg<VARIANT, L, 5>(codes, scales, biases, x, y, N, K, s);       \
    }
    TQ_XCASE(8) TQ_XCASE(16) TQ_XCASE(32) TQ_XCASE(64)
#undef TQ_XCASE
    return hipErrorInvalidValue;
}

}  // namespace

namespace {

// ---------------------------------------------------------------------------
// Small-batch GEMM on the VALU: the LDS-activation GEMV above with up to MC
// activation rows.  A code dword is decoded into its slot values once (the
// mask ops of tern_acc32 / bin_slots) and each value meets the MC rows with
// one v_dot2 apiece, so 16 ternary weights cost about 10 + 8 MC VALU ops
// instead of padding a two-row batch to the 16-row MFMA operand.  The
// activations of row m sit in LDS as pair quads
// xq[(m * QPC + q) * CAP + c] (quad q of chunk c, consecutive chunks
// adjacent, so the LPR lanes of a weight row read consecutive 16 bytes) and a
// seed per (row, chunk); rows m >= M and chunks past the row are zeros and
// add exactly nothing.
template <int VARIANT>
struct MCol {
    using XU = XUnit<VARIANT>;                        // 4 units per 16-byte chunk
    static constexpr int UNIT = XU::UNIT;             // weights per unit: 16 or 32
    static constexpr int QPU = UNIT / 8;              // pair quads per unit: 2 or 4
    static constexpr int QPC = 4 * QPU;               // pair quads per chunk: 8 or 16
    static constexpr int CPG = VARIANT == TQ_BINARY ? 1 : 2;  // chunks per group
};

template <int VARIANT, int MC, int LPR, int NU>
constexpr size_t mcol_lds_bytes() {
    return (size_t)MC * LPR * NU * (MCol<VARIANT>::QPC * 16 + 4);
}

// Pairs and the chunk's seed contribution of one staged unit (the pairing of
// XUnit::store), written as quads; lanes holding the 4 units of a chunk are
// 4 aligned consecutive lanes, so the seed reduces with seg_sum<4>.
template <int VARIANT, int CAP>
__device__ __forceinline__ void mcol_store(const XUnit<VARIANT> &xu, u32x4 *xq, float *xseed, int m,
                                           int u, bool real) {
    using MF = MCol<VARIANT>;
    constexpr int UNIT = MF::UNIT, V4 = UNIT / 8;
    uint32_t xp[UNIT / 2];
#pragma unroll
    for (int i = 0; i < UNIT / 4; ++i) {
        const uint32_t l = xu.v[i / 4][i % 4], h = xu.v[V4 / 2 + i / 4][i % 4];
        xp[2 * i] = real ? (l & 0xFFFFu) | (h << 16) : 0u;
        xp[2 * i + 1] = real ? (l >> 16) | (h & 0xFFFF0000u) : 0u;
    }
    float z = 0.0f;
#pragma unroll
    for (int i = 0; i < UNIT / 2; ++i) z = dot2(xp[i], XUnit<VARIANT>::zweight(i), z);
    const int c = u / 4, k = u % 4;
#pragma unroll
    for (int qq = 0; qq < MF::QPU; ++qq)
        xq[(m * MF::QPC + k * MF::QPU + qq) * CAP + c] =
            u32x4{xp[4 * qq], xp[4 * qq + 1], xp[4 * qq + 2], xp[4 * qq + 3]};
    z = seg_sum<4>(z) * -XUnit<VARIANT>::kSeedScale;
    if (k == 0) xseed[m * CAP + c] = z;
}

// One code dword (16 ternary or 32 binary weights) against MC rows of pairs
// xp[m][...] (unit-local pair order), accumulated into a[m].
template <int VARIANT, int MC>
__device__ __forceinline__ void mcol_dword(uint32_t d, const uint32_t (&xp)[MC][MCol<VARIANT>::UNIT / 2],
                                           float (&a)[MC], const Masks &k) {
    if constexpr (VARIANT == TQ_TERNARY) {
        const uint32_t c6 = d << 6, r4 = d >> 4;
        // slot values (pair p in the low half, p + 8 in the high half), as in tern_acc32
        const uint32_t w[8] = {(c6 & k.m6) | 0x14001400u, (c6 & k.m8) | 0x0C000C00u, c6 & 0x0C000C00u,
                               (d & k.m6) | 0x14001400u,  (d & k.m8) | 0x0C000C00u,  d & 0x0C000C00u,
                               (r4 & k.m8) | 0x0C000C00u, r4 & 0x0C000C00u};
#pragma unroll
        for (int p = 0; p < 8; ++p)
#pragma unroll
            for (int m = 0; m < MC; ++m) a[m] = dot2(w[p], xp[m][p], a[m]);
    } else {
        // bit slots as in bin_slots: copy d reads bits 11..6 (pairs 11..6),
        // d << 6 bits 5..0 (pairs 5..0), d >> 4 bits 15..12 (pairs 15..12)
        const uint32_t c6 = d << 6, r4 = d >> 4;
        const uint32_t src[3] = {d, c6, r4};
        const int p0[3] = {11, 5, 15}, cnt[3] = {6, 6, 4};
#pragma unroll
        for (int s = 0; s < 3; ++s) {
            const uint32_t c = src[s];
            const uint32_t w[6] = {c & 0x08000800u, (c & k.b10) | 0x08000800u, (c & k.b9) | 0x0C000C00u,
                                   (c & k.b8) | 0x10001000u, (c & k.b7) | 0x14001400u,
                                   (c & k.b6) | 0x18001800u};
#pragma unroll
            for (int b = 0; b < cnt[s]; ++b)
#pragma unroll
                for (int m = 0; m < MC; ++m) a[m] = dot2(w[b], xp[m][p0[s] - b], a[m]);
        }
    }
}

// Persistent workgroups as in gemv_kernel (one per CU, WAVES waves walking a
// contiguous range of row blocks) with the register kernel's pipelined loop:
// one register set of codes, each chunk refilled with the wave's next block
// as soon as it is used.  A block is RPL * 64/LPR weight rows: lane segment
// seg takes rows seg, seg + 64/LPR, ...; every activation quad read from LDS
// serves the RPL rows.  Y[m][n] for m < M.
template <int VARIANT, int MC, int LPR, int NU, int RPL, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void gemm_mcol_kernel(const uint8_t *__restrict__ codes,
                                                               const uint16_t *__restrict__ scales,
                                                               const uint16_t *__restrict__ X,
                                                               float *__restrict__ Y, int M, int N,
                                                               int K) {
    extern __shared__ uint32_t xs[];
    using MF = MCol<VARIANT>;
    using XU = XUnit<VARIANT>;
    constexpr int THREADS = 64 * WAVES, RS = 64 / LPR, RB = RS * RPL, CAP = LPR * NU;
    constexpr int TOTAL = MC * CAP * 4;  // staged units
    constexpr int XMAX = (TOTAL + THREADS - 1) / THREADS;
    constexpr int HP = MF::UNIT / 2;     // pairs per unit (per code dword)
    u32x4 *xq = reinterpret_cast<u32x4 *>(xs);
    float *xseed = reinterpret_cast<float *>(xs + MC * MF::QPC * CAP * 4);
    const int G = K >> 7, CPR = G * MF::CPG;
    const int nunits = CPR * 4;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int seg = lane / LPR, j = lane % LPR;
    const int nblocks = (N + RB - 1) / RB;
    const int b_begin = (int)(((long long)blockIdx.x * nblocks) / gridDim.x);
    const int b_end = (int)(((long long)(blockIdx.x + 1) * nblocks) / gridDim.x);
    const Masks km;
    // 1. activation loads (L2-resident), then the first block's codes
    XU xu[XMAX];
    int xm[XMAX], xu_i[XMAX];
#pragma unroll
    for (int k = 0; k < XMAX; ++k) {
        const int it = min((int)threadIdx.x + k * THREADS, TOTAL - 1);
        xm[k] = it / (CAP * 4);
        xu_i[k] = it % (CAP * 4);
        xu[k].load(X + (size_t)min(xm[k], M - 1) * K, min(xu_i[k], nunits - 1));
    }
    __builtin_amdgcn_sched_barrier(0);
    // one register set: chunk i of the next block is requested as soon as
    // chunk i of this one is used; every load is clamped into the range, so
    // the load order (and the compiler's wait before each chunk) never varies
    const int blast = b_end - 1;
    const int b0 = b_begin + wave;
    const int nb = b0 < b_end ? (b_end - b0 + WAVES - 1) / WAVES : 0;
    int ccol[NU];
#pragma unroll
    for (int i = 0; i < NU; ++i) ccol[i] = min(j + i * LPR, CPR - 1);
    u32x4 ca[NU][RPL];
    uint32_t sa[NU][RPL];
    auto load_chunk = [&](int bb, int i) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < RPL; ++r) {
            const int row = min(min(bb, blast) * RB + r * RS + seg, N - 1);
            sa[i][r] = scales[(size_t)row * G + ccol[i] / MF::CPG];
            ca[i][r] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4 *>(codes + (size_t)row * CPR * 16) + ccol[i]);
        }
    };
#pragma unroll
    for (int i = 0; i < NU; ++i) load_chunk(b0, i);
    __builtin_amdgcn_sched_barrier(0);

    // 2. pairs and seeds into LDS (threads past the last unit redo it; only
    // the first unit of a chunk writes its seed)
#pragma unroll
    for (int k = 0; k < XMAX; ++k)
        mcol_store<VARIANT, CAP>(xu[k], xq, xseed, xm[k], xu_i[k], xu_i[k] < nunits && xm[k] < M);
    __syncthreads();

    auto block = [&](auto refill, int bb, int bn) __attribute__((always_inline)) {
        // the activation reads are the same for every block: an opaque base
        // keeps them inside the loop (hoisted, they would pin NU * 4 * MC * QPU
        // quads in registers across it)
        uint32_t base = 0;
        asm volatile("" : "+v"(base));
        const u32x4 *xqb = xq + base;
        const float *xsb = xseed + base;
        float acc[RPL][MC];
#pragma unroll
        for (int r = 0; r < RPL; ++r)
#pragma unroll
            for (int m = 0; m < MC; ++m) acc[r][m] = 0.0f;
#pragma unroll
        for (int i = 0; i < NU; ++i) {
            const int col = j + i * LPR;  // x slot (zeros past the row)
            float a[RPL][MC];
#pragma unroll
            for (int m = 0; m < MC; ++m) {
                const float sd = xsb[m * CAP + col];
#pragma unroll
                for (int r = 0; r < RPL; ++r) a[r][m] = sd;
            }
#pragma unroll
            for (int dw = 0; dw < 4; ++dw) {
                uint32_t xp[MC][HP];
#pragma unroll
                for (int m = 0; m < MC; ++m)
#pragma unroll
                    for (int qq = 0; qq < MF::QPU; ++qq) {
                        const u32x4 v = xqb[(m * MF::QPC + dw * MF::QPU + qq) * CAP + col];
                        xp[m][4 * qq] = v[0];
                        xp[m][4 * qq + 1] = v[1];
                        xp[m][4 * qq + 2] = v[2];
                        xp[m][4 * qq + 3] = v[3];
                    }
#pragma unroll
                for (int r = 0; r < RPL; ++r) {
                    mcol_dword<VARIANT, MC>(ca[i][r][dw], xp, a[r], km);
                    // one dword's slot values and pairs live at a time: left
                    // free, the compiler sinks the later rows' dot products to
                    // the end of the block and keeps every decoded value for them
#pragma unroll
                    for (int m = 0; m < MC; ++m) asm volatile("" : "+v"(a[r][m]));
                }
            }
#pragma unroll
            for (int r = 0; r < RPL; ++r) {
                const float sc = (float)__builtin_bit_cast(_Float16, (uint16_t)sa[i][r]);
#pragma unroll
                for (int m = 0; m < MC; ++m) acc[r][m] = __builtin_fmaf(sc, a[r][m], acc[r][m]);
            }
            if constexpr (decltype(refill)::value) load_chunk(bn, i);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int r = 0; r < RPL; ++r) {
            const int rr = bb * RB + r * RS + seg;
#pragma unroll
            for (int m = 0; m < MC; ++m) {
                const float out = seg_sum<LPR>(acc[r][m]) * XU::kRowScale;
                if (j == 0 && rr < N && m < M) Y[(size_t)m * N + rr] = out;
            }
        }
    };

    // 3. this wave's blocks, each refilling the register set for the next
    using Refill = std::integral_constant<bool, true>;
    using Last = std::integral_constant<bool, false>;
    int k = 0;
    for (; k + 1 < nb; ++k) block(Refill{}, b0 + k * WAVES, b0 + (k + 1) * WAVES);
    if (k < nb) block(Last{}, b0 + k * WAVES, 0);
}

template <int VARIANT, int MC, int LPR, int NU, int RPL>
hipError_t launch_mcol(const uint8_t *codes, const uint16_t *scales, const uint16_t *X, float *Y,
                       int M, int N, int K, hipStream_t stream) {
    constexpr int WAVES = 8, RB = 64 / LPR * RPL;
    const int nblocks = (N + RB - 1) / RB;
    const int grid = max(1, min(device_cus(), (nblocks + WAVES - 1) / WAVES));
    constexpr size_t lds = mcol_lds_bytes<VARIANT, MC, LPR, NU>();
    static_assert(lds <= kMaxLds, "activation tile above the LDS of a workgroup");
    hipLaunchKernelGGL((gemm_mcol_kernel<VARIANT, MC, LPR, NU, RPL, WAVES>), dim3(grid),
                       dim3(64 * WAVES), lds, stream, codes, scales, X, Y, M, N, K);
    return hipGetLastError();
}

// Shapes (LPR, NU): the least chunk capacity LPR * NU that covers the row and
// whose MC-row activation tile fits the workgroup's LDS.
struct McolShape {
    int lpr, nu;
};
constexpr McolShape kMcolShapes[] = {{8, 5}, {16, 5}, {16, 9}, {32, 5}, {32, 9}, {64, 5}, {64, 9}};
constexpr int kMcolRpl = 2;  // weight rows per lane segment (one at nine chunks per lane)

template <int VARIANT, int MC>
hipError_t dispatch_mcol(int cpr, const uint8_t *codes, const uint16_t *scales, const uint16_t *X,
                         float *Y, int M, int N, int K, hipStream_t s, bool *handled) {
    constexpr size_t per_chunk = (size_t)MC * (MCol<VARIANT>::QPC * 16 + 4);
    for (const McolShape &sh : kMcolShapes) {
        if (sh.lpr * sh.nu < cpr || (size_t)sh.lpr * sh.nu * per_chunk > kMaxLds) continue;
        *handled = true;
#define TQ_MC(L, U)                                                                      \
    if constexpr (mcol_lds_bytes<VARIANT, MC, L, U>() <= kMaxLds)                          \
        if (sh.lpr == L && sh.nu == U)                                                     \
            return launch_mcol<VARIANT, MC, L, U, (U < 9 ? kMcolRpl : 1)>(codes, scales, X, Y, M, N, K, s);
        TQ_MC(8, 5) TQ_MC(16, 5) TQ_MC(16, 9) TQ_MC(32, 5) TQ_MC(32, 9) TQ_MC(64, 5) TQ_MC(64, 9)
#undef TQ_MC
    }
    *handled = false;
    return hipSuccess;
}

}  // namespace

// Small-batch GEMM on the VALU for M = 2 (ternary and binary) where the
// activation tile fits LDS; *handled is false otherwise (the caller then takes
// the MFMA kernels).  From M = 3 the v_dot2 per weight pair and row make this
// kernel VALU-bound above the MFMA kernels: at M = 4 it measured 15.2 us on
// 17408 x 5120 against 13.5 us, with the VALU busy 70 % of the time.
int32_t gemm_mcol_enqueue(const uint8_t *codes, const uint16_t *scales, const uint16_t *X, float *Y,
                          int64_t M, int64_t N, int64_t K, int32_t variant, hipStream_t stream,
                          bool *handled) {
    *handled = false;
    if (M != 2 || (variant != TQ_TERNARY && variant != TQ_BINARY)) return TQ_OK;
    const int cpr = (int)(K / 128) * (variant == TQ_TERNARY ? 2 : 1);
    const int m = (int)M, n = (int)N, k = (int)K;
    const hipError_t e =
        variant == TQ_TERNARY
            ? dispatch_mcol<TQ_TERNARY, 2>(cpr, codes, scales, X, Y, m, n, k, stream, handled)
            : dispatch_mcol<TQ_BINARY, 2>(cpr, codes, scales, X, Y, m, n, k, stream, handled);
    if (e != hipSuccess) return fail(TQ_ERR_HIP, "GEMM launch failed: %s", hipGetErrorString(e));
    return TQ_OK;
}

int32_t gemv_enqueue(const uint8_t *codes, const uint16_t *scales, const uint16_t *x, float *y,
                     int64_t N, int64_t K, int32_t variant, hipStream_t stream) {
    const int cpr = (int)(K / 128) * (variant == TQ_TERNARY ? 2 : 1);
    // register-activation kernel: 64-weight chunks (two per group) for both
    // variants; binary codes only with dword-aligned scales and an even group
    // count (its pipelined loop), else the LDS-activation kernel below
    const Config xc = pick_xreg((int)(K / 128) * 2);
    const bool bin_ok = (K / 128) % 2 == 0 && (reinterpret_cast<uintptr_t>(scales) & 3) == 0;
    if (xc.lpr && (variant == TQ_TERNARY || bin_ok)) {
        const hipError_t e =
            variant == TQ_TERNARY
                ? dispatch_xreg<TQ_TERNARY>(xc, codes, scales, nullptr, x, y, (int)N, (int)K, stream)
                : dispatch_xreg<TQ_BINARY>(xc, codes, scales, nullptr, x, y, (int)N, (int)K, stream);
        if (e != hipSuccess) return fail(TQ_ERR_HIP, "GEMV launch failed: %s", hipGetErrorString(e));
        return TQ_OK;
    }
    const Config c = pick(cpr);
    if (!c.lpr)
        return fail(TQ_ERR_SHAPE, "K=%lld is above the GEMV limit", (long long)K);
    size_t lds = 0;
    hipError_t e = variant == TQ_TERNARY
                       ? dispatch<TQ_TERNARY>(c, codes, scales, x, y, (int)N, (int)K, stream, &lds)
                       : dispatch<TQ_BINARY>(c, codes, scales, x, y, (int)N, (int)K, stream, &lds);
    if (lds > kMaxLds)
        return fail(TQ_ERR_SHAPE, "K=%lld needs %zu bytes of LDS, above %zu", (long long)K, lds,
                    kMaxLds);
    if (e != hipSuccess) return fail(TQ_ERR_HIP, "GEMV launch failed: %s", hipGetErrorString(e));
    return TQ_OK;
}

// Affine 2-bit levels: the register-activation kernel only (K <= 20480, the
// widest shape 64 lanes x 5 chunks of 64 weights).
int32_t gemv_affine_enqueue(const uint8_t *codes, const uint16_t *scales, const uint16_t *biases,
                            const uint16_t *x, float *y, int64_t N, int64_t K, hipStream_t stream) {
    const Config xc = pick_xreg((int)(K / 128) * 2);
    if (!xc.lpr)
        return fail(TQ_ERR_SHAPE, "K=%lld is above the affine GEMV limit 20480", (long long)K);
    const hipError_t e =
        dispatch_xreg<TQ_AFFINE2>(xc, codes, scales, biases, x, y, (int)N, (int)K, stream);
    if (e != hipSuccess) return fail(TQ_ERR_HIP, "GEMV launch failed: %s", hipGetErrorString(e));
    return TQ_OK;
}

}  // namespace tq
