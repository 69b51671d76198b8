// Batch-1 decode GEMV over ternary weights stored five trits per byte, gfx950.
//
// y[n] = sum_g s[n][g] * sum_{j<128} t[n][128g+j] * x[128g+j] with w = s_g * t
// (thakicloud.github.io, "Bonsai 27B: ternary and 1-bit quantization", "How
// the compression works").  The storage is the native ternary packing that
// the model card names as the step after 2-bit slots (aitrends.kr,
// "Ternary-Bonsai-27B-mlx-2bit", "Technical features"): byte b of a group
// holds trits 5b..5b+4 as the base-3 number sum_i (t_{5b+i} + 1) 3^i, 26
// bytes per group (the last one holds three trits), rows padded to 16 bytes.
// That is 1.75 bits per weight with the scale against 2.125 for 2-bit slots.
//
// Two kernels.  The register kernel (gemv5x_kernel, further down: even group
// count, dword-aligned scales, K <= 20480) looks each byte up as 2-bit slot
// codes and decodes them like the 2-bit format, with activations in
// registers.  The table kernel described next (gemv5_kernel) serves the other
// shapes.
//
// Decode.  Base-3 digits do not fall out of shifts and masks, so each code
// byte is looked up in a table in LDS whose 16-byte entry already holds the
// byte's five trits as FP16 {-1, 0, +1}, laid out against the activation
// pairs (x[2i], x[2i+1]) in natural order: a byte at an even position of its
// group starts on a pair boundary (halves t0..t4, 0), one at an odd position
// starts in the middle of a pair (halves 0, t0..t4).  So one lookup and three
// v_dot2_f32_f16 take five weights, with no activation permutation and no
// offset correction (the products t*x are exact).  The lookup address is
// byte * 256 + copy * 16 (+ table offset), built with one v_perm_b32; every
// lane of a 16-lane (or 8-lane) LDS phase reads its own copy of the table,
// which keeps the random lookups free of bank conflicts.
//
// Work split.  A lane owns units of two groups (52 code bytes, 13 dwords,
// dword aligned) of its rows; LPR lanes cover a row and 64/LPR rows make a
// wave-block.  Workgroups are persistent (one per CU) and walk contiguous
// ranges of blocks, with two register sets of codes in flight.  The partial
// sum of each group is scaled once by its FP16 scale; row partials are summed
// across the LPR lanes with DPP moves.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "tq_internal.h"

namespace tq {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4a __attribute__((ext_vector_type(4), aligned(4)));
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

constexpr size_t kMaxLds5 = 163840;
constexpr int kUnitDw = 13;      // code dwords per two-group unit
constexpr int kXUnitDw = 132;    // LDS dwords per unit of x: 128 + 4 (bank spread)

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c,
                                  false);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                                 0xF, 0xF, false));
}

// v + (v of the lane W = 16 or 32 away, within 2W-lane groups) by a
// v_permlane16/32_swap of v with itself (own and partner value, added), on
// the VALU instead of the LDS crossbar of a lane shuffle.
template <int W>
__device__ __forceinline__ float swap_sum(float v) {
    const uint32_t u = __builtin_bit_cast(uint32_t, v);
    const auto e = W == 16 ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                           : __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __builtin_bit_cast(float, (uint32_t)e[0]) + __builtin_bit_cast(float, (uint32_t)e[1]);
}

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

// Table geometry.  16 copies: entry (parity p, byte v, copy c) at
// p * 65536 + v * 256 + c * 16 (128 KiB).  8 copies: v * 256 + p * 128 + c * 16
// (64 KiB; two lanes of a 16-lane phase share a copy).
template <int COPIES>
struct Lut {
    static constexpr int BYTES = 2 * 256 * COPIES * 16;
    static __device__ __forceinline__ uint32_t base(int p, int lane) {
        const uint32_t c = (uint32_t)(lane & (COPIES - 1)) * 16u;
        return COPIES == 16 ? (uint32_t)p * 65536u + c : (uint32_t)p * 128u + c;
    }
    static __device__ __forceinline__ uint32_t addr(int p, int v, int c) {
        return COPIES == 16 ? (uint32_t)(p * 65536 + v * 256 + c * 16)
                            : (uint32_t)(v * 256 + p * 128 + c * 16);
    }
};

// FP16 bits of the trit (c - 1) for a base-3 digit c.
__device__ __forceinline__ uint32_t trit_half(uint32_t c) {
    return c == 0 ? 0xBC00u : (c == 2 ? 0x3C00u : 0u);
}

// Entry for byte value v: even layout (t0 t1 | t2 t3 | t4 0 | 0 0), odd
// layout (0 t0 | t1 t2 | t3 t4 | 0 0).  Bytes 243..255 hold no valid code
// and map to zeros.
__device__ __forceinline__ u32x4 lut_entry(int p, uint32_t v) {
    if (v >= 243u) return u32x4{0u, 0u, 0u, 0u};
    uint32_t h[5];
#pragma unroll
    for (int i = 0; i < 5; ++i) {
        h[i] = trit_half(v % 3u);
        v /= 3u;
    }
    if (p == 0) return u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4], 0u};
    return u32x4{h[0] << 16, h[1] | (h[2] << 16), h[3] | (h[4] << 16), 0u};
}

// Bytes [B0, B1) of one group (26 code bytes starting at byte 26*H of the
// unit's dwords cd) against the group's activation pairs xg (LDS), for RPL
// rows sharing x.  Only the pairs these bytes touch are read.
template <int H, int B0, int B1, int RPL>
__device__ __forceinline__ void bytes_dot(const uint32_t (&cd)[RPL][kUnitDw], const uint32_t *xg,
                                          const char *lut, uint32_t le, uint32_t lo,
                                          float (&a)[RPL]) {
    constexpr int P0 = (5 * B0) / 2 / 4 * 4;                  // first pair, rounded down to 4
    constexpr int P1 = ((5 * B1 + 1) / 2 + 3) / 4 * 4;         // one past the last, rounded up
    constexpr int NP = (P1 < 64 ? P1 : 64) - P0;
    uint32_t X[NP];
#pragma unroll
    for (int q = 0; q < NP / 4; ++q) {
        const u32x4 v = reinterpret_cast<const u32x4 *>(xg + P0)[q];
        X[4 * q] = v[0];
        X[4 * q + 1] = v[1];
        X[4 * q + 2] = v[2];
        X[4 * q + 3] = v[3];
    }
    // every lookup of the span is issued before the first use, so the LDS
    // latency is paid once per span rather than once per byte
    u32x4 E[RPL][B1 - B0];
#pragma unroll
    for (int b = B0; b < B1; ++b) {
        const int q = 26 * H + b;
        // result bytes: [base.b0, code byte, base.b2, 0]
        constexpr uint32_t kSelHi = 0x0C020000u;
        const uint32_t sel = kSelHi | ((uint32_t)(4 + (q & 3)) << 8);
#pragma unroll
        for (int r = 0; r < RPL; ++r) {
            const uint32_t ad = __builtin_amdgcn_perm(cd[r][q >> 2], (b & 1) ? lo : le, sel);
            E[r][b - B0] = *reinterpret_cast<const u32x4 *>(lut + ad);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int b = B0; b < B1; ++b) {
        const int x0 = ((b & 1) ? (5 * b - 1) / 2 : 5 * b / 2) - P0;
#pragma unroll
        for (int r = 0; r < RPL; ++r) {
            const u32x4 e = E[r][b - B0];
            a[r] = dot2(e[0], X[x0], a[r]);
            a[r] = dot2(e[1], X[x0 + 1], a[r]);
            if (b != 25) a[r] = dot2(e[2], X[x0 + 2], a[r]);
        }
    }
}

template <int H, int RPL>
__device__ __forceinline__ void group_dot(const uint32_t (&cd)[RPL][kUnitDw], const uint32_t *xg,
                                          const char *lut, uint32_t le, uint32_t lo,
                                          float (&a)[RPL]) {
    bytes_dot<H, 0, 7, RPL>(cd, xg, lut, le, lo, a);
    __builtin_amdgcn_sched_barrier(0);
    bytes_dot<H, 7, 13, RPL>(cd, xg, lut, le, lo, a);
    __builtin_amdgcn_sched_barrier(0);
    bytes_dot<H, 13, 20, RPL>(cd, xg, lut, le, lo, a);
    __builtin_amdgcn_sched_barrier(0);
    bytes_dot<H, 20, 26, RPL>(cd, xg, lut, le, lo, a);
}

__device__ __forceinline__ float half_f(uint32_t bits) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

// Loads for one block: per row r and unit slot i, the unit's 13 code dwords
// (group 0: bytes 0..27, group 1: bytes 28..51) and its two group scales.
// RAGGED clamps the last unit slot (the only one that can lie past the row:
// the host picks shapes with (NU - 1) * LPR <= units) to the last unit, and
// when a unit has no second group (an odd group count) reads group 1's dwords
// from the unit's start instead of past the row; those slots meet zero
// activations and contribute nothing.
template <int LPR, int NU, int RPL, bool RAGGED>
__device__ __forceinline__ void load_block5(const uint8_t *__restrict__ codes,
                                            const uint16_t *__restrict__ scales,
                                            const int (&row)[RPL], int j, int U, int G, int rbytes,
                                            uint32_t (&c)[NU][RPL][kUnitDw],
                                            uint32_t (&s)[NU][RPL]) {
    // the unit's two scales in one register (group 2u low, 2u + 1 high); an
    // even group count keeps every pair 4-byte aligned
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
        const uint16_t *sp = scales + (size_t)row[r] * G;
#pragma unroll
        for (int i = 0; i < NU; ++i) {
            const int u = (RAGGED && i == NU - 1) ? min(j + i * LPR, U - 1) : j + i * LPR;
            if (RAGGED)
                s[i][r] = (uint32_t)sp[2 * u] | ((uint32_t)sp[min(2 * u + 1, G - 1)] << 16);
            else
                s[i][r] = reinterpret_cast<const uint32_t *>(sp)[u];
        }
    }
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
        const uint8_t *rp = codes + (size_t)row[r] * rbytes;
#pragma unroll
        for (int i = 0; i < NU; ++i) {
            const int u = (RAGGED && i == NU - 1) ? min(j + i * LPR, U - 1) : j + i * LPR;
            const uint8_t *up = rp + 52 * u;
            const uint8_t *up1 = (!RAGGED || 2 * u + 1 < G) ? up + 28 : up;
            const u32x4a v0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4a *>(up));
            const u32x4a v1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4a *>(up + 12));
            const u32x4a v2 = __builtin_nontemporal_load(reinterpret_cast<const u32x4a *>(up1));
            const u32x4a v3 = __builtin_nontemporal_load(reinterpret_cast<const u32x4a *>(up1 + 8));
            // bytes 0..15 | 12..27 | 28..43 | 36..51
            c[i][r][0] = v0[0];
            c[i][r][1] = v0[1];
            c[i][r][2] = v0[2];
            c[i][r][3] = v1[0];
            c[i][r][4] = v1[1];
            c[i][r][5] = v1[2];
            c[i][r][6] = v1[3];
            c[i][r][7] = v2[0];
            c[i][r][8] = v2[1];
            c[i][r][9] = v2[2];
            c[i][r][10] = v3[1];
            c[i][r][11] = v3[2];
            c[i][r][12] = v3[3];
        }
    }
}

template <int CAP>
constexpr int copies_for() {
    return (size_t)Lut<16>::BYTES + (size_t)CAP * kXUnitDw * 4 <= kMaxLds5 ? 16 : 8;
}

template <int LPR, int NU>
constexpr size_t lds5_bytes() {
    return (size_t)Lut<copies_for<LPR * NU>()>::BYTES + (size_t)LPR * NU * kXUnitDw * 4;
}

template <int LPR, int NU, int RPL, int WAVES, bool RAGGED>
__global__ __launch_bounds__(64 * WAVES) void gemv5_kernel(const uint8_t *__restrict__ codes,
                                                           const uint16_t *__restrict__ scales,
                                                           const uint16_t *__restrict__ x,
                                                           float *__restrict__ y, int N, int K) {
    extern __shared__ u32x4 lds5[];
    constexpr int THREADS = 64 * WAVES;
    constexpr int CAP = LPR * NU;
    constexpr int COPIES = copies_for<CAP>();
    using L = Lut<COPIES>;
    constexpr int RS = 64 / LPR;
    constexpr int RB = RS * RPL;
    constexpr int XV = CAP * kXUnitDw / 4;             // 16-byte x slots in LDS
    constexpr int XPER = (XV + THREADS - 1) / THREADS;
    char *lut = reinterpret_cast<char *>(lds5);
    uint32_t *xs = reinterpret_cast<uint32_t *>(lut + L::BYTES);
    const int G = K >> 7, U = (G + 1) >> 1;
    const int rbytes = (26 * G + 15) & ~15;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int seg = lane / LPR, j = lane % LPR;
    const int nblocks = (N + RB - 1) / RB;
    const int b_begin = (int)(((long long)blockIdx.x * nblocks) / gridDim.x);
    const int b_end = (int)(((long long)(blockIdx.x + 1) * nblocks) / gridDim.x);

    // 1. x into registers: LDS slot v of unit u holds x dwords 4(v%33).. of
    // that unit (slots 32 of each unit are padding); zero past K
    const int xdw = K >> 1;  // x dwords
    u32x4 xv[XPER];
#pragma unroll
    for (int k = 0; k < XPER; ++k) {
        const int v = threadIdx.x + k * THREADS;
        const int u = v / (kXUnitDw / 4), w = v % (kXUnitDw / 4);
        const int d = u * 128 + 4 * w;
        xv[k] = (v < XV && w < 32 && d < xdw) ? reinterpret_cast<const u32x4 *>(x)[d >> 2]
                                             : u32x4{0u, 0u, 0u, 0u};
    }
    __builtin_amdgcn_sched_barrier(0);

    // 2. the first block's codes and scales
    uint32_t ca[NU][RPL][kUnitDw], cb[NU][RPL][kUnitDw];
    uint32_t sa[NU][RPL], sb[NU][RPL];
    int row[RPL];
    auto rows_of = [&](int bb) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < RPL; ++r) row[r] = min(bb * RB + r * RS + seg, N - 1);
    };
    int b = b_begin + wave;
    rows_of(min(b, b_end - 1));
    load_block5<LPR, NU, RPL, RAGGED>(codes, scales, row, j, U, G, rbytes, ca, sa);
    __builtin_amdgcn_sched_barrier(0);

    // 3. the lookup tables, every copy
    for (int e = threadIdx.x; e < 512; e += THREADS) {
        const int p = e >> 8, v = e & 255;
        const u32x4 ent = lut_entry(p, (uint32_t)v);
#pragma unroll
        for (int c = 0; c < COPIES; ++c)
            *reinterpret_cast<u32x4 *>(lut + L::addr(p, v, c)) = ent;
    }
    // 4. x into LDS
#pragma unroll
    for (int k = 0; k < XPER; ++k) {
        const int v = threadIdx.x + k * THREADS;
        if (v < XV) reinterpret_cast<u32x4 *>(xs)[v] = xv[k];
    }
    __syncthreads();

    const uint32_t le = L::base(0, lane), lo = L::base(1, lane);
    auto block = [&](const uint32_t (&c)[NU][RPL][kUnitDw], const uint32_t (&sv)[NU][RPL],
                     int bb) __attribute__((always_inline)) {
        float acc[RPL];
#pragma unroll
        for (int r = 0; r < RPL; ++r) acc[r] = 0.0f;
#pragma unroll
        for (int i = 0; i < NU; ++i) {
            const uint32_t *xu = xs + (j + i * LPR) * kXUnitDw;
            float a0[RPL], a1[RPL];
#pragma unroll
            for (int r = 0; r < RPL; ++r) a0[r] = a1[r] = 0.0f;
            group_dot<0, RPL>(c[i], xu, lut, le, lo, a0);
            group_dot<1, RPL>(c[i], xu + 64, lut, le, lo, a1);
#pragma unroll
            for (int r = 0; r < RPL; ++r) {
                acc[r] = __builtin_fmaf(half_f(sv[i][r] & 0xFFFFu), a0[r], acc[r]);
                acc[r] = __builtin_fmaf(half_f(sv[i][r] >> 16), a1[r], acc[r]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int r = 0; r < RPL; ++r) {
            const float out = seg_sum<LPR>(acc[r]);
            const int rr = bb * RB + r * RS + seg;
            if (j == 0 && rr < N) y[rr] = out;
        }
    };
    for (; b < b_end; b += 2 * WAVES) {
        const int b2 = b + WAVES;
        if (b2 < b_end) {
            rows_of(b2);
            load_block5<LPR, NU, RPL, RAGGED>(codes, scales, row, j, U, G, rbytes, cb, sb);
        }
        block(ca, sa, b);
        if (b2 >= b_end) break;
        const int b3 = b2 + WAVES;
        if (b3 < b_end) {
            rows_of(b3);
            load_block5<LPR, NU, RPL, RAGGED>(codes, scales, row, j, U, G, rbytes, ca, sa);
        }
        block(cb, sb, b2);
    }
}

// ---------------------------------------------------------------------------
// Register-activation kernel (the common case: even group count, dword-aligned
// scales, K <= 20480).
//
// A chunk is half a group: bytes 13s .. 13s + 12 of group g (s = 0, 1), trits
// 65s + 5k + i of the group for byte k, digit i.  Each code byte is looked up
// in a 64 KiB LDS table whose 32-bit entry holds the byte's five digits as
// 2-bit slots (digit i at bits [2i, 2i+2)); entry v of lane l sits at
// (v * 64 + l) * 4, so the 64 lanes of a lookup hit 64 different banks.  Two
// entries merge into one dword (bytes 2q and 2q + 1: low and high half), and
// the dword is decoded exactly as the 2-bit ternary slots are: copy d gives
// slot 4 (M4, bits [8,10) under exponent 3) and slot 3 (M16, bits [6,8) under
// exponent 5); copy d << 6 gives slot 2 (E, bits [10,12)), slot 1 (M4) and
// slot 0 (M16).  The chunk's 13th byte fills the low half of a seventh dword.
// Against it stand activation pairs (x[t], x[t + 5]) for t = 65s + 10q + i, or
// (x[65s + 60 + i], 0) for the 13th byte, with zeros past the group's 128
// trits; the chunk constant -(sum over the pairs of (1 + offset) (x_lo + x_hi))
// * 2^-14 removes the slot offsets and the t = c - 1 shift.  Lanes keep their
// chunks' 35 pairs and constant in registers; loads are unconditional
// (clamped) refills, as in the 2-bit ternary kernel's pipelined loop.
constexpr int kC5Pairs = 33;                 // pair dwords per chunk (6 dwords x 5 slots + 3)
constexpr int kC5SlotDw = 36;                // LDS dwords per chunk slot: pairs, constant, pad
constexpr int kLut5Bytes = 256 * 64 * 4;     // 64 KiB table, one copy per lane
constexpr int kC5MaxNU = 5;

// Digits of byte v as 2-bit slots; bytes above 242 hold no code and map to 0.
__device__ __forceinline__ uint32_t slot_codes(uint32_t v) {
    if (v >= 243u) return 0u;
    uint32_t r = 0;
#pragma unroll
    for (int i = 0; i < 5; ++i) {
        r |= (v % 3u) << (2 * i);
        v /= 3u;
    }
    return r;
}

// FP16 pair (1 + offset, 1 + offset) of slot i: M16 slots 0 and 3 (17), M4
// slots 1 and 4 (5), E slot 2 (1).
__device__ __forceinline__ uint32_t c5_zweight(int i) {
    return (i == 0 || i == 3) ? 0x4C404C40u : (i == 1 || i == 4) ? 0x45004500u : 0x3C003C00u;
}

// The 35 decoded slots of one chunk against its registers, into a (units of
// 2^-14).  w is the chunk's 16-byte window and off the chunk's byte offset in
// it; lbase is lane * 4.
__device__ __forceinline__ void c5_chunk(const u32x4 &w, uint32_t off, const uint32_t (&xr)[kC5Pairs],
                                         const char *lut, uint32_t lbase, float &a,
                                         uint32_t m8, uint32_t m6) {
    const uint32_t w0 = __builtin_amdgcn_alignbyte(w[1], w[0], off);
    const uint32_t w1 = __builtin_amdgcn_alignbyte(w[2], w[1], off);
    const uint32_t w2 = __builtin_amdgcn_alignbyte(w[3], w[2], off);
    const uint32_t w3 = __builtin_amdgcn_alignbyte(w[3], w[3], off);
    const uint32_t wd[4] = {w0, w1, w2, w3};
    // addresses bytes: [lane * 4, code byte k, 0, 0] = byte * 256 + lane * 4
    uint32_t ad[13];
#pragma unroll
    for (int k = 0; k < 13; ++k)
        ad[k] = __builtin_amdgcn_perm(wd[k >> 2], lbase, 0x0C0C0000u | ((uint32_t)(4 + (k & 3)) << 8));
    // bytes 2q and 2q + 1 read straight into the low and high half of one
    // register (the entries fit in 16 bits): the merge costs no VALU op
    uint32_t dq[6];
#pragma unroll
    for (int q = 0; q < 6; ++q) {
        u16x2 v;
        v.x = *reinterpret_cast<const uint16_t *>(lut + ad[2 * q]);
        v.y = *reinterpret_cast<const uint16_t *>(lut + ad[2 * q + 1]);
        dq[q] = __builtin_bit_cast(uint32_t, v);
    }
    const uint32_t e12 = *reinterpret_cast<const uint16_t *>(lut + ad[12]);
#pragma unroll
    for (int q = 0; q < 6; ++q) {
        const uint32_t d = dq[q];
        const uint32_t c6 = d << 6;
        const uint32_t *xp = xr + 5 * q;
        a = dot2((d & m8) | 0x0C000C00u, xp[4], a);   // M4  slot 4
        a = dot2((d & m6) | 0x14001400u, xp[3], a);   // M16 slot 3
        a = dot2(c6 & 0x0C000C00u, xp[2], a);         // E   slot 2
        a = dot2((c6 & m8) | 0x0C000C00u, xp[1], a);  // M4  slot 1
        a = dot2((c6 & m6) | 0x14001400u, xp[0], a);  // M16 slot 0
    }
    // the 13th byte: the low half keeps all five digits but only slots 0..2
    // are decoded (slots 3, 4 shift to bits [12,16), outside every mask);
    // digits 3, 4 go to the high half's slots 0, 1; three slots of d << 6
    const uint32_t d7 = e12 | ((e12 >> 6) << 16);
    const uint32_t c7 = d7 << 6;
    a = dot2(c7 & 0x0C000C00u, xr[32], a);            // E   slot 2: (x62, 0)
    a = dot2((c7 & m8) | 0x0C000C00u, xr[31], a);     // M4  slot 1: (x61, x64)
    a = dot2((c7 & m6) | 0x14001400u, xr[30], a);     // M16 slot 0: (x60, x63)
}

// dynamic LDS of the register kernel: chunk slots and x (the 64 KiB table is static)
template <int LPR, int NU>
constexpr size_t lds5x_bytes(int K) {
    return (size_t)LPR * NU * kC5SlotDw * 4 + (size_t)K * 2;
}

template <int LPR, int NU, int WAVES, bool RAGGED>
__global__ __launch_bounds__(64 * WAVES) void gemv5x_kernel(const uint8_t *__restrict__ codes,
                                                            const uint16_t *__restrict__ scales,
                                                            const uint16_t *__restrict__ x,
                                                            float *__restrict__ y, int N, int K) {
    // the table is static LDS (offset 0, folded into every lookup's address);
    // the chunk slots and x follow it in dynamic LDS
    __shared__ u32x4 lut5[kLut5Bytes / 16];
    extern __shared__ u32x4 lds5x[];
    constexpr int THREADS = 64 * WAVES;
    constexpr int RS = 64 / LPR;  // rows per block
    constexpr int CAP = LPR * NU;
    char *lut = reinterpret_cast<char *>(lut5);
    uint32_t *xs = reinterpret_cast<uint32_t *>(lds5x);
    uint16_t *xn = reinterpret_cast<uint16_t *>(xs + CAP * kC5SlotDw);
    const int G = K >> 7, CPR = 2 * G;
    const int rbytes = (26 * G + 15) & ~15;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int seg = lane / LPR, j = lane % LPR;
    const int nblocks = (N + RS - 1) / RS;
    const int b_begin = (int)(((long long)blockIdx.x * nblocks) / gridDim.x);
    const int b_end = (int)(((long long)(blockIdx.x + 1) * nblocks) / gridDim.x);
    const int blast = b_end - 1;
    const int b0 = b_begin + wave;
    const int nb = b0 < b_end ? (b_end - b0 + WAVES - 1) / WAVES : 0;

    // chunk column of slot i (clamped into the row when ragged), recomputed
    // where used rather than held: registers are the limit here
    auto hcol = [&](int i) __attribute__((always_inline)) {
        return RAGGED ? min(j + i * LPR, CPR - 1) : j + i * LPR;
    };
    const uint32_t *sc32 = reinterpret_cast<const uint32_t *>(scales);
    auto load_chunk = [&](int bb, int i, u32x4 (&c)[NU], uint32_t (&sv)[NU]) __attribute__((always_inline)) {
        const int r = min(min(bb, blast) * RS + seg, N - 1);
        const int h = hcol(i);
        sv[i] = sc32[((size_t)r * G + (h >> 1)) >> 1];
        c[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4a *>(
            codes + (size_t)r * rbytes + ((13 * h) & ~3)));
    };

    // 1. x (natural order) into registers, the first block's codes
    constexpr int XV = 20480 / 8 / THREADS + 1;        // 16-byte x pieces per thread, K <= 20480
    u32x4 xv[XV];
#pragma unroll
    for (int k = 0; k < XV; ++k) {
        const int v = threadIdx.x + k * THREADS;
        xv[k] = v * 8 < K ? reinterpret_cast<const u32x4 *>(x)[v] : u32x4{0u, 0u, 0u, 0u};
    }
    u32x4 ca[NU];
    uint32_t sa[NU];
#pragma unroll
    for (int i = 0; i < NU; ++i) load_chunk(b0, i, ca, sa);
    __builtin_amdgcn_sched_barrier(0);

    // 2. the 256 table entries, once each, staged where the chunk slots will
    // go (at least 288 dwords, ahead of x), and x into LDS; then every wave
    // copies its 256 / WAVES entries into all 64 lane copies (one broadcast
    // read and one conflict-free write per copy, no arithmetic)
    static_assert(THREADS >= 256 && 256 % WAVES == 0 && LPR * kC5SlotDw >= 256, "table staging");
    if (threadIdx.x < 256) xs[threadIdx.x] = slot_codes(threadIdx.x);
#pragma unroll
    for (int k = 0; k < XV; ++k) {
        const int v = threadIdx.x + k * THREADS;
        if (v * 8 < K) reinterpret_cast<u32x4 *>(xn)[v] = xv[k];
    }
    __syncthreads();
    {
        constexpr int PER = 256 / WAVES;
        const int v0 = wave * PER;
        uint32_t *dst = reinterpret_cast<uint32_t *>(lut) + v0 * 64 + lane;
#pragma unroll
        for (int k = 0; k < PER; k += 4) {
            const u32x4 e = reinterpret_cast<const u32x4 *>(xs + v0)[k / 4];
#pragma unroll
            for (int w = 0; w < 4; ++w) dst[(k + w) * 64] = e[w];
        }
    }
    __syncthreads();

    // 3. chunk slots: eight threads per chunk; thread q < 6 builds the five
    // pairs of byte pair q, thread 6 the three pairs of the 13th byte; the
    // chunk constant is their reduced weighted sum.  Without branches: reads
    // are clamped into x and masked, and the writes that have no pair (thread
    // 6's last two, all of thread 7's) store zeros into the slot's two pad
    // dwords
#pragma unroll
    for (int t0 = 0; t0 < CAP * 8; t0 += THREADS) {
        const int t = t0 + (int)threadIdx.x;
        if (CAP * 8 % THREADS != 0 && t >= CAP * 8) break;
        const int h = t >> 3, q = t & 7;
        const int g = min(h >> 1, G - 1), base = 65 * (h & 1);
        const bool real = h < CPR;
        const int np = q < 6 ? 5 : (q == 6 ? 3 : 0);
        float z = 0.0f;
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            // trits of the pair within the group; >= 128 means none
            const int tl = base + (q < 6 ? 10 * q + i : 60 + i);
            const int th = q < 6 ? base + 10 * q + 5 + i : (i < 2 ? base + 63 + i : 128);
            const bool on = real && i < np;
            const uint32_t lv = xn[g * 128 + min(tl, 127)];
            const uint32_t hv = xn[g * 128 + min(th, 127)];
            const uint32_t lo = (on && tl < 128) ? lv : 0u;
            const uint32_t hi = (on && th < 128) ? hv : 0u;
            const uint32_t pr = lo | (hi << 16);
            z = dot2(pr, c5_zweight(i), z);
            const int d = q < 6 ? 5 * q + i : (q == 6 && i < 3 ? 30 + i : kC5Pairs + 1 + (i & 1));
            xs[h * kC5SlotDw + d] = pr;
        }
        z = seg_sum<8>(z) * -6.103515625e-05f;
        if (q == 7) xs[h * kC5SlotDw + kC5Pairs] = __builtin_bit_cast(uint32_t, z);
    }
    __syncthreads();

    // 4. this lane's chunk pairs into registers (the chunk constants stay in
    // LDS and are read once per block)
    uint32_t xr[NU][kC5Pairs];
#pragma unroll
    for (int i = 0; i < NU; ++i) {
        const uint32_t *slot = xs + (j + i * LPR) * kC5SlotDw;
#pragma unroll
        for (int v = 0; v < kC5SlotDw / 4; ++v) {
            const u32x4 u = reinterpret_cast<const u32x4 *>(slot)[v];
#pragma unroll
            for (int w = 0; w < 4; ++w)
                if (4 * v + w < kC5Pairs) xr[i][4 * v + w] = u[w];
        }
    }

    uint32_t m8 = 0x03000300u, m6 = 0x00C000C0u;
    asm volatile("" : "+v"(m8));
    asm volatile("" : "+v"(m6));
    const uint32_t lbase = (uint32_t)lane * 4u;
    auto block = [&](auto refill, u32x4 (&c)[NU], uint32_t (&sv)[NU], int bb, int bn)
                     __attribute__((always_inline)) {
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < NU; ++i) {
            const int h = hcol(i);
            float a = __builtin_bit_cast(float, xs[(j + i * LPR) * kC5SlotDw + kC5Pairs]);
            c5_chunk(c[i], (uint32_t)h & 3u, xr[i], lut, lbase, a, m8, m6);   // 13 h mod 4
            acc = __builtin_fmaf(half_f(sv[i] >> (((uint32_t)(h >> 1) & 1u) * 16u)), a, acc);
            if constexpr (decltype(refill)::value) load_chunk(bn, i, c, sv);
            __builtin_amdgcn_sched_barrier(0);
        }
        const float out = seg_sum<LPR>(acc) * 16384.0f;
        const int rr = bb * RS + seg;
        if (j == 0 && rr < N) y[rr] = out;
    };
    // one register set: each chunk is refilled with the wave's next block as
    // soon as it is consumed, a block's time ahead of its use (two sets of
    // 16-byte windows do not fit next to 180 activation registers)
    using Refill = std::integral_constant<bool, true>;
    using Last = std::integral_constant<bool, false>;
    int k = 0;
    for (; k + 1 < nb; ++k) block(Refill{}, ca, sa, b0 + k * WAVES, b0 + (k + 1) * WAVES);
    if (k < nb) block(Last{}, ca, sa, b0 + k * WAVES, 0);
}


struct Config5 {
    int lpr, nu;
};

// (lanes per row, units per lane), least capacity first.
// The widest, 160 units (K = 40960), is the most whose activations fit next
// to the 64 KiB table.
constexpr Config5 kConfigs5[] = {{2, 1},  {4, 1},  {8, 1},  {4, 3},  {8, 2},  {4, 5},
                                 {8, 3},  {16, 2}, {8, 5},  {16, 3}, {16, 4}, {16, 5}, {32, 3},
                                 {32, 4}, {32, 5}};
constexpr int64_t kMaxK5 = 160 * 256;

Config5 pick5(int units) {
    Config5 best{0, 0};
    for (const Config5 &c : kConfigs5) {
        const int cap = c.lpr * c.nu;
        if (cap < units || (c.nu - 1) * c.lpr > units) continue;
        if (!best.lpr || cap < best.lpr * best.nu || (cap == best.lpr * best.nu && c.nu < best.nu))
            best = c;
    }
    return best;
}

constexpr int kWaves5 = 8;

int device_cus5() {
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

template <int LPR, int NU>
hipError_t launch5(const uint8_t *codes, const uint16_t *scales, const uint16_t *x, float *y, int N,
                   int K, hipStream_t stream) {
    constexpr int RPL = 1;
    constexpr size_t lds = lds5_bytes<LPR, NU>();
    static_assert(lds <= kMaxLds5, "LDS budget");
    constexpr int rows_per_block = (64 / LPR) * RPL;
    const int nblocks = (N + rows_per_block - 1) / rows_per_block;
    const int grid = max(1, min(device_cus5(), (nblocks + kWaves5 - 1) / kWaves5));
    const int G = K / 128;
    // the exact shape also reads each unit's two scales as one dword
    const bool exact = (G % 2 == 0) && (G / 2 == LPR * NU) &&
                       (reinterpret_cast<uintptr_t>(scales) & 3) == 0;
    if (exact)
        hipLaunchKernelGGL((gemv5_kernel<LPR, NU, RPL, kWaves5, false>), dim3(grid),
                           dim3(64 * kWaves5), lds, stream, codes, scales, x, y, N, K);
    else
        hipLaunchKernelGGL((gemv5_kernel<LPR, NU, RPL, kWaves5, true>), dim3(grid),
                           dim3(64 * kWaves5), lds, stream, codes, scales, x, y, N, K);
    return hipGetLastError();
}

hipError_t dispatch5(const Config5 &c, const uint8_t *codes, const uint16_t *scales,
                     const uint16_t *x, float *y, int N, int K, hipStream_t s) {
#define TQ5_CASE(L, U) \
    if (c.lpr == L && c.nu == U) return launch5<L, U>(codes, scales, x, y, N, K, s);
    TQ5_CASE(2, 1) TQ5_CASE(4, 1) TQ5_CASE(8, 1) TQ5_CASE(4, 3) TQ5_CASE(8, 2)
    TQ5_CASE(4, 5) TQ5_CASE(8, 3) TQ5_CASE(16, 2) TQ5_CASE(8, 5) TQ5_CASE(16, 3) TQ5_CASE(16, 4)
    TQ5_CASE(16, 5) TQ5_CASE(32, 3) TQ5_CASE(32, 4) TQ5_CASE(32, 5)
#undef TQ5_CASE
    return hipErrorInvalidValue;
}

// Register-activation kernel shapes: the least LPR * NU >= chunks per row
// (NU <= 5), ties to fewer chunks per lane; {0, 0} when none fits (K > 20480).
Config5 pick5x(int cpr) {
    Config5 best{0, 0};
    for (int lpr : {8, 16, 32, 64})
        for (int nu = 1; nu <= kC5MaxNU; ++nu) {
            const int cap = lpr * nu;
            if (cap < cpr) continue;
            if (!best.lpr || cap < best.lpr * best.nu || (cap == best.lpr * best.nu && nu < best.nu))
                best = Config5{lpr, nu};
        }
    return best;
}

template <int LPR, int NU>
hipError_t launch5x(const uint8_t *codes, const uint16_t *scales, const uint16_t *x, float *y,
                    int N, int K, hipStream_t stream) {
    constexpr int RS = 64 / LPR;
    const int nblocks = (N + RS - 1) / RS;
    const int grid = max(1, min(device_cus5(), (nblocks + kWaves5 - 1) / kWaves5));
    const size_t lds = lds5x_bytes<LPR, NU>(K);
    if (2 * (K / 128) == LPR * NU)
        hipLaunchKernelGGL((gemv5x_kernel<LPR, NU, kWaves5, false>), dim3(grid), dim3(64 * kWaves5),
                           lds, stream, codes, scales, x, y, N, K);
    else
        hipLaunchKernelGGL((gemv5x_kernel<LPR, NU, kWaves5, true>), dim3(grid), dim3(64 * kWaves5),
                           lds, stream, codes, scales, x, y, N, K);
    return hipGetLastError();
}

hipError_t dispatch5x(const Config5 &c, const uint8_t *codes, const uint16_t *scales,
                      const uint16_t *x, float *y, int N, int K, hipStream_t s) {
#define TQ5X_CASE(L)                                                             \
    if (c.lpr == L) switch (c.nu) {                                              \
        case 1: return launch5x<L, 1>(codes, scales, x, y, N, K, s);             \
        case 2: return launch5x<L, 2>(codes, scales, x, y, N, K, s);             \
        case 3: return launch5x<L, 3>(codes, scales, x, y, N, K, s);             \
        case 4: return launch5x<L, 4>(codes, scales, x, y, N, K, s);             \
        case 5: return launch5x<L, 5>(codes, scales, x, y, N, K, s);             \
    }
    TQ5X_CASE(8) TQ5X_CASE(16) TQ5X_CASE(32) TQ5X_CASE(64)
#undef TQ5X_CASE
    return hipErrorInvalidValue;
}

}  // namespace

int32_t gemv5_enqueue(const uint8_t *codes, const uint16_t *scales, const uint16_t *x, float *y,
                      int64_t N, int64_t K, hipStream_t stream) {
    const int G = (int)(K / 128);
    // register-activation kernel: half-group chunks, scales read as aligned dwords
    if (G % 2 == 0 && (reinterpret_cast<uintptr_t>(scales) & 3) == 0) {
        const Config5 c = pick5x(2 * G);
        if (c.lpr) {
            const hipError_t e = dispatch5x(c, codes, scales, x, y, (int)N, (int)K, stream);
            if (e != hipSuccess) return fail(TQ_ERR_HIP, "GEMV launch failed: %s", hipGetErrorString(e));
            return TQ_OK;
        }
    }
    const int units = (G + 1) / 2;
    const Config5 c = pick5(units);
    if (!c.lpr || K > kMaxK5)
        return fail(TQ_ERR_SHAPE, "K=%lld is above the five-trit GEMV limit %lld", (long long)K,
                    (long long)kMaxK5);
    const hipError_t e = dispatch5(c, codes, scales, x, y, (int)N, (int)K, stream);
    if (e != hipSuccess) return fail(TQ_ERR_HIP, "GEMV launch failed: %s", hipGetErrorString(e));
    return TQ_OK;
}

}  // namespace tq
