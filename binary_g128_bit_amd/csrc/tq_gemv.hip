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
// whose value is linear in the code, without a per-weight normalising op:
//   E: a 2-bit code moved to bits [10,12) of a half (the exponent LSBs, the
//      rest zero) is the FP16 c * 2^-14, exactly (0 for c = 0);
//   M: a code moved to bits [8,10) under an exponent field of 1 is the FP16
//      2^-14 * (1 + c/4): an offset only four times the code's unit.
// One shifted copy of a code dword serves one E pair and one M pair (slot p
// in the low half, slot p + 8 in the high half), so 16 weights cost 3 shifts,
// 8 masks and 8 v_dot2_f32_f16 into two fp32 accumulators.  Per group the
// offsets of the M pairs and sum x (t = c - 1) are removed with one constant
// computed while x is staged:  sum t*x = aE*2^14 + aM*2^16 - (sum x + 4 S_M),
// where S_M sums x over the M slots.  Rounding stays proportional to the
// terms summed: the largest offset is 4x the code unit, so a row of zero
// trits leaves only a residue of order 2^-22 * sum |s * x|.  The 1-bit
// variant uses the same E slot (bit 10) plus two M slots (bits 9 and 8) and
// forms 2 * sum b*x - sum x.
//
// Work split.  A wave owns 64/LPR row slots of LPR lanes each; lane j of a
// slot takes groups j, j+LPR, j+2*LPR, ... of its RPL rows.  Each lane first
// issues its share of the x loads for staging (L2-resident), then every code
// and scale load of its rows, so the workgroup's whole HBM share is in flight
// while x is permuted into LDS; groups are then processed in the order their
// codes arrive.  Per-row partial sums are reduced across the LPR lanes with
// DPP moves (quad_perm, row_half_mirror, row_mirror) and swizzles beyond 16.
#include <hip/hip_runtime.h>

#include "tq_internal.h"

namespace tq {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kXStride = 68;  // dwords per group in LDS: 64 pairs + 4 pad (bank spread)

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c,
                                  false);
}

// Masks used with v_and_or_b32 stay in VGPRs: gfx9 VOP3 encodings take no
// literal and read one SGPR at most, which then holds the exponent constant.
struct Masks {
    uint32_t m8, m9, b8;
    __device__ __forceinline__ Masks() : m8(0x03000300u), m9(0x02000200u), b8(0x01000100u) {
        asm volatile("" : "+v"(m8));
        asm volatile("" : "+v"(m9));
        asm volatile("" : "+v"(b8));
    }
};

constexpr uint32_t kExp1 = 0x04000400u;  // exponent field 1 in both halves

// 16 ternary codes of dword d against pairs xp[p] = (x[p], x[p+8]).
// aE gets c * 2^-14 * x for slots 1, 3, 5, 7; aM gets 2^-14 (1 + c/4) x for
// slots 0, 2, 4, 6.
__device__ __forceinline__ void tern_acc16(uint32_t d, const uint32_t *xp, float &aE, float &aM,
                                           const Masks &k) {
    aE = dot2(d & 0x0C000C00u, xp[5], aE);
    aM = dot2((d & k.m8) | kExp1, xp[4], aM);
    const uint32_t l4 = d << 4, l8 = d << 8, r4 = d >> 4;
    aE = dot2(l4 & 0x0C000C00u, xp[3], aE);
    aM = dot2((l4 & k.m8) | kExp1, xp[2], aM);
    aE = dot2(l8 & 0x0C000C00u, xp[1], aE);
    aM = dot2((l8 & k.m8) | kExp1, xp[0], aM);
    aE = dot2(r4 & 0x0C000C00u, xp[7], aE);
    aM = dot2((r4 & k.m8) | kExp1, xp[6], aM);
}

// 32 binary bits of dword d against pairs xp[p] = (x[p], x[p+16]).
// aE: b * 2^-14 (bit at 10); a9: 2^-14 (1 + b/2) (bit at 9); a8: 2^-14 (1 + b/4).
// Copies d << s for s in {0, 3, 6, 9, -3, -6} bring bits 10-s, 9-s, 8-s there.
__device__ __forceinline__ void bin_acc32(uint32_t d, const uint32_t *xp, float &aE, float &a9,
                                          float &a8, const Masks &k) {
    const uint32_t c0 = d, c3 = d << 3, c6 = d << 6, c9 = d << 9, r3 = d >> 3, r6 = d >> 6;
    aE = dot2(c0 & 0x04000400u, xp[10], aE);
    a9 = dot2((c0 & k.m9) | kExp1, xp[9], a9);
    a8 = dot2((c0 & k.b8) | kExp1, xp[8], a8);
    aE = dot2(c3 & 0x04000400u, xp[7], aE);
    a9 = dot2((c3 & k.m9) | kExp1, xp[6], a9);
    a8 = dot2((c3 & k.b8) | kExp1, xp[5], a8);
    aE = dot2(c6 & 0x04000400u, xp[4], aE);
    a9 = dot2((c6 & k.m9) | kExp1, xp[3], a9);
    a8 = dot2((c6 & k.b8) | kExp1, xp[2], a8);
    aE = dot2(c9 & 0x04000400u, xp[1], aE);
    a9 = dot2((c9 & k.m9) | kExp1, xp[0], a9);
    aE = dot2(r3 & 0x04000400u, xp[13], aE);
    a9 = dot2((r3 & k.m9) | kExp1, xp[12], a9);
    a8 = dot2((r3 & k.b8) | kExp1, xp[11], a8);
    a9 = dot2((r6 & k.m9) | kExp1, xp[15], a9);
    a8 = dot2((r6 & k.b8) | kExp1, xp[14], a8);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                                 0xF, 0xF, false));
}

// Sum over aligned segments of LPR lanes; every lane of a segment gets the sum.
template <int LPR>
__device__ __forceinline__ float seg_sum(float v) {
    if (LPR >= 2) v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
    if (LPR >= 4) v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
    if (LPR >= 8) v += dpp_f<0x141>(v);  // row_half_mirror
    if (LPR >= 16) v += dpp_f<0x140>(v); // row_mirror
    if (LPR >= 32) v += __shfl_xor(v, 16);
    if (LPR >= 64) v += __shfl_xor(v, 32);
    return v;
}

// x staging.  Ternary unit: 16 weights -> 8 pairs (p, p+8); binary unit:
// 32 weights -> 16 pairs (p, p+16).  The UPG units of a group sit in
// consecutive lanes, so their partial constants reduce with seg_sum.  LDS
// holds, per group, 64 pair dwords, then the group constant (a float) at [64].
template <int VARIANT>
struct XUnit {
    static constexpr int UNIT = VARIANT == TQ_TERNARY ? 16 : 32;
    static constexpr int UPG = 128 / UNIT;
    static constexpr int V4 = UNIT / 8;  // 16-byte loads per unit
    u32x4 v[V4];

    // FP16 pair (w, w) weighting pair p in the per-group constant
    static __device__ __forceinline__ uint32_t zweight(int p) {
        if constexpr (VARIANT == TQ_TERNARY) {
            return (p & 1) ? 0x3C003C00u : 0x45004500u;  // 1 : 5
        } else {
            // E slots 1, 4, 7, 10, 13; bit-9 slots 0, 3, 6, 9, 12, 15; bit-8 slots 2, 5, 8, 11, 14
            return (p % 3 == 1) ? 0x3C003C00u : (p % 3 == 0) ? 0x45004500u : 0x48804880u;  // 1 : 5 : 9
        }
    }

    __device__ __forceinline__ void load(const uint16_t *__restrict__ x, int u) {
        const u32x4 *src = reinterpret_cast<const u32x4 *>(x + (size_t)u * UNIT);
#pragma unroll
        for (int i = 0; i < V4; ++i) v[i] = src[i];
    }

    __device__ __forceinline__ void store(uint32_t *xs, int u) const {
        const int g = u / UPG, ug = u % UPG;
        uint32_t xp[UNIT / 2];
        // low halves x[0..UNIT/2), high halves x[UNIT/2..UNIT)
#pragma unroll
        for (int i = 0; i < UNIT / 4; ++i) {
            const uint32_t l = v[i / 4][i % 4], h = v[V4 / 2 + i / 4][i % 4];
            xp[2 * i] = (l & 0xFFFFu) | (h << 16);
            xp[2 * i + 1] = (l >> 16) | (h & 0xFFFF0000u);
        }
        // per-group constant: sum over the pairs of w_p * (x[p] + x[p+UNIT/2]) where
        // w = 1 for E slots and 1 + 4 (ternary M), 1 + 4 (binary bit 9) or
        // 1 + 8 (binary bit 8) for the offset-carrying slots
        float z = 0.0f;
#pragma unroll
        for (int i = 0; i < UNIT / 2; ++i) z = dot2(xp[i], zweight(i), z);
        uint32_t *dst = xs + g * kXStride + ug * (UNIT / 2);
#pragma unroll
        for (int i = 0; i < UNIT / 8; ++i)
            reinterpret_cast<u32x4 *>(dst)[i] = u32x4{xp[4 * i], xp[4 * i + 1], xp[4 * i + 2], xp[4 * i + 3]};
        z = seg_sum<UPG>(z);
        if (ug == 0) xs[g * kXStride + 64] = __builtin_bit_cast(uint32_t, z);
    }
};

template <int VARIANT, int LPR, int GPL, int RPL>
__global__ __launch_bounds__(kThreads) void gemv_kernel(const uint8_t *__restrict__ codes,
                                                        const uint16_t *__restrict__ scales,
                                                        const uint16_t *__restrict__ x,
                                                        float *__restrict__ y, int N, int K) {
    extern __shared__ uint32_t xs[];
    using XU = XUnit<VARIANT>;
    constexpr int RS = 64 / LPR;                       // row slots per wave
    constexpr int DW = VARIANT == TQ_TERNARY ? 8 : 4;  // code dwords per group
    // units of x each thread stages; held in registers when few enough
    constexpr int XMAX = (LPR * GPL * XU::UPG + kThreads - 1) / kThreads;
    constexpr bool XREG = XMAX <= 5;
    const int G = K >> 7;
    const int nunits = G * XU::UPG;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int seg = lane / LPR, j = lane % LPR;
    const Masks km;
    const int row0 = (blockIdx.x * kWaves + wave) * (RS * RPL) + seg;
    const size_t row_bytes = (size_t)K / (VARIANT == TQ_TERNARY ? 4 : 8);

    // All global loads below are unconditional (indices clamped into range) so
    // that the wait counters can be tracked exactly: each use waits only for
    // the loads it needs, never for the whole stream.
    // 1. x loads for staging first (L2-resident, short latency)
    XU xu[XREG ? XMAX : 1];
    if constexpr (XREG) {
#pragma unroll
        for (int k = 0; k < XMAX; ++k) xu[k].load(x, min((int)threadIdx.x + k * kThreads, nunits - 1));
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the x loads ahead of the code loads

    // 2. every code and scale load of this lane; groups past G get scale 0
    uint32_t cw[GPL][RPL][DW];
    uint32_t sb[GPL][RPL];
#pragma unroll
    for (int i = 0; i < GPL; ++i) {
        const int g = min(j + i * LPR, G - 1);
#pragma unroll
        for (int r = 0; r < RPL; ++r) {
            const int row = min(row0 + r * RS, N - 1);
            const u32x4 *p = reinterpret_cast<const u32x4 *>(codes + (size_t)row * row_bytes +
                                                             (size_t)g * (DW * 4));
#pragma unroll
            for (int v = 0; v < DW / 4; ++v) {
                const u32x4 q = __builtin_nontemporal_load(p + v);
#pragma unroll
                for (int w = 0; w < 4; ++w) cw[i][r][4 * v + w] = q[w];
            }
            sb[i][r] = scales[(size_t)row * G + g];
        }
    }
    __builtin_amdgcn_sched_barrier(0);  // staging must not be hoisted above the code loads

    // 3. permute x into LDS with the per-group constants
    if constexpr (XREG) {
        // lanes past the last unit re-store that unit's identical data; its group
        // constant is written only by the lane holding the group's first unit
#pragma unroll
        for (int k = 0; k < XMAX; ++k) xu[k].store(xs, min((int)threadIdx.x + k * kThreads, nunits - 1));
    } else {
        for (int u = threadIdx.x; u < nunits; u += kThreads) {
            xu[0].load(x, u);
            xu[0].store(xs, u);
        }
    }
    __syncthreads();

    // 4. decode, dot, scale -- group by group as the codes land
    float yacc[RPL];
#pragma unroll
    for (int r = 0; r < RPL; ++r) yacc[r] = 0.0f;
#pragma unroll
    for (int i = 0; i < GPL; ++i) {
        const bool live = j + i * LPR < G;
        const uint32_t *xg = xs + min(j + i * LPR, G - 1) * kXStride;
        const float z = __builtin_bit_cast(float, xg[64]);
        float aE[RPL], aM[RPL], a8[RPL];
#pragma unroll
        for (int r = 0; r < RPL; ++r) {
            aE[r] = 0.0f;
            if constexpr (VARIANT == TQ_TERNARY) {
                aM[r] = -z * 1.52587890625e-05f;  // -z * 2^-16
                a8[r] = 0.0f;
            } else {
                aM[r] = 0.0f;
                a8[r] = -z * 7.62939453125e-06f;  // -z * 2^-17
            }
        }
        if constexpr (VARIANT == TQ_TERNARY) {
#pragma unroll
            for (int d = 0; d < 8; ++d) {
                const u32x4 lo = reinterpret_cast<const u32x4 *>(xg + 8 * d)[0];
                const u32x4 hi = reinterpret_cast<const u32x4 *>(xg + 8 * d)[1];
                const uint32_t xp[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
                for (int r = 0; r < RPL; ++r) tern_acc16(cw[i][r][d], xp, aE[r], aM[r], km);
            }
        } else {
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                uint32_t xp[16];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const u32x4 q = reinterpret_cast<const u32x4 *>(xg + 16 * d)[v];
#pragma unroll
                    for (int w = 0; w < 4; ++w) xp[4 * v + w] = q[w];
                }
#pragma unroll
                for (int r = 0; r < RPL; ++r) bin_acc32(cw[i][r][d], xp, aE[r], aM[r], a8[r], km);
            }
        }
#pragma unroll
        for (int r = 0; r < RPL; ++r) {
            float t;
            if constexpr (VARIANT == TQ_TERNARY) {
                t = __builtin_fmaf(aM[r], 65536.0f, aE[r] * 16384.0f);  // aE 2^14 + aM 2^16
            } else {
                t = __builtin_fmaf(aM[r], 65536.0f, aE[r] * 32768.0f);  // aE 2^15 + a9 2^16
                t = __builtin_fmaf(a8[r], 131072.0f, t);                 //   + a8 2^17
            }
            const float s = live ? (float)__builtin_bit_cast(_Float16, (uint16_t)sb[i][r]) : 0.0f;
            yacc[r] = __builtin_fmaf(s, t, yacc[r]);
        }
    }

    // 5. reduce across the LPR lanes of each row slot and store
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
        const float v = seg_sum<LPR>(yacc[r]);
        const int row = row0 + r * RS;
        if (j == 0 && row < N) y[row] = v;
    }
}

struct Config {
    int lpr, gpl, rpl;
};

// Smallest lanes-per-row x groups-per-lane capacity that covers G groups.
Config pick(int G) {
    static const Config table[] = {{8, 1, 1}, {8, 2, 1}, {8, 4, 1}, {8, 5, 1}, {8, 6, 1},
                                   {16, 4, 1}, {32, 5, 1}, {64, 4, 1}};
    for (const Config &c : table)
        if (c.lpr * c.gpl >= G) return c;
    return {0, 0, 0};
}

template <int VARIANT, int LPR, int GPL, int RPL>
hipError_t launch(const uint8_t *codes, const uint16_t *scales, const uint16_t *x, float *y, int N,
                  int K, hipStream_t stream) {
    constexpr int rows_per_block = kWaves * (64 / LPR) * RPL;
    const int G = K / 128;
    const size_t lds = (size_t)G * kXStride * sizeof(uint32_t);
    const unsigned blocks = (unsigned)((N + rows_per_block - 1) / rows_per_block);
    hipLaunchKernelGGL((gemv_kernel<VARIANT, LPR, GPL, RPL>), dim3(blocks), dim3(kThreads), lds,
                       stream, codes, scales, x, y, N, K);
    return hipGetLastError();
}

template <int VARIANT>
hipError_t dispatch(const Config &c, const uint8_t *codes, const uint16_t *scales,
                    const uint16_t *x, float *y, int N, int K, hipStream_t s) {
#define TQ_CASE(L, Gp, R)                                   \
    if (c.lpr == L && c.gpl == Gp && c.rpl == R)             \
        return launch<VARIANT, L, Gp, R>(codes, scales, x, y, N, K, s);
    TQ_CASE(8, 1, 1)
    TQ_CASE(8, 2, 1)
    TQ_CASE(8, 4, 1)
    TQ_CASE(8, 5, 1)
    TQ_CASE(8, 6, 1)
    TQ_CASE(16, 4, 1)
    TQ_CASE(32, 5, 1)
    TQ_CASE(64, 4, 1)
#undef TQ_CASE
    return hipErrorInvalidValue;
}

}  // namespace

// Largest K whose staged x fits the 64 KiB of LDS a workgroup may use.
constexpr int64_t kGemvMaxK = (65536 / (kXStride * 4)) * 128;

int32_t gemv_enqueue(const uint8_t *codes, const uint16_t *scales, const uint16_t *x, float *y,
                     int64_t N, int64_t K, int32_t variant, hipStream_t stream) {
    if (K > kGemvMaxK)
        return fail(TQ_ERR_SHAPE, "K=%lld above the GEMV limit %lld", (long long)K,
                    (long long)kGemvMaxK);
    const Config c = pick((int)(K / 128));
    hipError_t e = variant == TQ_TERNARY
                       ? dispatch<TQ_TERNARY>(c, codes, scales, x, y, (int)N, (int)K, stream)
                       : dispatch<TQ_BINARY>(c, codes, scales, x, y, (int)N, (int)K, stream);
    if (e != hipSuccess) return fail(TQ_ERR_HIP, "GEMV launch failed: %s", hipGetErrorString(e));
    return TQ_OK;
}

}  // namespace tq
