// 4-bit KV cache and decode attention for the full-attention layers, gfx950.
//
// The model keeps K and V of its 16 full-attention layers (4 KV heads of
// dimension 256; 64 KiB per token at FP16) in a 4-bit cache
// (thakicloud.github.io, "Bonsai 27B: ternary and 1-bit quantization", the
// memory section; techtoast.kr, the KV-cache arithmetic; aitrends.kr,
// "Ternary-Bonsai-27B-mlx-2bit", "Technical features").  The pages give no
// 4-bit format.  Each head vector is cut into 8 groups of 32 dimensions, each
// with an FP16 scale d = fp16(amax / 7) and nibbles q + 8,
// q = clamp(rint(x / d), -8, 7), value (nibble - 8) * d.
//
// Physical layout (one layer and one sequence; capacity TC tokens, a
// multiple of 32), chosen for the MFMA operand layouts below:
//   K codes  [H][TC][32 dwords]: dword 8c + g holds dims 32g + 8c + e,
//            e = 2p + h at bits 16h + 4p (p = 0..3);
//   K scales [H][TC][8] FP16;
//   V codes  [H][TC/32][1024 dwords]: for the block of 32 tokens, dword
//            (16c + n) * 16 + j holds dim 16j + n of tokens tau(c, s),
//            s = 2p + h at bits 16h + 4p, with tau(c, s) = 4c + s for s < 4
//            and 16 + 4c + s - 4 for s >= 4;
//   V scales [H][TC/32][256] FP16: index (8c + g) * 8 + s is group g of
//            token tau(c, s).
//
// Decode attention.  Scores come from S^T = K Q^T on v_mfma_f32_16x16x32_f16
// with the keys as the A operand (16 tokens x 32 dims of one scale group)
// and the 16-padded query group as B.  A code nibble goes to mantissa bits
// [6,10) under exponent 19, the exact FP16 16 + nibble, so the MFMA returns
// sum (16 + nibble) q exactly and a group's score is d (D - 24 sum q): the
// scale applied once per group and token.  The softmax is online in the
// log2 domain.  O^T = V^T P^T takes the values as A (16 dims x 32 tokens,
// the same 16 + nibble decode) and P^T scaled by each token's value scale
// (FP16) as B; the token order of the K dimension is the one the score tiles
// leave in each lane, so P needs no data movement, and O = D - 24 sum B.  A
// workgroup of 4 waves splits a chunk of the sequence, stages its tiles in
// LDS, merges its waves there and writes (max, sum, output) per query head;
// a second kernel merges the chunks.
#include <hip/hip_runtime.h>

#include <mutex>

#include "tq_internal.h"

namespace tq {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kHD = 256;          // head dimension
constexpr int kWaves = 4;         // waves per attention workgroup
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ half8 as_half8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    const u32x4 v = {a, b, c, d};
    return __builtin_bit_cast(half8, v);
}

__device__ __forceinline__ f32x4 mfma(half8 a, half8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// 8 nibbles of a code dword as FP16 values, pairs in order: the nibble at
// mantissa bits [6,10) under exponent field 19 is exactly 16 + nibble.  The
// mask stays in a VGPR (gfx9 VOP3 takes no literal), so each pair is one
// shift and one v_and_or_b32.
constexpr uint32_t kExp19 = 0x4C004C00u;
__device__ __forceinline__ half8 decode8(uint32_t w, uint32_t mask) {
    return as_half8(((w << 6) & mask) | kExp19, ((w << 2) & mask) | kExp19, ((w >> 2) & mask) | kExp19,
                    ((w >> 6) & mask) | kExp19);
}

__device__ __forceinline__ float xor_max(float v, int m) { return fmaxf(v, __shfl_xor(v, m)); }

// v with the value of the lane W = 16 or 32 away (within 2W-lane groups)
// combined by sum or max: a v_permlane16/32_swap of v with itself leaves the
// lane's own value in one result and its partner's in the other, so this is
// the lane-xor shuffle's result on the VALU, without the LDS crossbar.
template <int W>
__device__ __forceinline__ void swap_pair(float v, float &a, float &b) {
    const uint32_t u = __builtin_bit_cast(uint32_t, v);
    const auto e = W == 16 ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                           : __builtin_amdgcn_permlane32_swap(u, u, false, false);
    a = __builtin_bit_cast(float, (uint32_t)e[0]);
    b = __builtin_bit_cast(float, (uint32_t)e[1]);
}
template <int W>
__device__ __forceinline__ float swap_sum(float v) {
    float a, b;
    swap_pair<W>(v, a, b);
    return a + b;
}
template <int W>
__device__ __forceinline__ float swap_max(float v) {
    float a, b;
    swap_pair<W>(v, a, b);
    return fmaxf(a, b);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF,
                                                                 false));
}

// Sum and maximum over the whole wave, every lane getting the result: DPP
// within 16-lane rows (quad_perm [1,0,3,2], [2,3,0,1], row_half_mirror,
// row_mirror), then the permlane exchanges across rows and halves.
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_f<0xB1>(v);
    v += dpp_f<0x4E>(v);
    v += dpp_f<0x141>(v);
    v += dpp_f<0x140>(v);
    return swap_sum<32>(swap_sum<16>(v));
}
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp_f<0xB1>(v));
    v = fmaxf(v, dpp_f<0x4E>(v));
    v = fmaxf(v, dpp_f<0x141>(v));
    v = fmaxf(v, dpp_f<0x140>(v));
    return swap_max<32>(swap_max<16>(v));
}

// ---------------------------------------------------------------- append
// One workgroup per (token, KV head), one thread per dimension.  A group of
// 32 dimensions is half a wave: its maximum comes from xor shuffles.
__global__ __launch_bounds__(256) void kv_append_kernel(const uint16_t *__restrict__ k,
                                                        const uint16_t *__restrict__ v,
                                                        int64_t pos, int H, int64_t TC,
                                                        uint32_t *__restrict__ kc,
                                                        uint16_t *__restrict__ ks,
                                                        uint32_t *__restrict__ vc,
                                                        uint16_t *__restrict__ vs) {
    const int tok = blockIdx.x / H, h = blockIdx.x % H;
    const int dim = threadIdx.x, g = dim >> 5;
    const int64_t t = pos + tok;
    const size_t src = ((size_t)tok * H + h) * kHD + dim;
    for (int which = 0; which < 2; ++which) {
        const float x = (float)__builtin_bit_cast(_Float16, (which ? v : k)[src]);
        float a = fabsf(x);
        a = xor_max(a, 1);
        a = xor_max(a, 2);
        a = xor_max(a, 4);
        a = xor_max(a, 8);
        a = xor_max(a, 16);
        const _Float16 d16 = (_Float16)__fdiv_rn(a, 7.0f);
        const float df = (float)d16;
        int q = 0;
        if (df != 0.0f) q = (int)fminf(fmaxf(rintf(__fdiv_rn(x, df)), -8.0f), 7.0f);
        const uint32_t nib = (uint32_t)(q + 8);
        const uint16_t dbits = __builtin_bit_cast(uint16_t, d16);
        if (which == 0) {
            // dword 8c + g with c = (dim % 32) / 8, e = dim % 8 at bits 16 (e & 1) + 4 (e >> 1)
            const int e = dim & 7, c = (dim >> 3) & 3;
            uint32_t part = nib << (16 * (e & 1) + 4 * (e >> 1));
            part |= __shfl_xor(part, 1);
            part |= __shfl_xor(part, 2);
            part |= __shfl_xor(part, 4);
            if (e == 0) kc[((size_t)h * TC + t) * 32 + 8 * c + g] = part;
            if ((dim & 31) == 0) ks[((size_t)h * TC + t) * 8 + g] = dbits;
        } else {
            const int64_t blk = t >> 5;
            const int r = (int)(t & 31);
            const int c = (r & 15) >> 2, s = r < 16 ? (r & 3) : 4 + (r & 3);
            const int sh = 16 * (s & 1) + 4 * (s >> 1);
            uint32_t *w = vc + ((size_t)h * (TC >> 5) + blk) * 1024 + (16 * c + (dim & 15)) * 16 + (dim >> 4);
            atomicAnd(w, ~(0xFu << sh));
            atomicOr(w, nib << sh);
            if ((dim & 31) == 0) vs[((size_t)h * (TC >> 5) + blk) * 256 + (8 * c + g) * 8 + s] = dbits;
        }
    }
}

// --------------------------------------------------------------- partial
// A 32-token tile of one KV head is four contiguous pieces of the cache: K
// codes (4 KiB), V codes of the token block (4 KiB), K scales and V scales
// (512 B each).  Each wave stages its tiles in LDS with direct global-to-LDS
// loads (nine dwordx4 loads per tile: lane l of a load fills bytes 16 l of
// its KiB) into a ring of two slots, and issues tile j + 1 before it computes
// tile j, so every wave keeps a tile in flight while it works.  The source
// address of each lane is permuted (16-byte units XOR-swizzled within a row)
// so that the MFMA operand reads below hit distinct LDS banks.
constexpr int kSlotBytes = 9216;  // K codes | V codes | K scales | V scales
constexpr int kOffV = 4096, kOffKs = 8192;
// direct-to-LDS loads per tile: one 1 KiB load (64 lanes x 16 bytes) per KiB
// of K codes and of V codes, and one for both scale pieces
constexpr int kKLoads = kOffV / 1024, kVLoads = (kOffKs - kOffV) / 1024, kScaleLoads = 1;
constexpr int kTileLoads = kKLoads + kVLoads + kScaleLoads;
static_assert(kSlotBytes - kOffKs == 64 * 16 * kScaleLoads, "one load carries both scale pieces");
static_assert(kTileLoads < 64, "vmcnt counts at most 63 loads");
constexpr int kRingBytes = 2 * kSlotBytes;  // per wave
static_assert(16 * (kHD + 2) * 4 <= kRingBytes, "a wave's merge rows fit in its ring");

__device__ __forceinline__ u32x4 lds16(const unsigned char *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}

// Stage tile tb of KV head h into the LDS slot dst (wave-uniform).
//   K codes: slot unit r * 8 + (j ^ (r & 7)) <- token r, 16-byte unit j;
//   V codes: slot unit R * 4 + (k ^ ((R >> 1) & 3)) <- row R = 16 c + n of
//            the block, unit k;
//   scales:  lanes 0-31 copy the tile's K scales, lanes 32-63 its V scales.
__device__ __forceinline__ void stage_tile(const uint32_t *__restrict__ kc, const uint16_t *__restrict__ ks,
                                           const uint32_t *__restrict__ vc, const uint16_t *__restrict__ vs,
                                           int64_t h, int64_t TC, int tb, unsigned char *dst, int lane) {
    const int64_t blk = tb >> 5;
    const unsigned char *kb = reinterpret_cast<const unsigned char *>(kc + (h * TC + tb) * 32);
    const unsigned char *vb = reinterpret_cast<const unsigned char *>(vc + (h * (TC >> 5) + blk) * 1024);
    const unsigned char *sb =
        lane < 32 ? reinterpret_cast<const unsigned char *>(ks + (h * TC + tb) * 8) + 16 * lane
                  : reinterpret_cast<const unsigned char *>(vs + (h * (TC >> 5) + blk) * 256) + 16 * (lane - 32);
#pragma unroll
    for (int i = 0; i < kKLoads; ++i) {
        const int L = 64 * i + lane, r = L >> 3, j = (L & 7) ^ (r & 7);
        __builtin_amdgcn_global_load_lds(kb + 16 * (8 * r + j), dst + 1024 * i, 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < kVLoads; ++i) {
        const int L = 64 * i + lane, R = L >> 2, k = (L & 3) ^ ((R >> 1) & 3);
        __builtin_amdgcn_global_load_lds(vb + 16 * (4 * R + k), dst + kOffV + 1024 * i, 16, 0, 0);
    }
    __builtin_amdgcn_global_load_lds(sb, dst + kOffKs, 16, 0, 0);
}

// Workgroup (chunk, KV head): 4 waves take consecutive 32-token tiles of the
// chunk round-robin.  Lane l: head column n = l % 16 (a query head of the
// group when n < R), lane group c = l / 16.
__global__ __launch_bounds__(64 * kWaves) void attn_partial_kernel(
    const uint16_t *__restrict__ q, const uint32_t *__restrict__ kc, const uint16_t *__restrict__ ks,
    const uint32_t *__restrict__ vc, const uint16_t *__restrict__ vs, int T, int64_t TC, int R,
    int chunk, float *__restrict__ ws) {
    __shared__ __attribute__((aligned(16))) unsigned char lds[kWaves * kRingBytes];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15, c = lane >> 4;
    const int h = blockIdx.y, ck = blockIdx.x;
    const int t_begin = ck * chunk, t_end = min(T, t_begin + chunk);
    const int nq = R;  // query heads of this KV head
    unsigned char *ring = lds + wave * kRingBytes;
    const int tfirst = t_begin + 32 * wave;
    const int ntiles = tfirst < t_end ? (t_end - tfirst + 32 * kWaves - 1) / (32 * kWaves) : 0;

    // the first two tiles go out before the query, whose wait covers them
    if (ntiles > 0) stage_tile(kc, ks, vc, vs, h, TC, tfirst, ring, lane);
    if (ntiles > 1) stage_tile(kc, ks, vc, vs, h, TC, tfirst + 32 * kWaves, ring + kSlotBytes, lane);
    // query as the B operand: B[k = 8c + s of group g][n] = q[n][32g + 8c + s];
    // columns n >= R load head R - 1 and are zeroed (one wait for all loads)
    u32x4 qv[8];
    const uint16_t *qrow = q + ((size_t)(h * nq + min(n, nq - 1))) * kHD + 8 * c;
#pragma unroll
    for (int g = 0; g < 8; ++g) qv[g] = *reinterpret_cast<const u32x4 *>(qrow + 32 * g);

    uint32_t mask = 0x03C003C0u;
    asm volatile("" : "+v"(mask));
    half8 qb[8];
    float qs24[8];
#pragma unroll
    for (int g = 0; g < 8; ++g) {
        const u32x4 v = n < nq ? qv[g] : u32x4{0u, 0u, 0u, 0u};
        qb[g] = __builtin_bit_cast(half8, v);
        const half2_t one2 = {(_Float16)1.0f, (_Float16)1.0f};
        const uint32_t v0 = v[0], v1 = v[1], v2 = v[2], v3 = v[3];
        float sq = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, v0), one2, 0.0f, false);
        sq = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, v1), one2, sq, false);
        sq = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, v2), one2, sq, false);
        sq = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, v3), one2, sq, false);
        sq = swap_sum<16>(sq);
        sq = swap_sum<32>(sq);
        qs24[g] = -24.0f * sq;
    }

    f32x4 oacc[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) oacc[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float m = -INFINITY, lsum = 0.0f, cs[8];
#pragma unroll
    for (int g = 0; g < 8; ++g) cs[g] = 0.0f;
    const float zs = kLog2e / 16.0f;  // 1 / sqrt(256), log2 domain

    for (int j = 0; j < ntiles; ++j) {
        const int tb = tfirst + 32 * kWaves * j;
        // in flight: tile j and, unless j is the last, tile j + 1 (whose
        // kTileLoads loads are the youngest: loads complete in order)
        if (j + 1 < ntiles)
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kTileLoads) : "memory");
        else
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        unsigned char *slot = ring + (j & 1) * kSlotBytes;
        // scores of the tile's two 16-token halves: z[u][i] for token
        // tb + 16u + 4c + i, head n
        float z[2][4];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int r = 16 * u + n;  // the A row this lane supplies
            const u32x4 k0 = lds16(slot + 16 * (8 * r + ((2 * c) ^ (r & 7))));
            const u32x4 k1 = lds16(slot + 16 * (8 * r + ((2 * c + 1) ^ (r & 7))));
            const uint32_t kw[8] = {k0[0], k0[1], k0[2], k0[3], k1[0], k1[1], k1[2], k1[3]};
            // scales of the lane's D rows: tokens 16u + 4c + i of the tile, all groups
            u32x4 sv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) sv[i] = lds16(slot + kOffKs + 16 * (16 * u + 4 * c + i));
            float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int g = 0; g < 8; ++g) {
                const f32x4 D = mfma(decode8(kw[g], mask), qb[g], f32x4{0.0f, 0.0f, 0.0f, 0.0f});
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t pair = sv[i][g >> 1];
                    const float d = (float)__builtin_bit_cast(_Float16, (uint16_t)(g & 1 ? pair >> 16 : pair));
                    acc[i] = __builtin_fmaf(d, D[i] + qs24[g], acc[i]);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = tb + 16 * u + 4 * c + i;
                z[u][i] = (t < t_end) ? acc[i] * zs : -INFINITY;
            }
        }
        // online softmax over the tile
        float mt = fmaxf(fmaxf(fmaxf(z[0][0], z[0][1]), fmaxf(z[0][2], z[0][3])),
                         fmaxf(fmaxf(z[1][0], z[1][1]), fmaxf(z[1][2], z[1][3])));
        mt = swap_max<16>(mt);
        mt = swap_max<32>(mt);
        const float mn = fmaxf(m, mt);
        // the running maximum moves only when a score passes it by more than
        // 2 (log2 domain): the probabilities below stay <= 4, so p d_V stays
        // inside the FP16 range for every finite FP16 value (4 * 65504 / 7),
        // and most tiles skip the rescale
        if (__any(mn > m + 2.0f)) {
            const float alpha = __builtin_amdgcn_exp2f(m - mn);  // 0 on the first tile (m = -inf)
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) oacc[jj] *= alpha;
            lsum *= alpha;
#pragma unroll
            for (int g = 0; g < 8; ++g) cs[g] *= alpha;
            m = mn;
        }
        float p[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            p[s] = __builtin_amdgcn_exp2f(z[s >> 2][s & 3] - m);
            lsum += p[s];
        }
        // P^T scaled by the value scales, per group: B'[k = s][n] = p_s d_V
        const half2_t p2[4] = {half2_t{(_Float16)p[0], (_Float16)p[1]}, half2_t{(_Float16)p[2], (_Float16)p[3]},
                               half2_t{(_Float16)p[4], (_Float16)p[5]}, half2_t{(_Float16)p[6], (_Float16)p[7]}};
        // Tokens at or past the chunk's end have p = 0, but their value
        // scales are whatever the cache holds there (a NaN or Inf would turn
        // 0 * d into NaN): in a tile that crosses the end, the scales of those
        // tokens are replaced by +0 before they meet p.  Token of pair half
        // (s & 1) of dword s / 2: tb + 16 (s / 4) + 4 c + (s % 4).
        uint32_t vmask[4] = {~0u, ~0u, ~0u, ~0u};
        if (tb + 32 > t_end) {
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2) {
                const int t0 = tb + 16 * (s2 >> 1) + 4 * c + 2 * (s2 & 1);
                vmask[s2] = (t0 < t_end ? 0x0000FFFFu : 0u) | (t0 + 1 < t_end ? 0xFFFF0000u : 0u);
            }
        }
        half8 bp[8];
#pragma unroll
        for (int g = 0; g < 8; ++g) {
            // (the elements go through plain uint32_t: a bit cast taken directly
            // of a vector element has read element 0 for every index)
            const u32x4 dv = lds16(slot + kOffKs + 512 + 128 * c + 16 * g);
            const uint32_t d0 = dv[0] & vmask[0], d1 = dv[1] & vmask[1], d2 = dv[2] & vmask[2],
                           d3 = dv[3] & vmask[3];
            const half2_t b0 = p2[0] * __builtin_bit_cast(half2_t, d0);
            const half2_t b1 = p2[1] * __builtin_bit_cast(half2_t, d1);
            const half2_t b2 = p2[2] * __builtin_bit_cast(half2_t, d2);
            const half2_t b3 = p2[3] * __builtin_bit_cast(half2_t, d3);
            bp[g] = as_half8(__builtin_bit_cast(uint32_t, b0), __builtin_bit_cast(uint32_t, b1),
                             __builtin_bit_cast(uint32_t, b2), __builtin_bit_cast(uint32_t, b3));
            const half2_t one2 = {(_Float16)1.0f, (_Float16)1.0f};
            float sum = __builtin_amdgcn_fdot2(b0, one2, 0.0f, false);
            sum = __builtin_amdgcn_fdot2(b1, one2, sum, false);
            sum = __builtin_amdgcn_fdot2(b2, one2, sum, false);
            cs[g] = __builtin_amdgcn_fdot2(b3, one2, sum, false) + cs[g];
        }
        // O^T += V^T P'^T over 16 tiles of 16 dimensions
        const int Rv = 16 * c + n;
        uint32_t vw[16];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const u32x4 v = lds16(slot + kOffV + 16 * (4 * Rv + (k ^ ((Rv >> 1) & 3))));
            vw[4 * k] = v[0];
            vw[4 * k + 1] = v[1];
            vw[4 * k + 2] = v[2];
            vw[4 * k + 3] = v[3];
        }
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) oacc[jj] = mfma(decode8(vw[jj], mask), bp[jj >> 1], oacc[jj]);
        // tile j + 2 into this slot: every read of it above has returned (its
        // value is in use)
        if (j + 2 < ntiles) stage_tile(kc, ks, vc, vs, h, TC, tb + 64 * kWaves, slot, lane);
    }

    // this wave's (max, sum, output) per head into LDS, over its own ring
    // once every load into it has landed: O = D - 24 cs
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lsum = swap_sum<16>(lsum);
    lsum = swap_sum<32>(lsum);
#pragma unroll
    for (int g = 0; g < 8; ++g) {
        cs[g] = swap_sum<16>(cs[g]);
        cs[g] = swap_sum<32>(cs[g]);
    }
    float *red = reinterpret_cast<float *>(ring);  // [16][kHD + 2]
#pragma unroll
    for (int jj = 0; jj < 16; ++jj)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            red[n * (kHD + 2) + 16 * jj + 4 * c + i] = __builtin_fmaf(-24.0f, cs[jj >> 1], oacc[jj][i]);
    if (c == 0) {
        red[n * (kHD + 2) + kHD] = m;
        red[n * (kHD + 2) + kHD + 1] = lsum;
    }
    __syncthreads();
    // the waves' weights per query head, once: thread (head hn, wave w) of wave 0
    __shared__ float wgt[16][kWaves];
    __shared__ float head_m[16], head_l[16];
    if (wave == 0) {
        const int hn = lane >> 2, w = lane & 3;
        const float *rw = reinterpret_cast<const float *>(lds + w * kRingBytes) + hn * (kHD + 2);
        const float mw = rw[kHD];
        float mx = fmaxf(mw, __shfl_xor(mw, 1));
        mx = fmaxf(mx, __shfl_xor(mx, 2));
        const float e = mw == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mw - mx);  // a wave with no tile
        float l = e * rw[kHD + 1];
        l += __shfl_xor(l, 1);
        l += __shfl_xor(l, 2);
        wgt[hn][w] = e;
        if (w == 0) {
            head_m[hn] = mx;
            head_l[hn] = l;
        }
    }
    __syncthreads();
    // merge the waves: thread = dimension, loop over the query heads
    const int dim = threadIdx.x;
    for (int hn = 0; hn < nq; ++hn) {
        float o = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w)
            o = __builtin_fmaf(wgt[hn][w], reinterpret_cast<const float *>(lds + w * kRingBytes)[hn * (kHD + 2) + dim], o);
        float *dst = ws + ((size_t)ck * gridDim.y * nq + h * nq + hn) * (kHD + 2);
        dst[dim] = o;
        if (dim == 0) {
            dst[kHD] = head_m[hn];
            dst[kHD + 1] = head_l[hn];
        }
    }
}

constexpr int kMaxChunks = 1024;
constexpr int kMergeRound = 32;  // chunk outputs a lane has in flight at once

// Merge the chunks.  Workgroup (query head, quarter of the dimensions); wave
// w takes a contiguous quarter of the chunks, lane = dimension.  Per round of
// up to 32 chunks a lane issues all 32 output loads at once while lane c also
// loads chunk c's (max, sum); the round's maximum and denominator are wave
// reductions and chunk c's weight reaches every lane by readlane.  Rounds
// fold into a running (max, numerator, denominator) by rescaling, and the four
// waves meet in LDS.  Up to 128 chunks cost one memory round trip.  Offsets
// stay below 2^31 (n_q <= 1024, chunks <= 1024).
__global__ __launch_bounds__(256) void attn_combine_kernel(const float *__restrict__ ws, int nchunks,
                                                           int nqh, float *__restrict__ out) {
    __shared__ float part_m[kWaves], part_d[kWaves], part_n[kWaves][64];
    const int hq = blockIdx.x, lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int dim = 64 * blockIdx.y + lane;
    const int stride = nqh * (kHD + 2);
    const float *base = ws + hq * (kHD + 2);
    const int per = (nchunks + kWaves - 1) / kWaves;
    const int c0 = wave * per, c1 = min(nchunks, c0 + per);
    float M = -INFINITY, num = 0.0f, den = 0.0f;
    for (int r = c0; r < c1; r += kMergeRound) {
        const int last = min(kMergeRound, c1 - r) - 1;
        const int mine = r + min(lane, last);
        const float m = base[mine * stride + kHD];
        const float l = base[mine * stride + kHD + 1];
        float o[kMergeRound];
#pragma unroll
        for (int i = 0; i < kMergeRound; ++i) o[i] = base[(r + min(i, last)) * stride + dim];
        float mx = m;
        mx = wave_max(mx);
        const float mn = fmaxf(M, mx);
        const float alpha = exp2f(M - mn);  // 0 on the first round
        const float e = lane <= last ? exp2f(m - mn) : 0.0f;
        float dr = e * l;
        dr = wave_sum(dr);
        float nr = 0.0f;
#pragma unroll
        for (int i = 0; i < kMergeRound; ++i)
            nr = __builtin_fmaf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, e), i)),
                                o[i], nr);
        num = __builtin_fmaf(num, alpha, nr);
        den = __builtin_fmaf(den, alpha, dr);
        M = mn;
    }
    part_n[wave][lane] = num;
    if (lane == 0) {
        part_m[wave] = M;
        part_d[wave] = den;
    }
    __syncthreads();
    if (wave == 0) {
        float mx = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, part_m[w]);
        float tn = 0.0f, td = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float mw = part_m[w];
            const float e = mw == -INFINITY ? 0.0f : exp2f(mw - mx);  // a wave with no chunks
            tn = __builtin_fmaf(e, part_n[w][lane], tn);
            td = __builtin_fmaf(e, part_d[w], td);
        }
        out[hq * kHD + dim] = tn / td;
    }
}

}  // namespace

// Tokens per attention chunk: a multiple of 32 * kWaves giving about two
// workgroups per CU over the KV heads, and never more than kMaxChunks chunks.
// ---------------------------------------------------------- no-allocation
// Scratch for the entry point that allocates nothing (tq_attn_decode_noalloc):
// the per-chunk (max, sum, output) rows of attn_partial_kernel, which the
// caller otherwise passes as a workspace.  8 MiB per GPU, held until the
// process ends; the model's shape (24 query heads over 4 KV heads) needs at
// most about 3 MiB at any context length.  Nothing in it has to start at
// zero: the partial kernel writes every row the merge reads in the same call.
// All calls on one GPU share it, so calls that overlap on a GPU (different
// streams, no ordering between them) race.
constexpr size_t kScratchBytes = size_t(8) << 20;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float *g_scratch_ptr[kMaxDevices] = {};
}  // namespace

size_t attn_scratch_bytes() { return kScratchBytes; }

// The current device's copy of `scratch`: looked up once per device (with
// that device current) and kept.  In host code the array's name is only a
// stand-in for the device symbol, so kernels get this address, never the name.
int32_t attn_scratch(float **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(TQ_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(TQ_ERR_HIP, "device %d above the %d supported", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(TQ_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        g_scratch_ptr[dev] = static_cast<float *>(p);
    }
    *out = g_scratch_ptr[dev];
    return TQ_OK;
}

int64_t attn_chunk(int64_t T, int64_t n_kv) {
    const int64_t step = 32 * kWaves;
    int64_t want = (T * n_kv + 511) / 512;
    const int64_t floor_c = (T + kMaxChunks - 1) / kMaxChunks;
    if (want < floor_c) want = floor_c;
    int64_t c = (want + step - 1) / step * step;
    if (c < step) c = step;
    return c;
}

int32_t kv_append_enqueue(const uint16_t *k, const uint16_t *v, int64_t n_tok, int64_t pos, int64_t H,
                          int64_t TC, uint8_t *kc, uint16_t *ks, uint8_t *vc, uint16_t *vs,
                          hipStream_t stream) {
    hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)(n_tok * H)), dim3(256), 0, stream, k, v, pos,
                       (int)H, TC, reinterpret_cast<uint32_t *>(kc), ks,
                       reinterpret_cast<uint32_t *>(vc), vs);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(TQ_ERR_HIP, "KV append launch failed: %s", hipGetErrorString(e));
    return TQ_OK;
}

int32_t attn_decode_enqueue(const uint16_t *q, const uint8_t *kc, const uint16_t *ks,
                            const uint8_t *vc, const uint16_t *vs, int64_t T, int64_t TC,
                            int64_t n_q, int64_t n_kv, float *out, float *ws, hipStream_t stream) {
    const int64_t chunk = attn_chunk(T, n_kv);
    const int64_t nchunks = (T + chunk - 1) / chunk;
    hipLaunchKernelGGL(attn_partial_kernel, dim3((unsigned)nchunks, (unsigned)n_kv), dim3(64 * kWaves), 0,
                       stream, q, reinterpret_cast<const uint32_t *>(kc), ks,
                       reinterpret_cast<const uint32_t *>(vc), vs, (int)T, TC, (int)(n_q / n_kv),
                       (int)chunk, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(TQ_ERR_HIP, "attention launch failed: %s", hipGetErrorString(e));
    hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)n_q, kHD / 64), dim3(64 * kWaves), 0, stream, ws,
                       (int)nchunks, (int)n_q, out);
    e = hipGetLastError();
    if (e != hipSuccess) return fail(TQ_ERR_HIP, "attention launch failed: %s", hipGetErrorString(e));
    return TQ_OK;
}

}  // namespace tq
