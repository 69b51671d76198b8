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
// log2 domain.  O^T = V^T P^T takes the values as A (16 dims x 32 tokens)
// and P^T scaled by each token's value scale (FP16) as B; the token order of
// the K dimension is the one the score tiles leave in each lane, so P needs
// no data movement.  A workgroup of 4 waves splits a chunk of the sequence,
// merges its waves in LDS and writes (max, sum, output) per query head; a
// second kernel merges the chunks.
#include <hip/hip_runtime.h>

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

// 8 nibbles of a code dword as FP16 values linear in the nibble, pairs in
// order: nibble at mantissa bits [6,10) under exponent field E, i.e.
// 2^(E-15) (1 + nibble/16).  E = 15 gives 1 + nibble/16, E = 19 gives
// 16 + nibble.  The mask stays in a VGPR (gfx9 VOP3 takes no literal), so each
// pair is one shift and one v_and_or_b32.
template <uint32_t EXP2>
__device__ __forceinline__ half8 decode8(uint32_t w, uint32_t mask) {
    return as_half8(((w << 6) & mask) | EXP2, ((w << 2) & mask) | EXP2, ((w >> 2) & mask) | EXP2,
                    ((w >> 6) & mask) | EXP2);
}
constexpr uint32_t kExp15 = 0x3C003C00u;  // 1 + nibble/16
constexpr uint32_t kExp19 = 0x4C004C00u;  // 16 + nibble

// token offset within a 32-token block of K slot s of lane group c
__device__ __forceinline__ int tau(int c, int s) { return s < 4 ? 4 * c + s : 12 + 4 * c + s; }

__device__ __forceinline__ float xor_max(float v, int m) { return fmaxf(v, __shfl_xor(v, m)); }

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
// Workgroup (chunk, KV head): 4 waves take consecutive 32-token tiles of the
// chunk round-robin.  Lane l: head column n = l % 16 (a query head of the
// group when n < R), lane group c = l / 16.
__global__ __launch_bounds__(64 * kWaves) void attn_partial_kernel(
    const uint16_t *__restrict__ q, const uint32_t *__restrict__ kc, const uint16_t *__restrict__ ks,
    const uint32_t *__restrict__ vc, const uint16_t *__restrict__ vs, int T, int64_t TC, int R,
    int chunk, float *__restrict__ ws) {
    __shared__ float red[kWaves][16][kHD + 2];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, c = lane >> 4;
    const int h = blockIdx.y, ck = blockIdx.x;
    const int t_begin = ck * chunk, t_end = min(T, t_begin + chunk);
    const int nq = R;  // query heads of this KV head

    uint32_t mask = 0x03C003C0u;
    asm volatile("" : "+v"(mask));
    // query as the B operand: B[k = 8c + s of group g][n] = q[n][32g + 8c + s]
    half8 qb[8];
    float qs24[8];
#pragma unroll
    for (int g = 0; g < 8; ++g) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (n < nq)
            v = *reinterpret_cast<const u32x4 *>(q + ((size_t)(h * nq + n)) * kHD + 32 * g + 8 * c);
        qb[g] = __builtin_bit_cast(half8, v);
        float sq = 0.0f;
#pragma unroll
        for (int s = 0; s < 8; ++s) sq += (float)qb[g][s];
        sq += __shfl_xor(sq, 16);
        sq += __shfl_xor(sq, 32);
        qs24[g] = -24.0f * sq;
    }

    f32x4 oacc[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) oacc[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float m = -INFINITY, lsum = 0.0f, cs[8];
#pragma unroll
    for (int g = 0; g < 8; ++g) cs[g] = 0.0f;
    const float zs = kLog2e / 16.0f;  // 1 / sqrt(256), log2 domain

    for (int tb = t_begin + 32 * wave; tb < t_end; tb += 32 * kWaves) {
        const int64_t blk = tb >> 5;
        // scores of the tile's two 16-token halves: z[u][i] for token
        // tb + 16u + 4c + i, head n
        float z[2][4];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int trow = tb + 16 * u + n;  // the A row this lane supplies
            const u32x4 *kr = reinterpret_cast<const u32x4 *>(kc + ((size_t)h * TC + trow) * 32 + 8 * c);
            const u32x4 k0 = kr[0], k1 = kr[1];
            const uint32_t kw[8] = {k0[0], k0[1], k0[2], k0[3], k1[0], k1[1], k1[2], k1[3]};
            // scales of the lane's D rows: tokens tb + 16u + 4c + i, all groups
            const uint16_t *sp = ks + ((size_t)h * TC + tb + 16 * u + 4 * c) * 8;
            u32x4 sv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) sv[i] = reinterpret_cast<const u32x4 *>(sp)[i];
            float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int g = 0; g < 8; ++g) {
                const f32x4 D = mfma(decode8<kExp19>(kw[g], mask), qb[g], f32x4{0.0f, 0.0f, 0.0f, 0.0f});
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
        mt = xor_max(mt, 16);
        mt = xor_max(mt, 32);
        const float mn = fmaxf(m, mt);
        if (__any(mn > m)) {
            const float alpha = exp2f(m - mn);  // 0 on the first tile (m = -inf)
#pragma unroll
            for (int j = 0; j < 16; ++j) oacc[j] *= alpha;
            lsum *= alpha;
#pragma unroll
            for (int g = 0; g < 8; ++g) cs[g] *= alpha;
            m = mn;
        }
        float p[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            p[s] = exp2f(z[s >> 2][s & 3] - m);
            lsum += p[s];
        }
        // P^T scaled by the value scales, per group: B'[k = s][n] = p_s d_V
        const half2_t p2[4] = {half2_t{(_Float16)p[0], (_Float16)p[1]}, half2_t{(_Float16)p[2], (_Float16)p[3]},
                               half2_t{(_Float16)p[4], (_Float16)p[5]}, half2_t{(_Float16)p[6], (_Float16)p[7]}};
        const u32x4 *vsp = reinterpret_cast<const u32x4 *>(vs + ((size_t)h * (TC >> 5) + blk) * 256 + 64 * c);
        half8 bp[8];
#pragma unroll
        for (int g = 0; g < 8; ++g) {
            // (the elements go through plain uint32_t: a bit cast taken directly
            // of a vector element has read element 0 for every index)
            const u32x4 dv = vsp[g];
            const uint32_t d0 = dv[0], d1 = dv[1], d2 = dv[2], d3 = dv[3];
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
        const u32x4 *vr = reinterpret_cast<const u32x4 *>(vc + ((size_t)h * (TC >> 5) + blk) * 1024 + (16 * c + n) * 16);
        const u32x4 v0 = vr[0], v1 = vr[1], v2 = vr[2], v3 = vr[3];
        const uint32_t vw[16] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3],
                                 v2[0], v2[1], v2[2], v2[3], v3[0], v3[1], v3[2], v3[3]};
#pragma unroll
        for (int j = 0; j < 16; ++j) oacc[j] = mfma(decode8<kExp15>(vw[j], mask), bp[j >> 1], oacc[j]);
    }

    // this wave's (max, sum, output) per head into LDS: O = 16 D - 24 cs
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
#pragma unroll
    for (int g = 0; g < 8; ++g) {
        cs[g] += __shfl_xor(cs[g], 16);
        cs[g] += __shfl_xor(cs[g], 32);
    }
#pragma unroll
    for (int j = 0; j < 16; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            red[wave][n][16 * j + 4 * c + i] = 16.0f * oacc[j][i] - 24.0f * cs[j >> 1];
    if (c == 0) {
        red[wave][n][kHD] = m;
        red[wave][n][kHD + 1] = lsum;
    }
    __syncthreads();
    // merge the waves: thread = dimension, loop over the query heads
    const int dim = threadIdx.x;
    for (int hn = 0; hn < nq; ++hn) {
        float mx = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, red[w][hn][kHD]);
        float o = 0.0f, l = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float mw = red[w][hn][kHD];
            const float e = mw == -INFINITY ? 0.0f : exp2f(mw - mx);
            o += e * red[w][hn][dim];
            l += e * red[w][hn][kHD + 1];
        }
        float *dst = ws + ((size_t)ck * gridDim.y * nq + h * nq + hn) * (kHD + 2);
        dst[dim] = o;
        if (dim == 0) {
            dst[kHD] = mx;
            dst[kHD + 1] = l;
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
#pragma unroll
        for (int s = 32; s >= 1; s >>= 1) mx = fmaxf(mx, __shfl_xor(mx, s));
        const float mn = fmaxf(M, mx);
        const float alpha = exp2f(M - mn);  // 0 on the first round
        const float e = lane <= last ? exp2f(m - mn) : 0.0f;
        float dr = e * l;
#pragma unroll
        for (int s = 32; s >= 1; s >>= 1) dr += __shfl_xor(dr, s);
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
