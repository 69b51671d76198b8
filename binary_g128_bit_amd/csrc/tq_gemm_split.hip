// Small-batch GEMM for 5..64 activation rows over packed ternary g128
// weights on v_mfma_f32_16x16x32_f16, gfx950: K split over workgroups, each
// workgroup's activation slice staged once in LDS.
//
// Y[m][n] = sum_g s[n][g] * sum_{j<128} t[n][128g+j] * X[m][128g+j]
// (w_i = s_g * t_i with one FP16 scale per 128 weights: thakicloud.github.io,
// "Bonsai 27B: ternary and 1-bit quantization", "How the compression works";
// the packed slots are read directly and the scale is applied inside the
// matmul: aitrends.kr, "Ternary-Bonsai-27B-mlx-2bit", "Technical features").
// Batches of this width are the speculative-verify and short prefill chunks
// of the same page of thakicloud.github.io ("Throughput and speculative
// decoding").
//
// Matrix cores.  In v_mfma_f32_16x16x32_f16 lane l supplies row l % 16 of A
// and column l % 16 of B, eight K values each from the slice 8 (l / 16), and
// receives D[4 (l / 16) + i][l % 16].  A is a tile of 16 activation rows
// (rows past M are zero; MT = 1, 2 or 4 tiles), B a tile of 16 weight rows,
// decoded once per window and used by every activation tile.  A window is 256 weights (two scale groups, 64 code bytes
// per row).  Lane group q loads bytes [16q, 16q + 16) of its row's window;
// one v_permlane32_swap per dword pair then leaves lane group q 8 bytes (32
// weights) of each group, weights [32 s, 32 s + 32) with s = (0, 2, 1, 3)[q],
// so that every MFMA sums within one group and its scale applies to its
// result.
//
// Decode (exact).  Codes become FP16 values linear in the code: E slots
// c 2^-14, M4 slots 2^-12 + c 2^-14, M16 slots 2^-10 + c 2^-14, as pairs
// (weight p, weight p + 8) of a code dword.  The activations are staged in
// LDS in the same pairing, so the A fragments are read as they are.  The
// offsets and t = c - 1 are removed by starting each group's MFMA chain from
// -C with C[m] = sum_k (1 + offset_k) 2^-14 x[m][k], summed while the slice
// is staged; each group's D = 2^-14 sum t x is scaled by its FP16 scale in
// FP32, and results by 2^14 at the end.
//
// Work split.  A workgroup of 8 waves owns 8 NT consecutive 16-row tiles and
// one K slice of at most split_max_win(MT) windows.  It stages the slice's activations
// (paired, in the MFMA lane order) and offset sums in LDS once; then each
// wave runs its NT tiles over the slice's windows, the code loads running PF
// window pairs ahead in registers (a pair is 128 code bytes of a row, both
// halves requested together).  With one slice the tiles go straight to Y;
// otherwise each slice writes its partial Y to a caller-provided workspace
// and a second kernel adds the slices in a fixed order, so results do not
// depend on timing.  (Letting the last workgroup of a tile block add them needs a
// device-scope release per workgroup, an L2 write-back that measured 5-9x
// slower in total.)
//
// Measured (MI355X, back to back): 16 rows on 17408 x 5120 in 16.5 us,
// 5120 x 17408 in 19 us, 34816 x 5120 in 28 us, against 22, 24.5 and 29 us
// for the per-group kernel of tq_gemm.hip; 32 rows 22.4 / 24.0 us against
// 35.8 / 46.5; 64 rows 32.5 / 32.3 us against 48 / 45.  Wave timestamps: about 3 us of each
// launch go to the activation slice (fetched at every launch), 1 us more to
// the first code pairs; the window loop then streams codes at about 5 TB/s.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>
#include <cstring>

#include "tq_internal.h"

namespace tq {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kSWaves = 8;
constexpr int kSThreads = 64 * kSWaves;
constexpr int kSWinLds = 8192 + 1024 + 128;  // LDS bytes per staged window and 16-row activation tile
// Windows per K slice by activation tiles: 74 KB of LDS for one tile (two
// workgroups per CU), 75 KB for two, 150 KB for four (one workgroup per CU).
__host__ __device__ constexpr int split_max_win(int mt) { return mt == 1 ? 8 : 4; }
__host__ __device__ constexpr int split_min_wg(int mt) { return mt == 4 ? 1 : 2; }
constexpr float kSInvUnit = 16384.0f;

__device__ __forceinline__ uint32_t svreg(uint32_t v) {
    asm volatile("" : "+v"(v));
    return v;
}

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a), __builtin_bit_cast(half8, b), c, 0,
                                                 0, 0);
}

// The 16 ternary weights of code dword d as pairs w[p] = (weight p, weight
// p + 8), p = 0..7.
__device__ __forceinline__ void sdecode(uint32_t d, uint32_t m8, uint32_t m6, uint32_t (&w)[8]) {
    const uint32_t c6 = d << 6, r4 = d >> 4;
    w[0] = (c6 & m6) | 0x14001400u;  // M16
    w[1] = (c6 & m8) | 0x0C000C00u;  // M4
    w[2] = c6 & 0x0C000C00u;         // E
    w[3] = (d & m6) | 0x14001400u;   // M16
    w[4] = (d & m8) | 0x0C000C00u;   // M4
    w[5] = d & 0x0C000C00u;          // E
    w[6] = (r4 & m8) | 0x0C000C00u;  // M4
    w[7] = r4 & 0x0C000C00u;         // E
}

// (1 + offset) 2^-14 of pair p as an FP16 pair: M16 17 2^-14 (p = 0, 3),
// M4 5 2^-14 (p = 1, 4, 6), E 2^-14 (p = 2, 5, 7); all exact FP16 normals.
__device__ __forceinline__ constexpr uint32_t sslot_w(int p) {
    return (p == 0 || p == 3) ? 0x14401440u : (p == 1 || p == 4 || p == 6) ? 0x0D000D00u : 0x04000400u;
}

// LDS layout of a slice of SW windows and MT activation tiles of 16 rows
// (u32x4 units):
//   xf   [SW][2 groups][MT][4 chunks][64 lanes]  A fragments: chunk c of lane
//        (m, q) holds pair dwords 4c..4c+3 of its 32 weights of the group
//        (unit 2 s + c / 2, pairs 4 (c % 2) .. 4 (c % 2) + 3) for row 16u + m;
//   cpart [SW][2][8 units][16 MT rows] float   per-unit offset sums;
//   cneg  [SW][2][16 MT rows] float            -C per group and row.
template <int NT, int PF, int MT>
__global__ __launch_bounds__(kSThreads, split_min_wg(MT)) void gemm_split_kernel(
    const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales, const uint16_t *__restrict__ X,
    float *__restrict__ Y, float *__restrict__ ws, int M, int N, int K, int KS) {
    constexpr int MR = 16 * MT;  // staged activation rows
    extern __shared__ u32x4 slds[];
    const int G = K >> 7, W = G >> 1;
    const int ks = blockIdx.y;
    const int wb = ks * W / KS, SW = (ks + 1) * W / KS - wb;  // this slice's windows
    u32x4 *xf = slds;
    float *cpart = reinterpret_cast<float *>(slds + SW * MT * 512);
    float *cneg = cpart + SW * MT * 256;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int n = lane & 15, q = lane >> 4;
    const int tile0 = (blockIdx.x * kSWaves + wave) * NT;

    // ---- 1. this thread's activation units of the slice (L2), then the
    // first PF windows' codes and scales (HBM): the staging below waits for
    // the activations only.  Unit e = (unit r = 16 window + u16 of 16 values,
    // row m = e % MR): the 16 lanes of a row group write 16 distinct LDS
    // slots (row-major order put all 16 units of a window on one bank group),
    // and every row's 128-byte line is read whole by 4 such groups.
    constexpr int kUnitsPerThread = MR * split_max_win(MT) * 16 / kSThreads;
    const int nunits = MR * SW * 16;
    u32x4 xlo[kUnitsPerThread], xhi[kUnitsPerThread];
#pragma unroll
    for (int j = 0; j < kUnitsPerThread; ++j) {
        const int e = (int)threadIdx.x + j * kSThreads;
        const int m = e % MR, r = e / MR;
        xlo[j] = xhi[j] = u32x4{0u, 0u, 0u, 0u};
        if (e < nunits && m < M) {
            const u32x4 *src = reinterpret_cast<const u32x4 *>(X + (size_t)m * K + (size_t)wb * 256 + 16 * r);
            xlo[j] = src[0];
            xhi[j] = src[1];
        }
    }

    const int row_bytes = G * 32;
    const __amdgpu_buffer_rsrc_t crs =
        __builtin_amdgcn_make_buffer_rsrc((void *)codes, 0, N * row_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t srs =
        __builtin_amdgcn_make_buffer_rsrc((void *)scales, 0, N * G * 2, 0x00020000);
    int coff[NT], soff[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int row = 16 * (tile0 + t) + n;  // rows past N read zeros
        coff[t] = row * row_bytes + 64 * wb + 16 * q;
        soff[t] = row * G * 2 + 4 * wb;
    }
    u32x4 rc[PF][NT][2];
    uint32_t rsc[PF][NT][2];
    const int NPR = (SW + 1) >> 1;  // window pairs of the slice
    auto load_pair = [&](int p, int wp) __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                rc[p][t][h] = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(crs, coff[t] + 64 * min(2 * wp + h, SW - 1), 0, 0));
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                rsc[p][t][h] = __builtin_amdgcn_raw_buffer_load_b32(srs, soff[t] + 4 * min(2 * wp + h, SW - 1), 0, 0);
    };
#pragma unroll
    for (int p = 0; p < PF; ++p) load_pair(p, min(p, NPR - 1));

    // ---- 2. stage the slice: pair dwords (x_p, x_p+8) of each unit into its
    // A fragment slot, and the unit's offset sum
#pragma unroll
    for (int j = 0; j < kUnitsPerThread; ++j) {
        const int e = (int)threadIdx.x + j * kSThreads;
        if (e >= nunits) break;
        const int m = e % MR, r = e / MR;
        const int wl = r >> 4, u16 = r & 15, g = u16 >> 3, u8 = u16 & 7;
        const int ut = m >> 4, mm = m & 15;  // activation tile, row in it
        uint32_t pr[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // v_perm_b32: bytes 0-3 select from the second source, 4-7 from the first
            pr[2 * i] = __builtin_amdgcn_perm(xhi[j][i], xlo[j][i], 0x05040100u);      // (x_2i, x_2i+8)
            pr[2 * i + 1] = __builtin_amdgcn_perm(xhi[j][i], xlo[j][i], 0x07060302u);  // (x_2i+1, x_2i+9)
        }
        const int sg = u8 >> 1, qq = ((sg & 1) << 1) | (sg >> 1), c0 = 2 * (u8 & 1);
        u32x4 *dst = xf + (((wl * 2 + g) * MT + ut) * 4 + c0) * 64 + 16 * qq + mm;
        dst[0] = u32x4{pr[0], pr[1], pr[2], pr[3]};
        dst[64] = u32x4{pr[4], pr[5], pr[6], pr[7]};
        float c = 0.0f;
#pragma unroll
        for (int p = 0; p < 8; ++p)
            c = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, pr[p]), __builtin_bit_cast(half2_t, sslot_w(p)),
                                       c, false);
        cpart[((wl * 2 + g) * 8 + u8) * MR + m] = c;
    }
    __syncthreads();
    for (int e = (int)threadIdx.x; e < SW * 2 * MR; e += kSThreads) {
        const float *src = cpart + (e / MR) * 8 * MR + e % MR;
        float c = 0.0f;
#pragma unroll
        for (int u = 0; u < 8; ++u) c += src[MR * u];
        cneg[e] = -c;
    }
    __syncthreads();

    // ---- 3. window pairs, PF at a time from the ring; slots past the slice
    // only reload its last pair (the loads stay unconditional, so the
    // compiler's waits are exact)
    const uint32_t m8 = svreg(0x03000300u), m6 = svreg(0x00C000C0u);
    f32x4 acc[NT][MT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int u = 0; u < MT; ++u) acc[t][u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int w0 = 0; w0 < NPR; w0 += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            const int wp = w0 + p;
            u32x4 cwp[NT][2];
            uint32_t svp[NT][2];
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    cwp[t][h] = rc[p][t][h];
                    svp[t][h] = rsc[p][t][h];
                }
            load_pair(p, min(wp + PF, NPR - 1));
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int wl = 2 * wp + h;
                if (wl >= SW) continue;  // wave-uniform: past the slice
                // v_permlane32_swap exchanges the upper 32 lanes of its first
                // operand with the lower 32 lanes of its second: afterwards
                // every lane holds its segment of the first group in dwords
                // 0, 1 and of the second group in dwords 2, 3
                uint32_t gd[NT][2][2];
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const auto e0 = __builtin_amdgcn_permlane32_swap(cwp[t][h][0], cwp[t][h][2], false, false);
                    const auto e1 = __builtin_amdgcn_permlane32_swap(cwp[t][h][1], cwp[t][h][3], false, false);
                    gd[t][0][0] = e0[0];
                    gd[t][0][1] = e1[0];
                    gd[t][1][0] = e0[1];
                    gd[t][1][1] = e1[1];
                }
#pragma unroll
                for (int g = 0; g < 2; ++g) {
                    // each tile's weights decoded once, used by every activation tile
                    uint32_t wd[NT][16];
                    float sc[NT];
#pragma unroll
                    for (int t = 0; t < NT; ++t) {
                        uint32_t wa[8], wq[8];
                        sdecode(gd[t][g][0], m8, m6, wa);
                        sdecode(gd[t][g][1], m8, m6, wq);
#pragma unroll
                        for (int i = 0; i < 8; ++i) {
                            wd[t][i] = wa[i];
                            wd[t][8 + i] = wq[i];
                        }
                        sc[t] = (float)__builtin_bit_cast(_Float16, (uint16_t)(g ? svp[t][h] >> 16 : svp[t][h]));
                    }
#pragma unroll
                    for (int u = 0; u < MT; ++u) {
                        const u32x4 *af = xf + ((wl * 2 + g) * MT + u) * 256 + lane;
                        const u32x4 a0 = af[0], a1 = af[64], a2 = af[128], a3 = af[192];
                        const f32x4 cn =
                            *reinterpret_cast<const f32x4 *>(cneg + (wl * 2 + g) * MR + 16 * u + 4 * q);
#pragma unroll
                        for (int t = 0; t < NT; ++t) {
                            f32x4 D = cn;
                            D = mfma16(a0, u32x4{wd[t][0], wd[t][1], wd[t][2], wd[t][3]}, D);
                            D = mfma16(a1, u32x4{wd[t][4], wd[t][5], wd[t][6], wd[t][7]}, D);
                            D = mfma16(a2, u32x4{wd[t][8], wd[t][9], wd[t][10], wd[t][11]}, D);
                            D = mfma16(a3, u32x4{wd[t][12], wd[t][13], wd[t][14], wd[t][15]}, D);
#pragma unroll
                            for (int i = 0; i < 4; ++i) acc[t][u][i] = __builtin_fmaf(sc[t], D[i], acc[t][u][i]);
                        }
                    }
                }
            }
        }
    }

    // ---- 4. outputs: lane (n, q) holds rows 4q + i of weight row n; with
    // several slices, this slice's partial Y in the workspace
    float *dst = KS == 1 ? Y : ws + (size_t)ks * M * N;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int row = 16 * (tile0 + t) + n;
#pragma unroll
        for (int u = 0; u < MT; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 16 * u + 4 * q + i;
                if (m < M && row < N) dst[(size_t)m * N + row] = acc[t][u][i] * kSInvUnit;
            }
    }
}

// Y = the KS partials added in slice order.
__global__ __launch_bounds__(256) void split_reduce_kernel(const float *__restrict__ ws, float *__restrict__ Y,
                                                           int MN, int KS) {
    const int e = blockIdx.x * 256 + (int)threadIdx.x;
    if (e >= MN) return;
    float y = 0.0f;
    for (int k = 0; k < KS; ++k) y += ws[(size_t)k * MN + e];
    Y[e] = y;
}

// The same sums four outputs per thread (16-byte loads and store), in the
// same order from the same zero start, so the bits match the scalar kernel:
// for MN divisible by 4 (every slice 16-byte aligned) and a 16-byte aligned
// Y.  Eight slices' loads are issued before their adds.
__global__ __launch_bounds__(256) void split_reduce4_kernel(const f32x4 *__restrict__ ws, f32x4 *__restrict__ Y,
                                                            int MN4, int KS) {
    const int e = blockIdx.x * 256 + (int)threadIdx.x;
    if (e >= MN4) return;
    f32x4 y = {0.0f, 0.0f, 0.0f, 0.0f};
    int k = 0;
    for (; k + 8 <= KS; k += 8) {
        f32x4 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = ws[(size_t)(k + j) * MN4 + e];
#pragma unroll
        for (int j = 0; j < 8; ++j) y += v[j];
    }
    for (; k < KS; ++k) y += ws[(size_t)k * MN4 + e];
    Y[e] = y;
}

struct SplitPlan {
    bool ok = false;
    int nt = 0, mt = 0;
    int64_t nblk = 0, kslices = 0;
    size_t ws_bytes = 0;
};

// 5 <= M <= 64 ternary with an even group count, N <= 131072 and 32-bit
// buffer offsets; MT = 1, 2 or 4 activation tiles of 16 rows.  Shape: the
// fewest K slices that fit LDS (more slices measured slower: every
// workgroup pays the activation staging).
// TQ_GEMM_SPLIT = "off" disables the kernel, "NT,KS" fixes the shape (for
// measurements).
SplitPlan split_plan(int64_t M, int64_t N, int64_t K, int32_t variant) {
    static const int forced_nt = [] {
        const char *v = getenv("TQ_GEMM_SPLIT");
        if (!v) return 0;
        return v[0] == 'o' ? -1 : atoi(v);
    }();
    static const int forced_ks = [] {
        const char *v = getenv("TQ_GEMM_SPLIT");
        const char *c = v ? strchr(v, ',') : nullptr;
        return c ? atoi(c + 1) : 0;
    }();
    SplitPlan pl;
    if (forced_nt < 0 || variant != TQ_TERNARY || M < 5 || M > 64 || K < 256 || (K / 128) % 2) return pl;
    const int64_t W = K / 256, ntiles = (N + 15) / 16;
    // very tall matrices keep the batched kernel of tq_gemm.hip: on the
    // 248320-row head with 8 rows it ran 113 us against 127 us here, the
    // staging and the K-split partials growing with N
    if (forced_nt == 0 && N > 131072) return pl;
    pl.mt = M <= 16 ? 1 : M <= 32 ? 2 : 4;
    // two weight tiles per wave for one activation tile, three for two or
    // four: with the VGPRs these take, one workgroup runs per CU, and three
    // tiles keep the MLP shapes to one round of workgroups (32 / 64 rows on
    // 17408 x 5120: 22.4 / 32.5 us against 26.5 / 41.2 with two tiles)
    pl.nt = forced_nt >= 1 && forced_nt <= 4 ? forced_nt : pl.mt == 1 ? 2 : 3;
    pl.nblk = (ntiles + kSWaves * pl.nt - 1) / (kSWaves * pl.nt);
    const int64_t maxw = split_max_win(pl.mt);
    const int64_t ks_min = (W + maxw - 1) / maxw;
    pl.kslices = std::min<int64_t>(W, std::max<int64_t>(ks_min, forced_ks));
    if (pl.nblk * kSWaves * pl.nt * 16 * (K / 4) >= (int64_t(1) << 31)) return pl;
    if (pl.kslices * M * N >= (int64_t(1) << 31)) return pl;
    pl.ws_bytes = pl.kslices > 1 ? (size_t)(pl.kslices * M * N) * sizeof(float) : 0;
    pl.ok = true;
    return pl;
}

}  // namespace

// Workspace bytes the split kernel needs for this shape (0: none, or the
// shape is not one it takes).
size_t gemm_split_ws_bytes(int64_t M, int64_t N, int64_t K, int32_t variant) {
    const SplitPlan pl = split_plan(M, N, K, variant);
    return pl.ok ? pl.ws_bytes : 0;
}

// *handled is false when the shape is not one the kernel takes or the
// workspace (ws, ws_bytes; may be NULL / 0) is smaller than it needs.
int32_t gemm_split_enqueue(const uint8_t *codes, const uint16_t *scales, const uint16_t *X, float *Y, int64_t M,
                           int64_t N, int64_t K, int32_t variant, float *ws, size_t ws_bytes, hipStream_t stream,
                           bool *handled) {
    *handled = false;
    const SplitPlan pl = split_plan(M, N, K, variant);
    if (!pl.ok || (pl.ws_bytes && (!ws || ws_bytes < pl.ws_bytes))) return TQ_OK;
    *handled = true;
    const int64_t W = K / 256;
    const int64_t sw_max = (W + pl.kslices - 1) / pl.kslices;
    const size_t lds = (size_t)sw_max * pl.mt * kSWinLds;
    const dim3 grid((unsigned)pl.nblk, (unsigned)pl.kslices), block(kSThreads);
    const int m = (int)M, n = (int)N, k = (int)K, kk = (int)pl.kslices;
#define TQ_SPLIT(NT_, MT_)                                                                                   \
    hipLaunchKernelGGL((gemm_split_kernel<NT_, 2, MT_>), grid, block, lds, stream, codes, scales, X, Y, ws, m, \
                       n, k, kk)
    if (pl.nt == 2) {
        if (pl.mt == 1) TQ_SPLIT(2, 1);
        else if (pl.mt == 2) TQ_SPLIT(2, 2);
        else TQ_SPLIT(2, 4);
    } else if (pl.nt == 3) {
        if (pl.mt == 1) TQ_SPLIT(3, 1);
        else if (pl.mt == 2) TQ_SPLIT(3, 2);
        else TQ_SPLIT(3, 4);
    } else if (pl.nt == 4) {
        if (pl.mt == 1) TQ_SPLIT(4, 1);
        else if (pl.mt == 2) TQ_SPLIT(4, 2);
        else TQ_SPLIT(4, 4);
    } else {
        if (pl.mt == 1) TQ_SPLIT(1, 1);
        else if (pl.mt == 2) TQ_SPLIT(1, 2);
        else TQ_SPLIT(1, 4);
    }
#undef TQ_SPLIT
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && kk > 1) {
        const int mn = m * n;
        // four outputs per thread from five slices up (measured: 17408 x 5120
        // at 64 rows, 5 slices, 32.6 -> 30.6 us per call; 5120 x 17408 at 16
        // rows, 9 slices, 19.0 -> 17.7 us); with three slices one output per
        // thread measured 0.4 us faster
        if (kk >= 5 && mn % 4 == 0 && (reinterpret_cast<uintptr_t>(Y) & 15) == 0) {
            const int mn4 = mn / 4;
            hipLaunchKernelGGL(split_reduce4_kernel, dim3((unsigned)((mn4 + 255) / 256)), dim3(256), 0, stream,
                               reinterpret_cast<const f32x4 *>(ws), reinterpret_cast<f32x4 *>(Y), mn4, kk);
        } else {
            hipLaunchKernelGGL(split_reduce_kernel, dim3((unsigned)((mn + 255) / 256)), dim3(256), 0, stream, ws, Y,
                               mn, kk);
        }
        e = hipGetLastError();
    }
    if (e != hipSuccess) return fail(TQ_ERR_HIP, "GEMM launch failed: %s", hipGetErrorString(e));
    return TQ_OK;
}

}  // namespace tq
