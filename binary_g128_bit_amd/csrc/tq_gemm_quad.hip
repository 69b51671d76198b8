// Small-batch GEMM for M <= 8 activation rows over packed ternary / binary
// g128 weights, gfx950.
//
// Y[m][n] = sum_g s[n][g] * sum_{j<128} t[n][128g+j] * X[m][128g+j]
// (w_i = s_g * t_i with one FP16 scale per 128 weights: thakicloud.github.io,
// "Bonsai 27B: ternary and 1-bit quantization", "How the compression works";
// the packed slots are consumed directly and the scale is applied inside the
// matmul: aitrends.kr, "Ternary-Bonsai-27B-mlx-2bit", "Technical features").
// Widths 2-4 are the speculative-verify batches (the same page of
// thakicloud.github.io, "Throughput and speculative decoding": k = 4 drafted
// tokens are checked at once).
//
// Matrix cores.  v_mfma_f32_4x4x4_16b_f16 runs 16 independent 4x4x4 products;
// product b lives on lanes 4b..4b+3: lane 4b+i supplies row i of A (four
// halves), lane 4b+j column j of B, and lane 4b+j receives D[i][j] in its
// register i.  Here A row i is activation row m = i and B column j is weight
// row j of a 4-row block, both over the same four K positions, so every
// product is useful: the decode of a weight is paid once for the 4 rows.
// Lane 4b+j therefore reads activation row j & 3 and decodes weight row j & 3
// of its block; the 16 products of one instruction are 16 different 16-byte
// code chunks (columns) of the same 4 weight rows, so one 16-byte load per
// lane reads 4 rows x 256 contiguous bytes.  For 5..8 rows a second row set
// (activation rows 4..7) takes a second chain of products on the same
// decoded weights, so the decode is paid once for 8 rows.
//
// Decode (exact).  As in the batch-1 GEMV: ternary codes placed in FP16
// exponent / mantissa bits are linear in the code (E: c 2^-14; M4: 2^-12 +
// c 2^-14; M16: 2^-10 + c 2^-14), binary bits likewise (bit 11: b 2^-13, bit
// q <= 10 under exponent 12 - q: 2^(-3-q) + b 2^-13).  The offsets and the
// shift t = c - 1 (t = 2b - 1) are removed by starting each chunk's MFMA
// chain from C = -sum_k w_k x_k * 2^-14 with w = 1 + offset (ternary) or
// 2 offset + 1 (binary): a per-(activation row, chunk) seed computed while
// the activations are staged, so D = 2^-14 sum t x.  One FP32 multiply-add
// per chunk applies the group scale; the row total is scaled by 2^14 once.
//
// Activations.  The workgroup stages X once into LDS as pair dwords
// (x_p, x_{p+8}) (ternary, per 16-weight unit) or (x_p, x_{p+16}) (binary,
// per 32-weight unit), the pairing the decode produces, 16-byte pieces
// XOR-swizzled so that the 16 lanes of an LDS read (4 chunks x 4 activation
// rows) hit distinct banks; rows m >= M and chunks past the row are zeros and
// contribute exactly nothing.  A chunk is 16 code bytes: 64 ternary or 128
// binary weights.
//
// Work split.  Each workgroup (16 waves) stages X once and takes an equal
// range of 4-row blocks, in one round of one workgroup per CU.  Its items are
// (chunk group i, block) pairs in i-major order; every wave takes a
// contiguous range of them, so all waves have equal work whatever the block
// count, and consecutive items of a wave share the activation fragment (one
// LDS read per group) while the weight rows change.  An item's 4 x 4 partial
// is summed over the instruction's columns by DPP within 16-lane rows and
// stored to LDS per row group; at the end the partials of each block are
// added in a fixed order (deterministic) and stored.
//
// Measured on the MLP shapes (MI355X, same box, back to back): M = 4 on
// 17408 x 5120 takes 10.2 us and on 5120 x 17408 12.2 us, against 8.1 /
// 8.2 us for the batch-1 GEMV.  Wave timestamps (17408 x 5120 / 5120 x
// 17408): the items start 3.3 / 4.5 us into the launch, after the staging
// and its barrier; a wave's item takes about 0.6 us of its time with 4 waves
// per SIMD, the decode (40 VALU ops), the sums (13) and the 16 MFMA issues.
// Loading each lane's own fragment instead of staging (no barrier) measured
// 35 % slower: every 16-byte load then touches 64 cache lines, and the
// fragments shared by two waves are read twice.
#include <hip/hip_runtime.h>

#include <cstdlib>
#include <type_traits>

#include "tq_internal.h"

namespace tq {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kQWaves = 16;            // waves per workgroup
constexpr int kQThreads = 64 * kQWaves;
// chunk items in flight per wave: four with one row set, three with two
// (whose second set of activation registers leaves no room for a fourth)
constexpr int q_prefetch(int MR) { return MR == 1 ? 4 : 3; }
constexpr int kQMaxLds = 163840;       // bytes of LDS a gfx950 workgroup may use
constexpr int kQRows = 4;              // activation rows per MFMA operand (a row set)
constexpr float kUnit = 6.103515625e-05f;  // 2^-14
constexpr float kInvUnit = 16384.0f;

__device__ __forceinline__ uint32_t vreg(uint32_t v) {
    asm volatile("" : "+v"(v));
    return v;
}

// Pins four values in registers at this point (no contraction or sinking
// across it).
__device__ __forceinline__ void fbar4(float (&v)[4]) {
    asm volatile("" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]));
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c, false);
}

__device__ __forceinline__ f32x4 mfma4(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1, f32x4 d) {
    return __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(half4_t, u32x2{a0, a1}),
                                             __builtin_bit_cast(half4_t, u32x2{b0, b1}), d, 0, 0, 0);
}

template <int VARIANT>
struct QFmt;

// Ternary: a 16-byte chunk is four 16-weight units (one code dword each), a
// unit gives pairs p = 0..7 of (weight p, weight p + 8).
template <>
struct QFmt<TQ_TERNARY> {
    static constexpr int kWeights = 64;          // per chunk
    static constexpr int kUnit = 16;             // weights per code dword
    // seed weight 1 + offset of pair p, as an FP16 pair: M16 slots 0, 3
    // (17), M4 slots 1, 4, 6 (5), E slots 2, 5, 7 (1)
    static __device__ __forceinline__ uint32_t zw(int p) {
        return (p == 0 || p == 3) ? 0x4C404C40u : (p == 1 || p == 4 || p == 6) ? 0x45004500u : 0x3C003C00u;
    }
};

// Binary: a chunk is 8 code bytes, two 32-weight units, a unit gives pairs
// p = 0..15 of (weight p, weight p + 16).
template <>
struct QFmt<TQ_BINARY> {
    static constexpr int kWeights = 64;
    static constexpr int kUnit = 32;
    // 2 offset + 1 for the slot that reads pair p: copies d << 6 (pairs 5..0
    // at bits 11..6), d (pairs 11..6) and d >> 4 (pairs 15..12 at bits 11..8)
    static __device__ __forceinline__ uint32_t zw(int p) {
        constexpr uint32_t w[16] = {0x50205020u, 0x4C404C40u, 0x48804880u, 0x45004500u,
                                    0x42004200u, 0x3C003C00u, 0x50205020u, 0x4C404C40u,
                                    0x48804880u, 0x45004500u, 0x42004200u, 0x3C003C00u,
                                    0x48804880u, 0x45004500u, 0x42004200u, 0x3C003C00u};
        return w[p];
    }
};

// LDS position (in 16-byte pieces) of piece q of chunk slot (m, c).  A slot
// is 8 pieces, half the 64 banks.  The 16 lanes served together read chunks
// c0..c0+3 of the 4 activation rows of one row set: (c & 1) picks the half
// and the XOR key (m & 3) + 4 ((c >> 1) & 1) spreads the 8 lanes that share
// it.
__device__ __forceinline__ int piece_at(int m, int c, int q, int capc) {
    return (m * capc + c) * 8 + (q ^ ((m & 3) + 4 * ((c >> 1) & 1)));
}

// The 16 ternary weights of code dword d as 8 pair dwords w[p], p = 0..7.
__device__ __forceinline__ void tern_decode(uint32_t d, uint32_t m8, uint32_t m6, uint32_t (&w)[8]) {
    const uint32_t c6 = d << 6, r4 = d >> 4;
    w[0] = (c6 & m6) | 0x14001400u;  // M16
    w[1] = (c6 & m8) | 0x0C000C00u;  // M4
    w[2] = c6 & 0x0C000C00u;         // E
    w[3] = (d & m6) | 0x14001400u;
    w[4] = (d & m8) | 0x0C000C00u;
    w[5] = d & 0x0C000C00u;
    w[6] = (r4 & m8) | 0x0C000C00u;
    w[7] = r4 & 0x0C000C00u;
}

struct BinMasks {
    uint32_t b10, b9, b8, b7, b6;
    __device__ __forceinline__ BinMasks()
        : b10(vreg(0x04000400u)), b9(vreg(0x02000200u)), b8(vreg(0x01000100u)), b7(vreg(0x00800080u)),
          b6(vreg(0x00400040u)) {}
};

// The 32 binary weights of code dword d as 16 pair dwords w[p].
__device__ __forceinline__ void bin_decode(uint32_t d, const BinMasks &k, uint32_t (&w)[16]) {
    const uint32_t src[3] = {d << 6, d, d >> 4};
    const int top[3] = {5, 11, 15};
#pragma unroll
    for (int s = 0; s < 3; ++s) {
        const uint32_t c = src[s];
        const int t = top[s];
        w[t] = c & 0x08000800u;                 // bit 11
        w[t - 1] = (c & k.b10) | 0x08000800u;   // bit 10
        w[t - 2] = (c & k.b9) | 0x0C000C00u;    // bit 9
        w[t - 3] = (c & k.b8) | 0x10001000u;    // bit 8
        if (s < 2) {
            w[t - 4] = (c & k.b7) | 0x14001400u;  // bit 7
            w[t - 5] = (c & k.b6) | 0x18001800u;  // bit 6
        }
    }
}

__device__ __forceinline__ float half_bits(uint32_t bits) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

// DPP move within 16-lane rows.  bound_ctrl is set: the permutations used
// here (rotations, quad permutes) leave no lane without a source, and with it
// the compiler folds the move into the add that consumes it.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF,
                                                                 true));
}

// v + (v of the lane W = 16 or 32 away, within 2W-lane groups), as
// v_permlane16/32_swap of v with itself: the swap leaves the lane's own value
// in one result and its partner's in the other (even 16-lane rows or the
// lower half: own value first), so the sum is the one a lane-xor shuffle
// gives, without the LDS crossbar.
template <int W>
__device__ __forceinline__ float swap_sum(float v) {
    const uint32_t u = __builtin_bit_cast(uint32_t, v);
    const auto e = W == 16 ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                           : __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __builtin_bit_cast(float, (uint32_t)e[0]) + __builtin_bit_cast(float, (uint32_t)e[1]);
}

// Stage X into LDS: one 16- or 32-weight unit per work item, the units of a
// chunk on consecutive threads, activation row m, chunk c; pairs as the
// decode produces them and each (row, chunk) seed.  Every thread of the
// workgroup runs the loop (the seed sum is a cross-lane op).
// Staged activation units of one thread: UMAX units of 16 (ternary) or 32
// (binary) weights, activation row m, chunk c; the units of a chunk sit on
// consecutive threads.
template <int VARIANT, int UMAX, int MR>
struct StageX {
    static constexpr int ROWS = kQRows * MR;              // staged activation rows
    using F = QFmt<VARIANT>;
    static constexpr int UPC = F::kWeights / F::kUnit;  // units per chunk: 4 or 2
    static constexpr int V4 = F::kUnit / 8;             // 16-byte loads per unit
    static constexpr int HP = F::kUnit / 2;             // pairs per unit
    u32x4 v[UMAX][V4];

    // every load first: they are issued before the code prologue, so the
    // wait for them does not cover the code stream
    __device__ __forceinline__ void load(const uint16_t *__restrict__ X, int M, int K, int CPR, int capc) {
        const int units = ROWS * capc * UPC;
#pragma unroll
        for (int k = 0; k < UMAX; ++k) {
            const int uu = k * kQThreads + (int)threadIdx.x;
            const int u = uu % UPC, mc = min(uu / UPC, ROWS * capc - 1);
            const int m = mc / capc, c = mc % capc;
            const bool real = uu < units && m < M && c < CPR;
            const u32x4 *src = reinterpret_cast<const u32x4 *>(X + (size_t)min(m, M - 1) * K +
                                                                (size_t)min(c, CPR - 1) * F::kWeights + u * F::kUnit);
#pragma unroll
            for (int i = 0; i < V4; ++i) v[k][i] = real ? src[i] : u32x4{0u, 0u, 0u, 0u};
        }
    }

    // pairs as the decode produces them and each (row, chunk) seed into LDS
    // (seeds[set][chunk], one f32x4 for the set's 4 rows); every thread runs
    // it (the seed sum is a cross-lane op)
    __device__ __forceinline__ void store(u32x4 *xs, f32x4 *seeds, int capc) const {
        const int units = ROWS * capc * UPC;
#pragma unroll
        for (int k = 0; k < UMAX; ++k) {
            const int uu = k * kQThreads + (int)threadIdx.x;
            const int u = uu % UPC, mc = min(uu / UPC, ROWS * capc - 1);
            const int m = mc / capc, c = mc % capc;
            uint32_t xp[HP];
#pragma unroll
            for (int i = 0; i < HP / 2; ++i) {
                const uint32_t lo = v[k][i / 4][i % 4], hi = v[k][V4 / 2 + i / 4][i % 4];
                xp[2 * i] = (lo & 0xFFFFu) | (hi << 16);
                xp[2 * i + 1] = (lo >> 16) | (hi & 0xFFFF0000u);
            }
            float z = 0.0f;
#pragma unroll
            for (int i = 0; i < HP; ++i) z = dot2(xp[i], F::zw(i), z);
            z += dpp_f<0xB1>(z);                // quad_perm [1,0,3,2]
            if (UPC == 4) z += dpp_f<0x4E>(z);  // quad_perm [2,3,0,1]
            if (uu < units) {
#pragma unroll
                for (int i = 0; i < HP / 4; ++i)
                    xs[piece_at(m, c, u * (HP / 4) + i, capc)] =
                        u32x4{xp[4 * i], xp[4 * i + 1], xp[4 * i + 2], xp[4 * i + 3]};
                if (u == 0) reinterpret_cast<float *>(seeds)[((m >> 2) * capc + c) * 4 + (m & 3)] = -z * kUnit;
            }
        }
    }
};

// One item's 16 MFMAs per row set: the chunk's 64 decoded weights of this
// lane's row against each set's activation pairs xa[set], each chain started
// from its set's seeds.  D[set] = 2^-14 sum t x for the set's 4 activation
// rows (register i) of this lane's weight row; the decode is paid once for
// all sets.
template <int VARIANT, int MR, typename Code>
__device__ __forceinline__ void item_mma(const Code &cw, const u32x4 (&xa)[MR][8], const f32x4 (&sd)[MR],
                                         uint32_t m8, uint32_t m6, const BinMasks &bk, f32x4 (&D)[MR]) {
#pragma unroll
    for (int s = 0; s < MR; ++s) D[s] = sd[s];
    if constexpr (VARIANT == TQ_TERNARY) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            uint32_t w[8];
            tern_decode(cw[u], m8, m6, w);
#pragma unroll
            for (int h = 0; h < 4; ++h)
#pragma unroll
                for (int s = 0; s < MR; ++s)
                    D[s] = mfma4(xa[s][2 * u + h / 2][2 * (h % 2)], xa[s][2 * u + h / 2][2 * (h % 2) + 1], w[2 * h],
                                 w[2 * h + 1], D[s]);
        }
    } else {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            uint32_t w[16];
            bin_decode(cw[u], bk, w);
#pragma unroll
            for (int h = 0; h < 8; ++h)
#pragma unroll
                for (int s = 0; s < MR; ++s)
                    D[s] = mfma4(xa[s][4 * u + h / 2][2 * (h % 2)], xa[s][4 * u + h / 2][2 * (h % 2) + 1], w[2 * h],
                                 w[2 * h + 1], D[s]);
        }
    }
}

// Kernel.  CPR: 64-weight chunks per row; capc: CPR rounded up to 16 (chunk
// slots per staged activation row); NI = capc / 16 chunk groups.  Items are
// (chunk group i, block) pairs in i-major order; a wave takes a contiguous
// range of them, so consecutive items share the activation fragment (read
// from LDS once per group) and differ in the 4 weight rows.  Each item's
// 4 x 4 partial, summed over the 4 instruction columns of each 16-lane row
// (DPP), goes to LDS as RP row-group partials (RP = 2 adds the two row pairs
// first, one cross-lane move per value, when LDS is short); the end adds
// the NI * RP partials of every block in a fixed order.
//
// Codes and scales are read through buffer descriptors: an offset past the
// matrix returns zeros, so rows past N (the last block) need no clamp, and
// chunk slots past a ragged row read bytes that meet zero activations.
template <int VARIANT, int UMAX, int RP, int MR>
__global__ __launch_bounds__(kQThreads) void gemm_quad_kernel(const uint8_t *__restrict__ codes,
                                                              const uint16_t *__restrict__ scales,
                                                              const uint16_t *__restrict__ X,
                                                              float *__restrict__ Y, int M, int N, int K,
                                                              int blocks_per_wg) {
    typedef typename std::conditional<VARIANT == TQ_TERNARY, u32x4, u32x2>::type Code;
    extern __shared__ u32x4 lds[];
    const int G = K >> 7;
    const int CPR = K >> 6;
    const int capc = (CPR + 15) & ~15;
    const int NI = capc >> 4;
    constexpr int PW = 16 * MR;  // partial floats per item and row group
    u32x4 *xs = lds;                                                         // [4 MR][capc][8 pieces]
    f32x4 *seeds = reinterpret_cast<f32x4 *>(lds + kQRows * MR * capc * 8);  // [MR][capc]
    float *part = reinterpret_cast<float *>(seeds + MR * capc);             // [NI][blocks][RP][PW]

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int q4 = lane & 3, b = lane >> 2;
    const int nblocks = (N + 3) >> 2;
    const int blk0 = blockIdx.x * blocks_per_wg;
    const int nb = max(0, min(blocks_per_wg, nblocks - blk0));
    const int items = nb * NI;
    const int it0 = (int)(((long long)wave * items) / kQWaves);
    const int it1 = (int)(((long long)(wave + 1) * items) / kQWaves);
    const int nit = it1 - it0;

    // ---- activation loads first (L2), then this wave's first code chunks
    // (HBM), so that the staging below waits for the activations only
    StageX<VARIANT, UMAX, MR> sx;
    sx.load(X, M, K, CPR, capc);

    constexpr int CB = sizeof(Code);  // code bytes per chunk
    const int row_bytes = CPR * CB;
    const __amdgpu_buffer_rsrc_t crs =
        __builtin_amdgcn_make_buffer_rsrc((void *)codes, 0, N * row_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t srs =
        __builtin_amdgcn_make_buffer_rsrc((void *)scales, 0, N * G * 2, 0x00020000);
    constexpr int kQPrefetch = q_prefetch(MR);
    constexpr int kQRing = kQPrefetch + 1;  // ring slots: one spare, see the item loop
    Code ring[kQRing];
    uint32_t sring[kQRing];
    // issue pointer: (group i, block lb) of the next item to load, advanced
    // in i-major order and held at the last item once the range is spent
    int ii = nb > 0 ? it0 / nb : 0, il = nb > 0 ? it0 - ii * nb : 0, left = nit;
    // byte offsets of the next item's code chunk and scale, stepped by one
    // block (4 rows) per item and recomputed when the group changes
    const int row0 = 4 * blk0 + q4;
    int coff = (row0 + 4 * il) * row_bytes + (b + 16 * ii) * CB;
    int soff = ((row0 + 4 * il) * G + ((b + 16 * ii) >> 1)) * 2;
    auto issue = [&](int slot) __attribute__((always_inline)) {
        if constexpr (VARIANT == TQ_TERNARY)
            ring[slot] = __builtin_bit_cast(Code, __builtin_amdgcn_raw_buffer_load_b128(crs, coff, 0, 0));
        else
            ring[slot] = __builtin_bit_cast(Code, __builtin_amdgcn_raw_buffer_load_b64(crs, coff, 0, 0));
        sring[slot] = __builtin_amdgcn_raw_buffer_load_b16(srs, soff, 0, 0);
        if (left > 1) {
            --left;
            if (++il == nb) {
                il = 0;
                ++ii;
                coff = row0 * row_bytes + (b + 16 * ii) * CB;
                soff = (row0 * G + ((b + 16 * ii) >> 1)) * 2;
            } else {
                coff += 4 * row_bytes;
                soff += 8 * G;
            }
        }
    };
    // half the ring before the staging, half after its barrier: with the
    // whole ring in flight the code stream (most of a short range) competes
    // with the activation reads that every item waits for
#pragma unroll
    for (int p = 0; p < kQPrefetch / 2; ++p) issue(p);

    sx.store(xs, seeds, capc);
    __syncthreads();
#pragma unroll
    for (int p = kQPrefetch / 2; p < kQPrefetch; ++p) issue(p);

    // ---- items: lane 4b+j decodes weight row 4 blk + j at chunk b + 16 i and
    // supplies activation row j of that chunk.  The loads are unconditional
    // (loads under a branch made the compiler merge the ring registers with
    // moves at the loop latch, which wait for every load in flight); only
    // the compute of the last round's items past the range is skipped.
    const uint32_t m8 = vreg(0x03000300u), m6 = vreg(0x00C000C0u);
    const BinMasks bk;
    int cur_i = -1;
    u32x4 xa[MR][8];
    f32x4 sd[MR];
    int i = nb > 0 ? it0 / nb : 0, lb = nb > 0 ? it0 - i * nb : 0;  // compute pointer
    // Item p of an unrolled round reads slot p and refills slot p - 1, read
    // by the item before: the load never targets a register still in use, so
    // the slots keep their registers across the loop latch.  (With the
    // refill in the slot being read, the scheduler hoists the load above the
    // decode, and the ring rotates through register moves at the latch that
    // wait for every load in flight.)
    for (int t0 = 0; t0 < nit; t0 += kQRing) {
#pragma unroll
        for (int p = 0; p < kQRing; ++p) {
            const int t = t0 + p;
            if (i != cur_i) {  // wave-uniform: a new chunk group's activations and seeds
                const int c = b + 16 * i;
#pragma unroll
                for (int rs = 0; rs < MR; ++rs) {
#pragma unroll
                    for (int q = 0; q < 8; ++q) xa[rs][q] = xs[piece_at(4 * rs + q4, c, q, capc)];
                    sd[rs] = seeds[rs * capc + c];
                }
                cur_i = i;
            }
            const Code cw = ring[p];
            const float s = half_bits(sring[p]);
            issue((p + kQRing - 1) % kQRing);
            if (t < nit) {  // wave-uniform: the last round's items past the range only load
                f32x4 D[MR];
                item_mma<VARIANT, MR>(cw, xa, sd, m8, m6, bk, D);
                // the scaled partial stays a separate product (no contraction
                // into the adds) and the sum is formed before the store branch,
                // so that each add takes its cross-lane operand as a DPP source
                float v[MR][4];
#pragma unroll
                for (int rs = 0; rs < MR; ++rs) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) v[rs][r] = s * D[rs][r];
                    fbar4(v[rs]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) v[rs][r] += dpp_f<0x124>(v[rs][r]);  // row_ror:4
#pragma unroll
                    for (int r = 0; r < 4; ++r) v[rs][r] += dpp_f<0x128>(v[rs][r]);  // row_ror:8
                    fbar4(v[rs]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        if (RP <= 2) v[rs][r] = swap_sum<16>(v[rs][r]);
                        if (RP == 1) v[rs][r] = swap_sum<32>(v[rs][r]);
                    }
                }
                // lanes 0-3 of each (RP = 4) or every other (RP = 2) 16-lane
                // row hold their rows' sums for weight row j
                const int grp = lane >> 4;
                if ((lane & 15) < 4 && (RP == 4 || (RP == 2 && (grp & 1) == 0) || grp == 0)) {
                    float *dst = part + ((size_t)(i * nb + lb) * RP + (RP == 4 ? grp : grp >> 1)) * PW;
#pragma unroll
                    for (int rs = 0; rs < MR; ++rs)
#pragma unroll
                        for (int r = 0; r < 4; ++r) dst[rs * 16 + r * 4 + q4] = v[rs][r];
                }
            }
            if (t + 1 < nit && ++lb == nb) {  // next item (held at the last one)
                lb = 0;
                ++i;
            }
        }
    }
    __syncthreads();

    // ---- per (block, activation row, weight row): the partials in a fixed order
    for (int e = (int)threadIdx.x; e < nb * PW; e += kQThreads) {
        const int lb = e / PW, w = e % PW;  // w = 16 set + 4 (row in set) + weight row
        const int m = 4 * (w >> 4) + ((w >> 2) & 3), j = w & 3;
        const int row = 4 * (blk0 + lb) + j;
        float y = 0.0f;
        for (int i = 0; i < NI; ++i) {
            const float *src = part + (size_t)(i * nb + lb) * RP * PW;
#pragma unroll
            for (int g = 0; g < RP; ++g) y += src[g * PW + w];
        }
        if (m < M && row < N) Y[(size_t)m * N + row] = y * kInvUnit;
    }
}

}  // namespace

// LDS bytes of the staged activations and seeds of MR row sets for K.
size_t gemm_quad_stage_lds(int64_t K, int MR) {
    const int64_t capc = (K / 64 + 15) / 16 * 16;
    return (size_t)(MR * (kQRows * capc * 8 * 16 + capc * 16));
}

int device_cu_count() {
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cache[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev] = n;
    }
    return cache[dev];
}

// M <= 8 on the quad kernel (one row set for M <= 4, two for 5..8) when the
// staged activations and at least one block's partials fit LDS (two sets:
// in one round of workgroups) and the packed matrix is below 2^31 bytes
// (32-bit buffer offsets); *handled is false otherwise.  Blocks are dealt to workgroups evenly, as many per
// workgroup as their partials fit beside the activations, in whole rounds of
// one workgroup per CU.  Four row-group partials per item when they fit at
// one round, else two, else one.
template <int VARIANT, int UMAX, int MR>
hipError_t launch_quad(const uint8_t *codes, const uint16_t *scales, const uint16_t *X, float *Y, int M, int N,
                       int K, int rp, int grid, int bpw, size_t lds, hipStream_t stream) {
    if (rp == 4)
        hipLaunchKernelGGL((gemm_quad_kernel<VARIANT, UMAX, 4, MR>), dim3(grid), dim3(kQThreads), lds, stream, codes,
                           scales, X, Y, M, N, K, bpw);
    else if (rp == 2)
        hipLaunchKernelGGL((gemm_quad_kernel<VARIANT, UMAX, 2, MR>), dim3(grid), dim3(kQThreads), lds, stream, codes,
                           scales, X, Y, M, N, K, bpw);
    else
        hipLaunchKernelGGL((gemm_quad_kernel<VARIANT, UMAX, 1, MR>), dim3(grid), dim3(kQThreads), lds, stream, codes,
                           scales, X, Y, M, N, K, bpw);
    return hipGetLastError();
}

int32_t gemm_quad_enqueue(const uint8_t *codes, const uint16_t *scales, const uint16_t *X, float *Y,
                          int64_t M, int64_t N, int64_t K, int32_t variant, hipStream_t stream, bool *handled) {
    *handled = false;
    if (M < 1 || M > 2 * kQRows || (variant != TQ_TERNARY && variant != TQ_BINARY)) return TQ_OK;
    const int MR = M <= kQRows ? 1 : 2;
    const int64_t cpr = K / 64, capc = (cpr + 15) / 16 * 16, NI = capc / 16;
    if (N * cpr * (variant == TQ_TERNARY ? 16 : 8) >= (int64_t(1) << 31)) return TQ_OK;
    const int64_t stage = (int64_t)gemm_quad_stage_lds(K, MR);
    const int64_t nblocks = (N + 3) / 4;
    const int64_t cus = device_cu_count();
    int rp = 0;
    int64_t grid = 0, bpw = 0;
    for (int try_rp : {4, 2, 1}) {
        const int64_t per_block = NI * try_rp * 64 * MR;
        if (stage + per_block > kQMaxLds) continue;
        const int64_t max_b = (kQMaxLds - stage) / per_block;
        int64_t g = cus;
        while ((nblocks + g - 1) / g > max_b) g += cus;
        if (g > cus && try_rp > 1) continue;  // fewer partials per item keep one round
        rp = try_rp;
        grid = g;
        break;
    }
    if (!rp) return TQ_OK;
    // Two row sets only in one round of workgroups: on the 248320-row head
    // (two rounds, re-staging the activations) they measured 112 / 112 us at
    // M = 5 / 8 against 101 / 108 us for the per-group MFMA kernel
    if (MR == 2 && grid > cus) return TQ_OK;
    *handled = true;
    if (grid > nblocks) grid = nblocks;
    bpw = (nblocks + grid - 1) / grid;
    grid = (nblocks + bpw - 1) / bpw;
    const size_t lds = (size_t)(stage + bpw * NI * rp * 64 * MR);
    const int64_t upc = variant == TQ_TERNARY ? 4 : 2;
    const int64_t umax = (kQRows * MR * capc * upc + kQThreads - 1) / kQThreads;
    if (umax > (variant == TQ_TERNARY ? 5 : 3)) {  // unreachable while the stage fits LDS
        *handled = false;
        return TQ_OK;
    }
    hipError_t e = hipErrorInvalidValue;
    const int m = (int)M, n = (int)N, k = (int)K, g = (int)grid, bb = (int)bpw;
#define TQ_QL(V, U, R) e = launch_quad<V, U, R>(codes, scales, X, Y, m, n, k, rp, g, bb, lds, stream)
    // the staged activations fit LDS, so a thread stages at most 5 ternary
    // (16-weight) or 3 binary (32-weight) units
    if (variant == TQ_TERNARY) {
        if (MR == 1) {
            if (umax <= 2) TQ_QL(TQ_TERNARY, 2, 1);
            else TQ_QL(TQ_TERNARY, 5, 1);
        } else {
            if (umax <= 3) TQ_QL(TQ_TERNARY, 3, 2);
            else TQ_QL(TQ_TERNARY, 5, 2);
        }
    } else {
        if (MR == 1) {
            if (umax <= 1) TQ_QL(TQ_BINARY, 1, 1);
            else TQ_QL(TQ_BINARY, 3, 1);
        } else {
            if (umax <= 2) TQ_QL(TQ_BINARY, 2, 2);
            else TQ_QL(TQ_BINARY, 3, 2);
        }
    }
#undef TQ_QL
    if (e != hipSuccess) return fail(TQ_ERR_HIP, "GEMM launch failed: %s", hipGetErrorString(e));
    return TQ_OK;
}

}  // namespace tq
