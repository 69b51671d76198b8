/*
 * tq.h -- C ABI of the ternary / binary g128 packed-weight matmul for
 * AMD MI355X (gfx950).
 *
 * The operation (thakicloud.github.io, "Bonsai 27B: ternary and 1-bit
 * quantization", section "How the compression works"): every weight is a
 * code t in {-1, 0, +1} (ternary) or {-1, +1} (binary, the 1-bit build), and
 * each group of 128 weights shares one FP16 scale s_g, so w_i = s_g * t_i.
 * The kernels read the packed slots directly and apply the group scale
 * inside the matmul instead of expanding the weights to FP16 in memory
 * (aitrends.kr, "Ternary-Bonsai-27B-mlx-2bit", section "Technical
 * features": trits live in 2-bit slots; the scale is applied in the matmul).
 *
 * Storage format (the pages name the slots but not their layout; the layout
 * below is this library's documented reading):
 *   - W is N x K (out x in), y = W x.  A group is 128 consecutive weights of
 *     one row along K.  K must be a positive multiple of 128; group must be 128.
 *   - Ternary codes: uint8 [N][K/4].  Code c = t + 1 (0 -> -1, 1 -> 0,
 *     2 -> +1), 4 per byte, LSB-first: weight k of a row lives in byte k/4 at
 *     bits [2(k%4), 2(k%4)+2).  Code 3 is invalid.
 *   - Binary codes: uint8 [N][K/8].  Bit b = (t + 1)/2, weight k at bit k%8
 *     of byte k/8.
 *   - Scales: IEEE binary16 bit patterns, uint16 [N][K/128], row-major, any
 *     finite value (negative and subnormal allowed).
 *   - Activations: binary16 bit patterns, x[K] or X[M][K] row-major.
 *   - Output: float32 y[N] or Y[M][N] row-major; overwritten, never
 *     accumulated into.
 *
 * Conventions for every entry point:
 *   - Ownership: the caller owns every buffer; the library keeps no pointer
 *     after the call returns and allocates no device memory.
 *   - Streams: `stream` is a hipStream_t (NULL = the default stream).  GPU
 *     work is enqueued asynchronously on it; buffers must stay valid until
 *     the stream has passed the call.  Launch failures are reported at once
 *     (TQ_ERR_HIP); faults inside a kernel surface at the caller's next
 *     synchronisation.
 *   - Validation happens on the host, before any HIP call, in this order:
 *     NULL pointer, shape, group, variant, alignment.  No work is enqueued
 *     when a call returns an error.  tq_last_error() then describes it.
 *   - Device inputs are not inspected: codes passed to the GPU entry points
 *     must be valid (a ternary code 3 gives an unspecified result, never a
 *     fault).  tq_pack never produces code 3.
 *   - Outputs must not alias inputs.  Functions are reentrant; the only
 *     library state is the calling thread's last-error record.
 *   - Byte offsets are 64-bit (N*K reaches 1.27e9 for a 248320 x 5120 head).
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* weight variants */
#define TQ_TERNARY 0 /* t in {-1,0,+1}, 2-bit slots, 2.125 bits/weight stored */
#define TQ_BINARY 1  /* t in {-1,+1},   1-bit slots, 1.125 bits/weight stored */
/* t in {-1,0,+1} stored five trits to a byte: the native ternary packing
 * the model card names as the step after 2-bit slots (aitrends.kr,
 * "Ternary-Bonsai-27B-mlx-2bit", "Technical features"; 3^5 = 243 <= 256).
 * Byte b (0..25) of a 128-weight group holds trits 5b..5b+4 of the group as
 * sum_i (t_{5b+i} + 1) * 3^i, least significant digit first; byte 25 holds
 * trits 125..127 and its digits 3 and 4 are 0.  A row is its K/128 groups
 * of 26 bytes followed by zero bytes up to a multiple of 16, so rows stay
 * 16-byte aligned: 1.75 bits/weight stored (with the scale) when K is a
 * multiple of 1024.  Supported by tq_codes_bytes, tq_pack, tq_unpack,
 * tq_gemv and tq_gemm with M == 1 (K <= 40960); other entry points return
 * TQ_ERR_VARIANT. */
#define TQ_TERNARY5 2
/* Affine 2-bit levels as the MLX packaging stores them, a scale and a bias
 * per group (aitrends.kr, "Ternary-Bonsai-27B-mlx-2bit", "Technical
 * features"): q in {0,1,2,3} in the 2-bit slots of TQ_TERNARY (same bytes,
 * code 3 allowed), w = s_g * q + b_g with FP16 s_g and b_g per 128-weight
 * group, 2.25 bits/weight stored.  Ternary weights are q = t + 1 with
 * b_g = -s_g.  tq_pack / tq_unpack take and return q.  The product is
 * tq_gemv_affine; the other device entry points return TQ_ERR_VARIANT. */
#define TQ_AFFINE2 3

/* status codes */
#define TQ_OK 0
#define TQ_ERR_NULL 1    /* a required pointer is NULL                          */
#define TQ_ERR_SHAPE 2   /* M or N < 1, K < 128, K % 128 != 0, or too large     */
#define TQ_ERR_GROUP 3   /* group != 128                                         */
#define TQ_ERR_VARIANT 4 /* unknown variant, or one the entry point does not take */
#define TQ_ERR_VALUE 5   /* tq_pack: a t outside the variant's set              */
#define TQ_ERR_CODE 6    /* tq_unpack: a ternary code 3 or a bad five-trit byte  */
#define TQ_ERR_ALIGN 7   /* a device pointer is not aligned as required          */
#define TQ_ERR_HIP 8     /* the HIP runtime rejected a launch                    */

/* Size of the packed code array: N*K/4 bytes (ternary), N*K/8 (binary) or
 * N * roundup(26*K/128, 16) (five-trit bytes).  Returns 0 for an invalid
 * shape or variant.  Passage: each trit sits in a 2-bit slot (aitrends.kr,
 * "Ternary-Bonsai-27B-mlx-2bit", "Technical features"); the 1-bit build keeps
 * one bit per weight (thakicloud.github.io, "Bonsai 27B: ternary and 1-bit
 * quantization", "How the compression works", whose bits-per-weight figures
 * 1.71 and 1.125 include the 16-bit scale of every 128 weights). */
size_t tq_codes_bytes(int64_t N, int64_t K, int32_t variant);

/* Number of FP16 scales: N*K/group, one per 128 weights of a row along K
 * (thakicloud.github.io, "Bonsai 27B: ternary and 1-bit quantization", "How
 * the compression works": one FP16 scale shared by each group of 128
 * weights).  Returns 0 for an invalid shape/group. */
size_t tq_scales_count(int64_t N, int64_t K, int32_t group);

/* Host -> host.  Pack t (int8 [N][K], row-major) into `codes`
 * (tq_codes_bytes(N,K,variant) bytes, fully overwritten).  Scales are not
 * touched: they pass through unchanged.  The value sets are the pages'
 * ternary {-1, 0, +1} and binary {-1, +1} (thakicloud.github.io, "Bonsai 27B:
 * ternary and 1-bit quantization", "How the compression works"), stored as
 * 2-bit slots (aitrends.kr, "Ternary-Bonsai-27B-mlx-2bit", "Technical
 * features"); the code map and bit order are this header's stated layout.
 * Arguments: t host, N*K bytes; codes host, caller-owned.  A value outside
 * the variant's set returns TQ_ERR_VALUE; tq_last_error_index() gives its
 * flat index n*K+k and `codes` is left in an unspecified state.  NULL
 * pointers return TQ_ERR_NULL, bad shapes TQ_ERR_SHAPE / TQ_ERR_GROUP. */
int32_t tq_pack(const int8_t *t, int64_t N, int64_t K, int32_t group,
                int32_t variant, uint8_t *codes);

/* Host -> host.  Inverse of tq_pack: writes t (int8 [N][K], caller-owned)
 * from the slots of the layout above (passages as tq_pack).  A ternary
 * code 3 returns TQ_ERR_CODE; tq_last_error_index() gives the flat weight
 * index of the first such slot.  TQ_TERNARY5: a byte >= 243, or a last byte
 * of a group >= 27, returns TQ_ERR_CODE with the flat index of the byte's
 * first trit; padding bytes are not read. */
int32_t tq_unpack(const uint8_t *codes, int64_t N, int64_t K, int32_t group,
                  int32_t variant, int8_t *t);

/* Device.  y[n] = sum_g s[n][g] * sum_{j<128} t[n][128g+j] * x[128g+j],
 * accumulated in fp32 (batch-1 decode GEMV).  Passage: w_i = s_g * t_i with
 * one FP16 scale per 128 weights (thakicloud.github.io, "Bonsai 27B: ternary
 * and 1-bit quantization", "How the compression works"), the packed slots
 * read directly and the scale applied inside the matmul (aitrends.kr,
 * "Ternary-Bonsai-27B-mlx-2bit", "Technical features"); decoding one token
 * is bound by memory bandwidth (thakicloud.github.io, same page,
 * "Throughput and speculative decoding").
 *   codes  : device, tq_codes_bytes(N,K,variant) bytes, 16-byte aligned
 *   scales : device, uint16 [N][K/128] (fp16 bits), 2-byte aligned
 *   x      : device, uint16 [K] (fp16 bits), 16-byte aligned
 *   y      : device, float [N], 4-byte aligned; overwritten
 * Limits: 1 <= N < 2^31, 128 <= K <= 65536 (a workgroup keeps the whole
 * permuted activation vector in LDS); a larger K returns TQ_ERR_SHAPE. */
int32_t tq_gemv(const uint8_t *codes, const uint16_t *scales, const uint16_t *x,
                float *y, int64_t N, int64_t K, int32_t group, int32_t variant,
                void *stream);

/* Device.  Y[m][n] = sum_g s[n][g] * sum_j t[n][128g+j] * X[m][128g+j]
 * for m < M (small-batch GEMM: speculative-verify and prefill-chunk widths:
 * thakicloud.github.io, "Bonsai 27B: ternary and 1-bit quantization",
 * "Throughput and speculative decoding", which verifies k = 4 drafted
 * tokens at once and measures 512-token prefill; the product is the one of
 * tq_gemv for every row of X).
 * X is uint16 [M][K] (16-byte aligned), Y is float [M][N]; other arguments as
 * tq_gemv.  M == 1 is the GEMV.  Limits: 1 <= M <= 65536, N and K as tq_gemv. */
int32_t tq_gemm(const uint8_t *codes, const uint16_t *scales, const uint16_t *X,
                float *Y, int64_t M, int64_t N, int64_t K, int32_t group,
                int32_t variant, void *stream);

/* Host.  Bytes of device workspace tq_gemm_ws can use for this shape: the
 * partial products of a K split (the product of tq_gemm, same passages), for
 * 5 <= M <= 64 ternary weights with an even group count and N <= 131072
 * rows; 0 when the shape takes no workspace (or a K split into one slice) or
 * the arguments are invalid (no error is recorded). */
size_t tq_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t group,
                               int32_t variant);

/* Device.  tq_gemm (same product and passages: thakicloud.github.io, "Bonsai
 * 27B: ternary and 1-bit quantization", "How the compression works" and
 * "Throughput and speculative decoding") with a caller-owned workspace:
 * workspace is device memory, 16-byte aligned, of workspace_bytes bytes
 * (NULL / 0 allowed).  With at least tq_gemm_workspace_bytes(...) bytes,
 * 5..64-row ternary batches take a K-split kernel whose slices are added in a
 * fixed order; with less, the call behaves as tq_gemm.  The workspace is
 * overwritten and in use until the work enqueued on `stream` completes:
 * calls that share one workspace must be ordered (the same stream).
 * Errors as tq_gemm; a misaligned workspace returns TQ_ERR_ALIGN. */
int32_t tq_gemm_ws(const uint8_t *codes, const uint16_t *scales, const uint16_t *X,
                   float *Y, int64_t M, int64_t N, int64_t K, int32_t group,
                   int32_t variant, void *workspace, size_t workspace_bytes,
                   void *stream);

/* Device.  Embedding rows: out[i][k] = s[ids[i]][k/128] * t[ids[i]][k] as
 * IEEE FP16 for i < n_ids, k < K.  Every weight matrix of the model is ternary,
 * the token embedding included (aitrends.kr, "Ternary-Bonsai-27B-mlx-2bit",
 * section on what sets the build apart), and w = s_g * t (thakicloud.github.io,
 * "Bonsai 27B: ternary and 1-bit quantization", "How the compression works");
 * with t in {-1, 0, +1} each output is exact (a signed zero keeps the sign
 * of s * 0).  codes / scales: the packed table, as tq_gemv (N rows, K per
 * row); codes need 4-byte alignment only.  ids: int32 [n_ids] device,
 * 4-byte aligned.  out: uint16 (FP16 bits) [n_ids][K] device, 16-byte
 * aligned, caller-owned.  An id outside [0, N) yields a row of +0 (nothing is
 * read for it).  n_ids == 0 returns TQ_OK without touching any pointer;
 * n_ids < 0 or >= 2^31 returns TQ_ERR_SHAPE.  Other errors as tq_gemv. */
int32_t tq_embed(const uint8_t *codes, const uint16_t *scales, const int32_t *ids,
                 uint16_t *out, int64_t n_ids, int64_t N, int64_t K, int32_t group,
                 int32_t variant, void *stream);

/* Device.  y[n] = sum_g (s[n][g] * sum_j q[n][128g+j] * x[128g+j]
 *                      + b[n][g] * sum_j x[128g+j])
 * i.e. y = W x with w = s_g * q + b_g (the affine 2-bit levels of
 * TQ_AFFINE2), accumulated in fp32.  codes as tq_gemv with K/4 bytes per row;
 * scales and biases are uint16 (fp16 bits) [N][K/128], 2-byte aligned; x and
 * y as tq_gemv.  Limits: 1 <= N < 2^31, 128 <= K <= 20480 (the activations
 * of a lane's columns stay in registers); a larger K returns TQ_ERR_SHAPE.
 * group must be 128. */
int32_t tq_gemv_affine(const uint8_t *codes, const uint16_t *scales, const uint16_t *biases,
                       const uint16_t *x, float *y, int64_t N, int64_t K, int32_t group,
                       void *stream);

/* ---- 4-bit KV cache and decode attention (one layer, one sequence) ----
 * The full-attention layers keep K and V in a 4-bit cache (thakicloud.github.io,
 * "Bonsai 27B: ternary and 1-bit quantization", memory section: 64 KiB per
 * token at FP16 for 16 layers x 2 x 4 KV heads x 256; aitrends.kr,
 * "Ternary-Bonsai-27B-mlx-2bit", "Technical features").  Format (the pages
 * give none): each head vector of 256 is cut into 8 groups of 32 dimensions,
 * each with an FP16 scale d = fp16(amax / 7) (amax / 7 in fp32, rounded to
 * nearest even) and per element the nibble q + 8, q = clamp(rint(x / d),
 * -8, 7) (x / d in fp32, ties to even); the value is (nibble - 8) * d.
 * Head dimension 256 only.  The four cache arrays (device, 16-byte aligned,
 * caller-owned) hold n_kv heads x t_cap tokens (t_cap a multiple of 32):
 *   K codes  [n_kv][t_cap][32 dwords]: dword 8c + g holds dims 32g + 8c + e,
 *            e = 2p + h at bits 16h + 4p (p = 0..3, h = 0..1);
 *   K scales [n_kv][t_cap][8] FP16;
 *   V codes  [n_kv][t_cap/32][1024 dwords]: for a block of 32 tokens, dword
 *            (16c + n) * 16 + j holds dim 16j + n of tokens tau(c, s), s = 2p + h
 *            at bits 16h + 4p, tau(c, s) = 4c + s (s < 4), 16 + 4c + s - 4 (s >= 4);
 *   V scales [n_kv][t_cap/32][256] FP16: index (8c + g) * 8 + s is group g of
 *            token tau(c, s).
 * Tokens at or past T are never read into a result, but the attention reads
 * whole 32-token blocks: give the arrays finite contents (allocate them
 * zero-filled). */
#define TQ_KV_K_CODES 0
#define TQ_KV_K_SCALES 1
#define TQ_KV_V_CODES 2
#define TQ_KV_V_SCALES 3

/* Bytes of one cache array (part TQ_KV_*); 0 for an invalid request
 * (n_kv outside [1, 64], t_cap not a positive multiple of 32 below 2^31). */
size_t tq_kv_bytes(int64_t n_kv, int64_t t_cap, int32_t part);

/* Device.  Quantizes n_tok new tokens k, v (uint16 fp16 bits
 * [n_tok][n_kv][256], 2-byte aligned) into cache positions [pos, pos+n_tok).
 * Positions outside [0, t_cap) return TQ_ERR_SHAPE; n_tok == 0 does nothing.
 * Other tokens of the cache are left as they are (value codes of a 32-token
 * block share dwords; the writes are atomic per dword). */
int32_t tq_kv_append(const uint16_t *k, const uint16_t *v, int64_t n_tok, int64_t pos,
                     int64_t n_kv, int64_t t_cap, uint8_t *kc, uint16_t *ks, uint8_t *vc,
                     uint16_t *vs, void *stream);

/* Bytes of device workspace tq_attn_decode needs for T tokens (0 when the
 * shape is invalid). */
size_t tq_attn_workspace_bytes(int64_t T, int64_t n_q, int64_t n_kv);

/* Device.  Decode attention of one query token over cache positions
 * [0, T): for query head h (KV head h / (n_q / n_kv)),
 *   out[h] = sum_t softmax_t(q_h . k_t / sqrt(256)) v_t
 * with k_t, v_t the dequantized cache vectors, in fp32.  q: uint16 fp16
 * [n_q][256], 16-byte aligned; out: float [n_q][256]; workspace: device,
 * 16-byte aligned, at least tq_attn_workspace_bytes(T, n_q, n_kv) bytes,
 * overwritten.  n_q must be a multiple of n_kv, at most 16 times it;
 * 1 <= T <= t_cap. */
int32_t tq_attn_decode(const uint16_t *q, const uint8_t *kc, const uint16_t *ks,
                       const uint8_t *vc, const uint16_t *vs, int64_t T, int64_t n_q,
                       int64_t n_kv, int64_t t_cap, float *out, void *workspace,
                       size_t workspace_bytes, void *stream);

/* Device.  For callers that cannot allocate (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): tq_attn_decode
 * with the same arguments minus the workspace, running the same kernels on a
 * scratch array the library holds in device memory (8 MiB per GPU, kept until
 * the process ends; the model's 24 query heads over 4 KV heads need about
 * 3 MiB at any T).  A call whose workspace would exceed it (see
 * tq_attn_workspace_bytes) returns TQ_ERR_SHAPE before any HIP call.  The
 * first call on a device looks the array up (one hipGetSymbolAddress; a
 * failure returns TQ_ERR_HIP); no call allocates.  Every call on a GPU shares
 * that GPU's array: calls that overlap on one GPU (streams with no ordering
 * between them) race and must be serialised by the caller.  Results are
 * identical to tq_attn_decode's. */
int32_t tq_attn_decode_noalloc(const uint16_t *q, const uint8_t *kc, const uint16_t *ks,
                               const uint8_t *vc, const uint16_t *vs, int64_t T, int64_t n_q,
                               int64_t n_kv, int64_t t_cap, float *out, void *stream);

/* Measurement aid, not part of the matmul: a plain streaming read of `bytes`
 * (a positive multiple of 16) of the device buffer `buf` (16-byte aligned),
 * each 16-byte unit loaded once, on `blocks_per_cu` (1..8) workgroups of 512
 * threads per compute unit.  It gives the ceiling that a bandwidth-bound
 * launch reading as many bytes is measured against.  `sink`: 4 bytes of
 * device memory the kernel may write (in practice never).  Errors:
 * TQ_ERR_NULL, TQ_ERR_SHAPE, TQ_ERR_ALIGN, TQ_ERR_HIP. */
int32_t tq_stream_read(const void *buf, size_t bytes, uint32_t *sink, int32_t blocks_per_cu,
                       void *stream);

/* Text of the calling thread's last error ("" if none). */
const char *tq_last_error(void);

/* Flat index attached to the last TQ_ERR_VALUE / TQ_ERR_CODE, else -1. */
int64_t tq_last_error_index(void);

/* Library version string. */
const char *tq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */
