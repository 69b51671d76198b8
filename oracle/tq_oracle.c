/*
 * tq_oracle.c -- plain, slow, fp64 CPU oracle for the ternary / binary g128
 * packed-weight matrix multiply.
 *
 * TEST INFRASTRUCTURE ONLY.  The tests, the smoke check and the bench's CPU
 * baseline call it; the product library never links, loads or runs it, and
 * this file includes nothing from the product.  Build: gcc -O2 -fopenmp,
 * no fast-math.
 *
 * What the method computes
 * ------------------------
 * Each weight is a trit t in {-1, 0, +1} (or a sign t in {-1, +1} for the
 * 1-bit build) and every group of 128 weights shares one FP16 scale s_g, so
 * the weight that takes part in the product is w_i = s_g * t_i.
 *   - thakicloud.github.io, "Bonsai 27B: ternary and 1-bit quantization",
 *     section "How the compression works" (w_i = s_g * t_i; one FP16 scale per
 *     128-weight group; ternary {-1,0,+1}, binary {-1,+1}).
 *   - aitrends.kr, "Ternary-Bonsai-27B-mlx-2bit", section "Technical
 *     features" (the group scale is applied inside the matmul; current
 *     kernels keep each trit in a 2-bit slot).
 *
 * Readings taken where the pages are silent (each stated once here):
 *   R1  a group is 128 consecutive weights along K (the reduction axis) of
 *       one output row;
 *   R2  2-bit code c = t + 1 (0 -> -1, 1 -> 0, 2 -> +1); code 3 is invalid;
 *   R3  slots are LSB-first: weight k of a row sits in byte k/4 at bits
 *       [2(k mod 4), 2(k mod 4) + 2); rows are contiguous, row-major;
 *   R4  binary: bit b = (t + 1) / 2, 8 weights per byte, LSB-first;
 *   R5  scales are a separate FP16 array [N][K/128], row-major;
 *   R6  activations FP16 row-major X[M][K], output Y[M][N] (y = W x);
 *   R7  five-trit bytes (the native ternary packing the model card names as
 *       the next step, aitrends.kr, "Ternary-Bonsai-27B-mlx-2bit", section
 *       "Technical features"; 3^5 = 243 <= 256): a group's 128 trits fill
 *       26 bytes, byte b holding trits 5b .. 5b+4 of the group as the base-3
 *       number sum_i (t_{5b+i} + 1) * 3^i (least significant digit first,
 *       like the 2-bit slots); byte 25 holds trits 125..127 and its digits
 *       3 and 4 are 0.  A row's G groups are consecutive and the row is
 *       padded with zero bytes to a multiple of 16 bytes;
 *   R8  affine 2-bit storage (the MLX packaging keeps a scale and a bias per
 *       group, aitrends.kr, "Ternary-Bonsai-27B-mlx-2bit", "Technical
 *       features"): an unsigned level q in {0,1,2,3} per weight in the 2-bit
 *       slots of R3, and per group an FP16 scale s_g and FP16 bias b_g with
 *       w = s_g * q + b_g.  Ternary weights are the case q = t + 1,
 *       b_g = -s_g.  pack / unpack take and return q itself.
 *
 * The product is the plain definition, evaluated in fp64:
 *   Y[m][n] = sum_g s[n][g] * ( sum_{j<128} t[n][128g+j] * X[m][128g+j] )
 * Every t*x is exact in fp64 and a 128-term sum of FP16 values is exact in
 * fp64, so only the scale product and the group additions round.  The
 * oracle also returns A[m][n] = sum_g |s[n][g]| * sum_j |t * x|, the
 * magnitude bound used by the acceptance tolerance.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_OK = 0, OR_ERR_NULL = 1, OR_ERR_SHAPE = 2, OR_ERR_GROUP = 3,
       OR_ERR_VARIANT = 4, OR_ERR_VALUE = 5, OR_ERR_CODE = 6, OR_ERR_NOMEM = 7 };
enum { OR_TERNARY = 0, OR_BINARY = 1, OR_TERNARY5 = 2, OR_AFFINE2 = 3 };

/* R7: bytes of one row of five-trit codes (26 per group, padded to 16). */
static int64_t ternary5_row_bytes(int64_t K)
{
    int64_t raw = 26 * (K / 128);
    return (raw + 15) / 16 * 16;
}

/* IEEE-754 binary16 bit pattern -> real value, from the format's definition:
 * sign bit, 5-bit exponent (bias 15), 10-bit fraction; exponent 0 is the
 * subnormal range f * 2^-24, exponent 31 is Inf / NaN. */
double oracle_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int f = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return sign ? -v : v;
}

/* Bytes of packed codes for an N x K weight: 4 slots per byte (ternary) or
 * 8 per byte (binary). */
int64_t oracle_codes_bytes(int64_t N, int64_t K, int variant)
{
    if (variant == OR_TERNARY || variant == OR_AFFINE2) return N * K / 4;
    if (variant == OR_BINARY) return N * K / 8;
    if (variant == OR_TERNARY5) return N * ternary5_row_bytes(K);
    return -1;
}

/* Number of FP16 scales: one per 128-weight group of every row. */
int64_t oracle_scales_count(int64_t N, int64_t K, int32_t group)
{
    return N * (K / group);
}

static int check_args(int64_t N, int64_t K, int32_t group, int variant)
{
    if (group != 128) return OR_ERR_GROUP;
    if (N < 1 || K < 128 || K % 128 != 0) return OR_ERR_SHAPE;
    if (variant != OR_TERNARY && variant != OR_BINARY && variant != OR_TERNARY5 &&
        variant != OR_AFFINE2)
        return OR_ERR_VARIANT;
    return OR_OK;
}

/* Pack trits t[N][K] (int8) into slots.  On a value outside the variant's
 * set, returns OR_ERR_VALUE and writes the flat index of the first bad
 * element to *bad. */
int oracle_pack(const int8_t *t, int64_t N, int64_t K, int32_t group,
                int variant, uint8_t *codes, int64_t *bad)
{
    if (!t || !codes) return OR_ERR_NULL;
    int rc = check_args(N, K, group, variant);
    if (rc) return rc;
    int64_t nbytes = oracle_codes_bytes(N, K, variant);
    for (int64_t i = 0; i < N * K; i++) {
        int v = t[i];
        int ok = (variant == OR_BINARY)    ? (v == -1 || v == 1)
                 : (variant == OR_AFFINE2) ? (v >= 0 && v <= 3)
                                           : (v >= -1 && v <= 1);
        if (!ok) {
            if (bad) *bad = i;
            return OR_ERR_VALUE;
        }
    }
    memset(codes, 0, (size_t)nbytes);
    if (variant == OR_TERNARY5) {
        int64_t rb = ternary5_row_bytes(K);
        for (int64_t n = 0; n < N; n++)
            for (int64_t g = 0; g < K / 128; g++)
                for (int b = 0; b < 26; b++) {                  /* R7 */
                    int value = 0, power = 1;
                    for (int i = 0; i < 5 && 5 * b + i < 128; i++) {
                        value += (t[n * K + 128 * g + 5 * b + i] + 1) * power;
                        power *= 3;
                    }
                    codes[n * rb + 26 * g + b] = (uint8_t)value;
                }
        return OR_OK;
    }
    for (int64_t n = 0; n < N; n++) {
        for (int64_t k = 0; k < K; k++) {
            int v = t[n * K + k];
            if (variant == OR_AFFINE2) {
                int64_t byte = n * (K / 4) + k / 4;             /* R8, R3 */
                codes[byte] |= (uint8_t)(v << (2 * (k % 4)));
            } else if (variant == OR_TERNARY) {
                int c = v + 1;                                  /* R2 */
                int64_t byte = n * (K / 4) + k / 4;             /* R3 */
                codes[byte] |= (uint8_t)(c << (2 * (k % 4)));
            } else {
                int b = (v + 1) / 2;                            /* R4 */
                int64_t byte = n * (K / 8) + k / 8;
                codes[byte] |= (uint8_t)(b << (k % 8));
            }
        }
    }
    return OR_OK;
}

/* Unpack slots back to trits.  A ternary code 3 returns OR_ERR_CODE with the
 * flat weight index of the first bad slot in *bad. */
int oracle_unpack(const uint8_t *codes, int64_t N, int64_t K, int32_t group,
                  int variant, int8_t *t, int64_t *bad)
{
    if (!codes || !t) return OR_ERR_NULL;
    int rc = check_args(N, K, group, variant);
    if (rc) return rc;
    if (variant == OR_TERNARY5) {
        /* R7: a byte is valid when it is below 3^5 and, in byte 25 of a group,
         * its digits 3 and 4 are 0; otherwise OR_ERR_CODE with the flat index
         * of the byte's first trit.  Padding bytes are not read. */
        int64_t rb = ternary5_row_bytes(K);
        for (int64_t n = 0; n < N; n++)
            for (int64_t g = 0; g < K / 128; g++)
                for (int b = 0; b < 26; b++) {
                    int value = codes[n * rb + 26 * g + b];
                    for (int i = 0; i < 5; i++) {
                        int c = value % 3;
                        value /= 3;
                        if (5 * b + i < 128)
                            t[n * K + 128 * g + 5 * b + i] = (int8_t)(c - 1);
                        else if (c != 0)
                            value = -1;
                        if (value < 0) break;
                    }
                    if (value != 0) {
                        if (bad) *bad = n * K + 128 * g + 5 * b;
                        return OR_ERR_CODE;
                    }
                }
        return OR_OK;
    }
    for (int64_t n = 0; n < N; n++) {
        for (int64_t k = 0; k < K; k++) {
            if (variant == OR_AFFINE2) {
                uint8_t byte = codes[n * (K / 4) + k / 4];
                t[n * K + k] = (int8_t)((byte >> (2 * (k % 4))) & 3);
            } else if (variant == OR_TERNARY) {
                uint8_t byte = codes[n * (K / 4) + k / 4];
                int c = (byte >> (2 * (k % 4))) & 3;
                if (c == 3) {
                    if (bad) *bad = n * K + k;
                    return OR_ERR_CODE;
                }
                t[n * K + k] = (int8_t)(c - 1);
            } else {
                uint8_t byte = codes[n * (K / 8) + k / 8];
                int b = (byte >> (k % 8)) & 1;
                t[n * K + k] = (int8_t)(2 * b - 1);
            }
        }
    }
    return OR_OK;
}

/* Y[M][N] (and the bound A[M][N], if A is not NULL) from packed codes,
 * FP16 scales [N][K/128] and FP16 activations X[M][K], all as bit patterns.
 * Rows of W are independent, so `threads` > 1 splits the row loop across
 * OpenMP threads; the arithmetic of each output is the same either way. */
int oracle_gemm(const uint8_t *codes, const uint16_t *scales, const uint16_t *X,
                int64_t M, int64_t N, int64_t K, int32_t group, int variant,
                double *Y, double *A, int threads)
{
    if (!codes || !scales || !X || !Y) return OR_ERR_NULL;
    int rc = check_args(N, K, group, variant);
    if (rc) return rc;
    if (variant == OR_AFFINE2) return OR_ERR_VARIANT;   /* needs biases: oracle_affine_gemm */
    if (M < 1) return OR_ERR_SHAPE;
    int64_t G = K / group;
    int64_t row_bytes = oracle_codes_bytes(1, K, variant);

    /* activations decoded once */
    double *x = (double *)malloc((size_t)(M * K) * sizeof(double));
    if (!x) return OR_ERR_NOMEM;
    for (int64_t i = 0; i < M * K; i++) x[i] = oracle_half_to_double(X[i]);

    int status = OR_OK;
    if (threads < 1) threads = 1;
#pragma omp parallel num_threads(threads)
    {
        int8_t *t = (int8_t *)malloc((size_t)K);
        if (!t) {
#pragma omp atomic write
            status = OR_ERR_NOMEM;
        }
#pragma omp for schedule(static)
        for (int64_t n = 0; n < N; n++) {
            if (!t) continue;
            int64_t badi = 0;
            int urc = oracle_unpack(codes + n * row_bytes, 1, K, group, variant, t, &badi);
            if (urc) {
#pragma omp atomic write
                status = urc;
                continue;
            }
            for (int64_t m = 0; m < M; m++) {
                double acc = 0.0, bound = 0.0;
                for (int64_t g = 0; g < G; g++) {
                    double s = oracle_half_to_double(scales[n * G + g]);
                    double part = 0.0, apart = 0.0;
                    for (int64_t j = 0; j < group; j++) {
                        double tx = (double)t[g * group + j] * x[m * K + g * group + j];
                        part += tx;
                        apart += fabs(tx);
                    }
                    acc += s * part;
                    bound += fabs(s) * apart;
                }
                Y[m * N + n] = acc;
                if (A) A[m * N + n] = bound;
            }
        }
        free(t);
    }
    free(x);
    return status;
}

/* Embedding rows: out[i][k] = s[id_i][k / group] * t[id_i][k] in fp64, for
 * i < n, from the oracle's own unpack.  Every weight matrix of the model is
 * ternary, the token embedding included (aitrends.kr,
 * "Ternary-Bonsai-27B-mlx-2bit", section on what sets the build apart;
 * thakicloud.github.io, "Bonsai 27B: ternary and 1-bit quantization", "What
 * the technology is"), so a token's input vector is its row w = s_g * t.
 * Ids must lie in [0, N); anything else returns OR_ERR_SHAPE. */
int oracle_embed(const uint8_t *codes, const uint16_t *scales, const int32_t *ids, int64_t n,
                 int64_t N, int64_t K, int32_t group, int variant, double *out)
{
    if (!codes || !scales || !ids || !out) return OR_ERR_NULL;
    int rc = check_args(N, K, group, variant);
    if (rc) return rc;
    if (variant == OR_AFFINE2) return OR_ERR_VARIANT;
    if (n < 0) return OR_ERR_SHAPE;
    int64_t G = K / group;
    int64_t row_bytes = oracle_codes_bytes(1, K, variant);
    int8_t *t = (int8_t *)malloc((size_t)K);
    if (!t) return OR_ERR_NOMEM;
    for (int64_t i = 0; i < n; i++) {
        int64_t id = ids[i];
        if (id < 0 || id >= N) {
            free(t);
            return OR_ERR_SHAPE;
        }
        int64_t badi = 0;
        rc = oracle_unpack(codes + id * row_bytes, 1, K, group, variant, t, &badi);
        if (rc) {
            free(t);
            return rc;
        }
        for (int64_t k = 0; k < K; k++)
            out[i * K + k] = oracle_half_to_double(scales[id * G + k / group]) * (double)t[k];
    }
    free(t);
    return OR_OK;
}

/* Affine 2-bit product (R8): Y[m][n] = sum_k (s[n][g] * q[n][k] + b[n][g]) *
 * X[m][k], g = k / group, with the weight formed per element in fp64 as the
 * definition states.  A[m][n] = sum_g (|s| * sum_j |q * x| + |b| * sum_j |x|)
 * bounds the magnitude of the terms a kernel that applies the scale and the
 * bias per group (s * sum q x + b * sum x) adds up. */
int oracle_affine_gemm(const uint8_t *codes, const uint16_t *scales, const uint16_t *biases,
                       const uint16_t *X, int64_t M, int64_t N, int64_t K, int32_t group,
                       double *Y, double *A, int threads)
{
    if (!codes || !scales || !biases || !X || !Y) return OR_ERR_NULL;
    int rc = check_args(N, K, group, OR_AFFINE2);
    if (rc) return rc;
    if (M < 1) return OR_ERR_SHAPE;
    int64_t G = K / group;
    double *x = (double *)malloc((size_t)(M * K) * sizeof(double));
    if (!x) return OR_ERR_NOMEM;
    for (int64_t i = 0; i < M * K; i++) x[i] = oracle_half_to_double(X[i]);
    int status = OR_OK;
    if (threads < 1) threads = 1;
#pragma omp parallel num_threads(threads)
    {
        int8_t *q = (int8_t *)malloc((size_t)K);
        if (!q) {
#pragma omp atomic write
            status = OR_ERR_NOMEM;
        }
#pragma omp for schedule(static)
        for (int64_t n = 0; n < N; n++) {
            if (!q) continue;
            int64_t badi = 0;
            oracle_unpack(codes + n * (K / 4), 1, K, group, OR_AFFINE2, q, &badi);
            for (int64_t m = 0; m < M; m++) {
                double acc = 0.0, bound = 0.0;
                for (int64_t k = 0; k < K; k++) {
                    double sg = oracle_half_to_double(scales[n * G + k / group]);
                    double bg = oracle_half_to_double(biases[n * G + k / group]);
                    double w = sg * (double)q[k] + bg;
                    acc += w * x[m * K + k];
                    bound += fabs(sg) * fabs((double)q[k] * x[m * K + k]) + fabs(bg) * fabs(x[m * K + k]);
                }
                Y[m * N + n] = acc;
                if (A) A[m * N + n] = bound;
            }
        }
        free(q);
    }
    free(x);
    return status;
}

/* ------------------------------------------------------------------------
 * 4-bit KV cache and decode attention.
 *
 * The model keeps K and V of its 16 full-attention layers (4 KV heads of
 * dimension 256) in a 4-bit cache that the pages call near-lossless
 * (aitrends.kr, "Ternary-Bonsai-27B-mlx-2bit", "Technical features";
 * thakicloud.github.io, "Bonsai 27B: ternary and 1-bit quantization", the
 * memory section: 64 KiB per token at FP16, a quarter of that at 4 bits;
 * techtoast.kr, the KV-cache arithmetic: 2 x 4 heads x 256 x 16 layers).
 * The pages give no 4-bit format.  Reading R9: each head vector of 256 is
 * cut into 8 groups of 32 consecutive dimensions; a group keeps one FP16
 * scale d = fp16(amax / 7) (amax = max |x| over the group, the division in
 * fp32, the conversion round-to-nearest-even) and per element the nibble
 * q + 8 with q = clamp(rint(x / d), -8, 7) (x / d in fp32, rint half-to-even);
 * an all-zero group stores d = 0 and nibbles 8.  The dequantized value is
 * (nibble - 8) * d.  Decode attention for query head h reads KV head
 * h / (n_q / n_kv): out_h = sum_t softmax_t(q_h . k_t / sqrt(256)) v_t.
 * Logical layouts here: nibbles [n_vec][256] (one byte each), scales
 * [n_vec][8].
 * ------------------------------------------------------------------------ */

/* IEEE binary32 -> binary16 bits, round to nearest even, from the formats'
 * definitions (finite inputs below 65520 in magnitude). */
uint16_t oracle_float_to_half(float f)
{
    union { float f; uint32_t u; } v = { f };
    uint32_t sign = (v.u >> 16) & 0x8000u;
    uint32_t mag = v.u & 0x7FFFFFFFu;
    if (mag == 0) return (uint16_t)sign;
    int e = (int)(mag >> 23) - 127;                /* unbiased exponent */
    uint32_t m = (mag & 0x7FFFFFu) | 0x800000u;    /* 24-bit significand */
    /* value = m * 2^(e - 23); binary16 keeps 11 bits for e >= -14, and a
     * fixed quantum of 2^-24 below */
    int shift = (e >= -14) ? 13 : 13 + (-14 - e);
    uint32_t q;
    if (shift >= 32) {
        q = 0;                                     /* below 2^-32: far under half of 2^-24 */
    } else {
        q = m >> shift;
        uint32_t rem = m & ((1u << shift) - 1u), half = 1u << (shift - 1);
        if (rem > half || (rem == half && (q & 1u))) q++;
    }
    uint32_t h;
    if (e >= -14) {
        /* q in [2^10, 2^11]; carry may bump the exponent */
        int he = e + 15;
        if (q >= 2048u) { q >>= 1; he++; }
        h = ((uint32_t)he << 10) | (q & 0x3FFu);
    } else {
        h = q;                                     /* subnormal (or 2^-14 on carry) */
    }
    return (uint16_t)(sign | h);
}

int oracle_kv_quant(const uint16_t *x, int64_t n_vec, uint8_t *nib, uint16_t *scales)
{
    if (!x || !nib || !scales) return OR_ERR_NULL;
    if (n_vec < 0) return OR_ERR_SHAPE;
    for (int64_t v = 0; v < n_vec; v++)
        for (int g = 0; g < 8; g++) {
            const uint16_t *xg = x + v * 256 + 32 * g;
            float amax = 0.0f;
            for (int j = 0; j < 32; j++) {
                float a = fabsf((float)oracle_half_to_double(xg[j]));
                if (a > amax) amax = a;
            }
            uint16_t d = oracle_float_to_half(amax / 7.0f);
            float df = (float)oracle_half_to_double(d);
            scales[v * 8 + g] = d;
            for (int j = 0; j < 32; j++) {
                int q = 0;
                if (df != 0.0f) {
                    float r = rintf((float)oracle_half_to_double(xg[j]) / df);
                    q = r < -8.0f ? -8 : r > 7.0f ? 7 : (int)r;
                }
                nib[v * 256 + 32 * g + j] = (uint8_t)(q + 8);
            }
        }
    return OR_OK;
}

/* out[h][256] (and the bound A[h][256] = sum_t p_t |v_t|) in fp64 from the
 * logical cache: knib / vnib [n_kv][T][256], ks / vs [n_kv][T][8]. */
int oracle_attn_decode(const uint16_t *q, const uint8_t *knib, const uint16_t *ks,
                       const uint8_t *vnib, const uint16_t *vs, int64_t T, int64_t n_q,
                       int64_t n_kv, double *out, double *A)
{
    if (!q || !knib || !ks || !vnib || !vs || !out) return OR_ERR_NULL;
    if (T < 1 || n_kv < 1 || n_q < 1 || n_q % n_kv) return OR_ERR_SHAPE;
    int64_t rep = n_q / n_kv;
    double *s = (double *)malloc((size_t)T * sizeof(double));
    if (!s) return OR_ERR_NOMEM;
    for (int64_t h = 0; h < n_q; h++) {
        int64_t kvh = h / rep;
        double smax = -INFINITY;
        for (int64_t t = 0; t < T; t++) {
            const uint8_t *kn = knib + (kvh * T + t) * 256;
            const uint16_t *kd = ks + (kvh * T + t) * 8;
            double dot = 0.0;
            for (int j = 0; j < 256; j++)
                dot += oracle_half_to_double(q[h * 256 + j]) *
                       ((double)kn[j] - 8.0) * oracle_half_to_double(kd[j / 32]);
            s[t] = dot / 16.0;                     /* 1 / sqrt(256) */
            if (s[t] > smax) smax = s[t];
        }
        double sum = 0.0;
        for (int64_t t = 0; t < T; t++) {
            s[t] = exp(s[t] - smax);
            sum += s[t];
        }
        for (int j = 0; j < 256; j++) {
            double o = 0.0, a = 0.0;
            for (int64_t t = 0; t < T; t++) {
                double vv = ((double)vnib[(kvh * T + t) * 256 + j] - 8.0) *
                            oracle_half_to_double(vs[(kvh * T + t) * 8 + j / 32]);
                o += s[t] / sum * vv;
                a += s[t] / sum * fabs(vv);
            }
            out[h * 256 + j] = o;
            if (A) A[h * 256 + j] = a;
        }
    }
    free(s);
    return OR_OK;
}

