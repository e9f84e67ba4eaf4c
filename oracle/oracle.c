/*
 * oracle.c -- plain, slow, obviously-correct CPU oracle for the group-quantised
 * 4-bit-weight matrix multiply (AWQ W4A16) and its QQQ-style W4A8 variant.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the reference that the GPU library is
 * checked against.  Only the test suite, the smoke check and the benchmark's
 * cpu_baseline leg may load it.  It shares no code, header, table or helper with
 * the GPU library, and the GPU library never loads it.
 *
 * Everything is scalar C: integers for bit work, int64 for integer dot
 * products, IEEE double for floating point.  No blocking, fusion or reordering:
 * each output is the sum over k in increasing k order.  Threads only split the
 * set of output columns.
 *
 * Sources (web pages; cited by title and passage):
 *  [P1] vLLM pull request "Speed up AWQ 2.5x with updated kernel": the reviewer's
 *       list of differences between the first-generation AWQ GEMM packing and
 *       the newer one (the order map [0,2,4,6,1,3,5,7] of the old GEMM format),
 *       and the dispatch snippet that passes (inputs, qweight, scales, qzeros,
 *       group_size) to the kernels.
 *  [P2] AutoAWQ pull request "Marlin symmetric quantization and inference": the
 *       symmetric (no zero point) variant.
 *  [P5] vLLM pull request "Support W4A8 quantization for vllm" (QQQ): the
 *       dynamic per-token int8 activation quantisation (the dynamic_quant helper
 *       in the consistency script: row abs-max divided by 127, round, clamp to
 *       [-128,127]); the per-group quantiser's affine form scale*(q - zero);
 *       the kernel review notes (int4 placed in the top nibble of an int8,
 *       int32 global reduce, per-token s1 and per-channel s2 applied to the
 *       output, per-group scales used in addition to per-channel ones).
 *
 * Readings where the pages leave a point open (each is listed in the design
 * notes of the repository):
 *  - Order map direction: nibble i (bits 4i..4i+3, word read as uint32) of a
 *    packed AWQ word holds output column 8j + AWQ_ORDER[i].
 *  - qzeros are packed exactly like qweight; a missing qzeros means z = 8.
 *  - W4A8 weights: two's-complement int4 packed along K, nibble i of word
 *    [kb][n] holds k = 8kb + K8_ORDER[i].
 *  - W4A8 per-group scales s3 are small integers (1..16) so that q*s3 is an
 *    int8 and the whole-K accumulation stays an exact int32; per-channel is the
 *    case with no s3 (w8 = q).
 *  - A row whose fp16 scale s1 rounds to zero quantises to all zeros.
 *  - Second AWQ packing (named by its differences only): identity order map,
 *    qweight [K, N/8] and scales [K/G, N] as before, qzeros [N, ceil(K/G/8)]
 *    packed along the groups with the nibbles past the last group skipped.
 *  - INT4-FP8 (the QQQ authors' announced follow-up, named only): the int8
 *    recipe with OCP FP8 E4M3 codes and 448 in place of int8 codes and 127,
 *    round to nearest even with saturation at +-448, per-channel scales.
 *
 * Parity unpinned: compatibility with real AWQ checkpoints and QQQ exports
 * (how real files apply the order map, and QQQ's own weight layout).  No such
 * file or packing source is available; every function here is pinned against
 * the pages' definitions and the mathematics only.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_EINVAL (-1)

/* [P1] first-generation AWQ GEMM order map: nibble i holds column 8j + AWQ_ORDER[i]. */
static const int AWQ_ORDER[8] = {0, 2, 4, 6, 1, 3, 5, 7};
/* W4A8 K-packed layout: nibble i of word [kb][n] holds k = 8kb + K8_ORDER[i]. */
static const int K8_ORDER[8] = {0, 4, 1, 5, 2, 6, 3, 7};

/* ------------------------------------------------------------------ */
/* Floating-point formats, decoded from their IEEE-754 bit definitions. */

/* binary16 -> double (exact). */
double orc_f16_to_f64(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24); /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m | 0x400), e - 25); /* (1024 + m) * 2^(e-15-10) */
    return sign ? -v : v;
}

/* bfloat16 -> double (exact): the top 16 bits of a binary32. */
double orc_bf16_to_f64(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* double -> binary16, round to nearest, ties to even (one rounding of the
 * double value).  Overflow goes to infinity, NaN to the quiet NaN 0x7e00. */
uint16_t orc_f64_to_f16(double v) {
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isnan(v)) return 0x7e00;
    if (a >= 65520.0) return sign | 0x7c00; /* halfway to 2^16 rounds up to inf */
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: the quantum is 2^-24; a result of 1024 quanta is the
         * smallest normal, whose encoding is the same integer 0x400. */
        double r = nearbyint(ldexp(a, 24));
        return sign | (uint16_t)r;
    }
    int e2;
    frexp(a, &e2);          /* a in [2^(e2-1), 2^e2) */
    int E = e2 - 1;         /* unbiased exponent */
    double r = nearbyint(ldexp(a, 10 - E)); /* significand in [1024, 2048] */
    if (r == 2048.0) {
        r = 1024.0;
        E += 1;
    }
    if (E > 15) return sign | 0x7c00;
    return sign | (uint16_t)((E + 15) << 10) | (uint16_t)((int)r - 1024);
}

/* double -> bfloat16 (the top 16 bits of a binary32: 8-bit significand,
 * binary32's exponent range), round to nearest, ties to even (one rounding of
 * the double value).  Overflow goes to infinity, NaN to the quiet NaN 0x7fc0. */
uint16_t orc_f64_to_bf16(double v) {
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isnan(v)) return 0x7fc0;
    /* the largest finite value is (2 - 2^-7) * 2^127; halfway to 2^128 rounds up */
    if (a >= ldexp(2.0 - ldexp(1.0, -8), 127)) return sign | 0x7f80;
    if (a < ldexp(1.0, -126)) {
        /* subnormal range: the quantum is 2^-133; 128 quanta is the smallest
         * normal, whose encoding is the same integer 0x80. */
        double r = nearbyint(ldexp(a, 133));
        return sign | (uint16_t)r;
    }
    int e2;
    frexp(a, &e2);         /* a in [2^(e2-1), 2^e2) */
    int E = e2 - 1;        /* unbiased exponent */
    double r = nearbyint(ldexp(a, 7 - E)); /* significand in [128, 256] */
    if (r == 256.0) {
        r = 128.0;
        E += 1;
    }
    if (E > 127) return sign | 0x7f80;
    return sign | (uint16_t)((E + 127) << 7) | (uint16_t)((int)r - 128);
}

/* a value rounded to the activation type (fp16 = 0, bf16 = 1) and widened back */
static double round_act(double v, int dtype) {
    return dtype == 1 ? orc_bf16_to_f64(orc_f64_to_bf16(v)) : orc_f16_to_f64(orc_f64_to_f16(v));
}

static double decode_act(uint16_t bits, int dtype) {
    return dtype == 1 ? orc_bf16_to_f64(bits) : orc_f16_to_f64(bits);
}

/* ------------------------------------------------------------------ */
/* Packing (AWQ N-packed and W4A8 K-packed).                          */

/* unpack AWQ words [rows, cols/8] -> values [rows, cols] in 0..15. */
int orc_unpack_n8(const int32_t *packed, uint8_t *vals, int64_t rows, int64_t cols) {
    if (cols % 8) return ORC_EINVAL;
    int64_t wc = cols / 8;
    for (int64_t r = 0; r < rows; r++)
        for (int64_t j = 0; j < wc; j++) {
            uint32_t w = (uint32_t)packed[r * wc + j];
            for (int i = 0; i < 8; i++)
                vals[r * cols + 8 * j + AWQ_ORDER[i]] = (uint8_t)((w >> (4 * i)) & 0xF);
        }
    return ORC_OK;
}

/* pack values [rows, cols] (expected 0..15) -> AWQ words [rows, cols/8].
 * Values above 15 are clamped to 15; the number clamped is returned in
 * *n_clamped (a missing clamp was a real packing bug reported in [P5]). */
int orc_pack_n8(const uint8_t *vals, int32_t *packed, int64_t rows, int64_t cols,
                int64_t *n_clamped) {
    if (cols % 8) return ORC_EINVAL;
    int64_t wc = cols / 8, bad = 0;
    for (int64_t r = 0; r < rows; r++)
        for (int64_t j = 0; j < wc; j++) {
            uint32_t w = 0;
            for (int i = 0; i < 8; i++) {
                unsigned v = vals[r * cols + 8 * j + AWQ_ORDER[i]];
                if (v > 15) {
                    v = 15;
                    bad++;
                }
                w |= (uint32_t)v << (4 * i);
            }
            packed[r * wc + j] = (int32_t)w;
        }
    if (n_clamped) *n_clamped = bad;
    return ORC_OK;
}

static int sext4(unsigned v) { return (int)(v ^ 8u) - 8; }

/* unpack W4A8 words [K/8, N] -> int4 values [K, N] in -8..7. */
int orc_unpack_k8(const int32_t *packed, int8_t *vals, int64_t K, int64_t N) {
    if (K % 8) return ORC_EINVAL;
    for (int64_t kb = 0; kb < K / 8; kb++)
        for (int64_t n = 0; n < N; n++) {
            uint32_t w = (uint32_t)packed[kb * N + n];
            for (int i = 0; i < 8; i++)
                vals[(8 * kb + K8_ORDER[i]) * N + n] = (int8_t)sext4((w >> (4 * i)) & 0xF);
        }
    return ORC_OK;
}

/* pack int4 values [K, N] (expected -8..7) -> W4A8 words [K/8, N]; out-of-range
 * values are clamped and counted. */
int orc_pack_k8(const int8_t *vals, int32_t *packed, int64_t K, int64_t N, int64_t *n_clamped) {
    if (K % 8) return ORC_EINVAL;
    int64_t bad = 0;
    for (int64_t kb = 0; kb < K / 8; kb++)
        for (int64_t n = 0; n < N; n++) {
            uint32_t w = 0;
            for (int i = 0; i < 8; i++) {
                int v = vals[(8 * kb + K8_ORDER[i]) * N + n];
                if (v < -8) { v = -8; bad++; }
                if (v > 7) { v = 7; bad++; }
                w |= ((uint32_t)v & 0xFu) << (4 * i);
            }
            packed[kb * N + n] = (int32_t)w;
        }
    if (n_clamped) *n_clamped = bad;
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* W4A16: Y = X . dequant(qweight, qzeros, scales),  w = (q - z) * s.  */

typedef struct {
    const double *x; /* [M, K], decoded activations */
    const int32_t *qweight, *qzeros;
    const uint16_t *scales;
    int64_t M, N, K;
    int G, dtype;
    double *y;          /* [M, N] */
    int64_t j0, j1;     /* word-column range [j0, j1) handled by this thread */
} w4a16_job;

/* Dequantise the 8 columns packed in word-column j into w[8][K] (double). */
static void dequant_word_column(const w4a16_job *t, int64_t j, double *w) {
    int64_t wc = t->N / 8;
    for (int64_t k = 0; k < t->K; k++) {
        int64_t g = k / t->G;
        uint32_t qw = (uint32_t)t->qweight[k * wc + j];
        uint32_t zw = t->qzeros ? (uint32_t)t->qzeros[g * wc + j] : 0x88888888u;
        for (int i = 0; i < 8; i++) {
            int col = AWQ_ORDER[i];
            int q = (int)((qw >> (4 * i)) & 0xF);
            int z = (int)((zw >> (4 * i)) & 0xF);
            double s = decode_act(t->scales[g * t->N + 8 * j + col], t->dtype);
            w[col * t->K + k] = (double)(q - z) * s;
        }
    }
}

static void *w4a16_worker(void *arg) {
    w4a16_job *t = (w4a16_job *)arg;
    double *w = (double *)malloc(sizeof(double) * 8 * (size_t)t->K);
    if (!w) return (void *)1;
    for (int64_t j = t->j0; j < t->j1; j++) {
        dequant_word_column(t, j, w);
        for (int c = 0; c < 8; c++) {
            const double *wc = w + (size_t)c * t->K;
            for (int64_t m = 0; m < t->M; m++) {
                const double *xr = t->x + m * t->K;
                double acc = 0.0;
                for (int64_t k = 0; k < t->K; k++) acc += xr[k] * wc[k];
                t->y[m * t->N + 8 * j + c] = acc;
            }
        }
    }
    free(w);
    return NULL;
}

static int check_w4a16_shape(int64_t M, int64_t N, int64_t K, int G) {
    if (M < 0 || N <= 0 || K <= 0 || G <= 0) return ORC_EINVAL;
    if (N % 8 || K % G) return ORC_EINVAL;
    return ORC_OK;
}

/* Y64[m,n] = sum_k x[m,k] * (q[k,n] - z[k/G,n]) * s[k/G,n], all in double.
 * x, scales: fp16 (dtype 0) or bf16 (dtype 1) bit patterns.  qzeros may be NULL
 * (symmetric, z = 8). */
int orc_w4a16(const uint16_t *x, const int32_t *qweight, const uint16_t *scales,
              const int32_t *qzeros, int64_t M, int64_t N, int64_t K, int G, int dtype,
              double *y, int nthreads) {
    if (check_w4a16_shape(M, N, K, G)) return ORC_EINVAL;
    if (nthreads < 1) nthreads = 1;
    double *xd = (double *)malloc(sizeof(double) * (size_t)(M * K + 1));
    if (!xd) return ORC_EINVAL;
    for (int64_t i = 0; i < M * K; i++) xd[i] = decode_act(x[i], dtype);
    int64_t wc = N / 8;
    if (nthreads > wc) nthreads = (int)wc;
    w4a16_job *jobs = (w4a16_job *)calloc((size_t)nthreads, sizeof(w4a16_job));
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    int rc = ORC_OK;
    for (int i = 0; i < nthreads; i++) {
        w4a16_job *t = &jobs[i];
        t->x = xd; t->qweight = qweight; t->qzeros = qzeros; t->scales = scales;
        t->M = M; t->N = N; t->K = K; t->G = G; t->dtype = dtype; t->y = y;
        t->j0 = wc * i / nthreads;
        t->j1 = wc * (i + 1) / nthreads;
    }
    for (int i = 1; i < nthreads; i++) pthread_create(&th[i], NULL, w4a16_worker, &jobs[i]);
    if (w4a16_worker(&jobs[0])) rc = ORC_EINVAL;
    for (int i = 1; i < nthreads; i++) {
        void *r;
        pthread_join(th[i], &r);
        if (r) rc = ORC_EINVAL;
    }
    free(th); free(jobs); free(xd);
    return rc;
}

/* The dequantised weight matrix W[k,n] = (q - z) * s in double, [K, N]. */
int orc_dequant(const int32_t *qweight, const uint16_t *scales, const int32_t *qzeros,
                int64_t N, int64_t K, int G, int dtype, double *w_out) {
    if (check_w4a16_shape(0, N, K, G)) return ORC_EINVAL;
    w4a16_job t;
    memset(&t, 0, sizeof t);
    t.qweight = qweight; t.qzeros = qzeros; t.scales = scales;
    t.N = N; t.K = K; t.G = G; t.dtype = dtype;
    double *w = (double *)malloc(sizeof(double) * 8 * (size_t)K);
    if (!w) return ORC_EINVAL;
    for (int64_t j = 0; j < N / 8; j++) {
        dequant_word_column(&t, j, w);
        for (int c = 0; c < 8; c++)
            for (int64_t k = 0; k < K; k++) w_out[k * N + 8 * j + c] = w[(size_t)c * K + k];
    }
    free(w);
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* W4A8 (QQQ): per-token int8 activations, int4 weights, exact integer  */
/* accumulation, output scaled by s1[m] * s2[n].                        */

/* Dynamic per-token quantisation of activations [M, K] ([P5], the
 * dynamic_quant helper), fp16 (dtype 0) or bf16 (dtype 1):
 *   amax  = max_k |x[m,k]|                          (exact in the activation type)
 *   s1    = float( act( float(amax) / 127 ) )        (the quotient is taken on the
 *                                                     activation tensor, then widened)
 *   a8    = clamp( round_half_even( float(x) / s1 ), -128, 127 )   (fp32 divide)
 * A row with s1 == 0 gives a8 = 0.  The bf16 form is this library's reading of
 * how the pages' fp16 recipe carries over to bf16 models (the pages list bf16
 * as not yet supported). */
int orc_quant_act(const uint16_t *x, int64_t M, int64_t K, int dtype, int8_t *a8, float *s1) {
    if (M < 0 || K <= 0 || (dtype != 0 && dtype != 1)) return ORC_EINVAL;
    for (int64_t m = 0; m < M; m++) {
        const uint16_t *row = x + m * K;
        double amax = 0.0;
        for (int64_t k = 0; k < K; k++) {
            double v = fabs(decode_act(row[k], dtype));
            if (v > amax) amax = v;
        }
        float q32 = (float)amax / 127.0f;                 /* fp32, correctly rounded */
        float s = (float)round_act((double)q32, dtype);   /* to the activation type and back */
        s1[m] = s;
        for (int64_t k = 0; k < K; k++) {
            if (s == 0.0f) {
                a8[m * K + k] = 0;
                continue;
            }
            float xf = (float)decode_act(row[k], dtype);
            float r = rintf(xf / s); /* round half to even (default rounding mode) */
            if (r < -128.0f) r = -128.0f;
            if (r > 127.0f) r = 127.0f;
            a8[m * K + k] = (int8_t)r;
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* Second AWQ packing ([P1]: the reviewer's list of differences of the   */
/* newer llm-awq format: order map [0,1,...,7] instead of                 */
/* [0,2,4,6,1,3,5,7]; some zeros skipped during packing; a zeros width    */
/* from calculate_zeros_width giving other shapes).  Reading, changing    */
/* only what the list names: qweight [K, N/8] with nibble i of word j     */
/* holding column 8j + i; scales [K/G, N] as before; qzeros [N, ZW] with  */
/* ZW = ceil((K/G) / 8) words per output channel, nibble i of word j      */
/* holding the zero point of group 8j + i, the nibbles past the last      */
/* group skipped (left 0).                                                */

/* words [rows, ceil(cols/8)] -> values [rows, cols] (identity order; nibbles
 * past the last column ignored) */
int orc_unpack_v2(const int32_t *packed, uint8_t *vals, int64_t rows, int64_t cols) {
    if (rows < 0 || cols < 0) return ORC_EINVAL;
    int64_t wc = (cols + 7) / 8;
    for (int64_t r = 0; r < rows; r++)
        for (int64_t c = 0; c < cols; c++)
            vals[r * cols + c] = (uint8_t)(((uint32_t)packed[r * wc + c / 8] >> (4 * (c % 8))) & 0xF);
    return ORC_OK;
}

/* values [rows, cols] -> words [rows, ceil(cols/8)]; nibbles past the last
 * column stay 0 (skipped); values above 15 are clamped and counted */
int orc_pack_v2(const uint8_t *vals, int32_t *packed, int64_t rows, int64_t cols, int64_t *n_clamped) {
    if (rows < 0 || cols < 0) return ORC_EINVAL;
    int64_t wc = (cols + 7) / 8, bad = 0;
    for (int64_t r = 0; r < rows; r++)
        for (int64_t j = 0; j < wc; j++) {
            uint32_t word = 0;
            for (int i = 0; i < 8; i++) {
                int64_t c = 8 * j + i;
                if (c >= cols) continue; /* skipped */
                unsigned v = vals[r * cols + c];
                if (v > 15) { v = 15; bad++; }
                word |= (uint32_t)v << (4 * i);
            }
            packed[r * wc + j] = (int32_t)word;
        }
    if (n_clamped) *n_clamped = bad;
    return ORC_OK;
}

/* Y64 = X . W with W[k,n] = (q[k,n] - z[n,k/G]) * s[k/G,n] read straight from
 * the second packing (qzeros NULL: z = 8), in double, summed in k order. */
int orc_w4a16_v2(const uint16_t *x, const int32_t *qweight, const uint16_t *scales, const int32_t *qzeros,
                 int64_t M, int64_t N, int64_t K, int G, int dtype, double *y) {
    if (check_w4a16_shape(M, N, K, G)) return ORC_EINVAL;
    int64_t wc = N / 8, groups = K / G, zw = (groups + 7) / 8;
    double *w = (double *)malloc(sizeof(double) * (size_t)K);
    if (!w) return ORC_EINVAL;
    for (int64_t n = 0; n < N; n++) {
        for (int64_t k = 0; k < K; k++) {
            int64_t g = k / G;
            int q = (int)(((uint32_t)qweight[k * wc + n / 8] >> (4 * (n % 8))) & 0xF);
            int z = qzeros ? (int)(((uint32_t)qzeros[n * zw + g / 8] >> (4 * (g % 8))) & 0xF) : 8;
            w[k] = (double)(q - z) * decode_act(scales[g * N + n], dtype);
        }
        for (int64_t m = 0; m < M; m++) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; k++) acc += decode_act(x[m * K + k], dtype) * w[k];
            y[m * N + n] = acc;
        }
    }
    free(w);
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* INT4-FP8 W4A8 ([P5]: the authors' announced follow-up, "INT4-FP8 QQQ  */
/* (W4A8)"; the pages give no more than its name).  Reading: the int8     */
/* recipe with the int8 code replaced by an OCP FP8 E4M3 code (1 sign,    */
/* 4 exponent bits with bias 7, 3 mantissa bits; no infinities, largest   */
/* finite 448; the all-ones pattern is NaN), the divisor 127 replaced by  */
/* 448, rounding to nearest even with saturation at +-448; int4 weights   */
/* are exact in E4M3; per-channel scales only.                            */

/* E4M3 code -> double (exact). */
double orc_e4m3_to_f64(uint8_t c) {
    int sign = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        v = ldexp((double)m, -9); /* subnormal: m * 2^-9 */
    else
        v = ldexp((double)(8 + m), e - 10); /* (1 + m/8) * 2^(e-7) */
    return sign ? -v : v;
}

/* double -> E4M3, round to nearest, ties to even, saturating at +-448
 * (the value is clamped into [-448, 448] first); NaN -> 0x7f. */
uint8_t orc_f64_to_e4m3(double v) {
    uint8_t sign = signbit(v) ? 0x80 : 0;
    double a = fabs(v);
    if (isnan(v)) return 0x7f;
    if (a > 448.0) a = 448.0;
    if (a < ldexp(1.0, -6)) {
        /* subnormal range: quantum 2^-9; 8 quanta is the smallest normal,
         * whose code is the same integer 0x08 */
        double r = nearbyint(ldexp(a, 9));
        return sign | (uint8_t)r;
    }
    int e2;
    frexp(a, &e2);        /* a in [2^(e2-1), 2^e2) */
    int E = e2 - 1;       /* unbiased exponent, -6..8 */
    double r = nearbyint(ldexp(a, 3 - E)); /* significand in [8, 16] */
    if (r == 16.0) {
        r = 8.0;
        E += 1;
    }
    return sign | (uint8_t)((E + 7) << 3) | (uint8_t)((int)r - 8);
}

/* Per-token FP8 quantisation of activations [M, K] (fp16 dtype 0, bf16 1):
 *   amax  = max_k |x[m,k]|
 *   s1    = float( act( float(amax) / 448 ) )        (fp32 divide, rounded to the activation type)
 *   a[m,k]= e4m3( clamp( float(x) / s1, -448, 448 ) ) (fp32 divide, nearest even)
 *   asum  = float( sum_k e4m3_value(a[m,k]) )        (the exact sum, rounded once)
 * A row with s1 == 0 gives codes 0 and asum 0.  asum is the row sum of the
 * quantised activations, which the GPU GEMM needs (it stores the weights with
 * an offset of 8). */
int orc_quant_act_fp8(const uint16_t *x, int64_t M, int64_t K, int dtype, uint8_t *a, float *s1,
                      float *asum) {
    if (M < 0 || K <= 0 || (dtype != 0 && dtype != 1)) return ORC_EINVAL;
    for (int64_t m = 0; m < M; m++) {
        const uint16_t *row = x + m * K;
        double amax = 0.0;
        for (int64_t k = 0; k < K; k++) {
            double mag = fabs(decode_act(row[k], dtype));
            if (mag > amax) amax = mag;
        }
        float quot = (float)amax / 448.0f;
        float s = (float)round_act((double)quot, dtype);
        s1[m] = s;
        double sum = 0.0; /* exact: multiples of 2^-9 below 2^53 * 2^-9 */
        for (int64_t k = 0; k < K; k++) {
            uint8_t c = 0;
            if (s != 0.0f) {
                float q = (float)decode_act(row[k], dtype) / s;
                if (q > 448.0f) q = 448.0f;
                if (q < -448.0f) q = -448.0f;
                c = orc_f64_to_e4m3((double)q);
            }
            a[m * K + k] = c;
            sum += orc_e4m3_to_f64(c);
        }
        asum[m] = (float)sum;
    }
    return ORC_OK;
}

/* acc[m,n] = sum_k e4m3_value(a[m,k]) * q[k,n]   (exact in double: every
 * product is a multiple of 2^-9 and every partial sum stays far below 2^44)
 * Y64[m,n] = acc * s1[m] * s2[n], with q the K8-packed int4 weights and s2
 * per output channel (fp16 dtype 0 / bf16 dtype 1).  Either output may be
 * NULL. */
int orc_w4a8_fp8(const uint8_t *a, const int32_t *b, const float *s1, const uint16_t *s2, int64_t M,
                 int64_t N, int64_t K, int dtype, double *acc, double *y) {
    if (M < 0 || N <= 0 || K <= 0 || K % 8 || (dtype != 0 && dtype != 1)) return ORC_EINVAL;
    double *av = (double *)malloc(sizeof(double) * (size_t)(M * K + 1));
    int *q = (int *)malloc(sizeof(int) * (size_t)K);
    if (!av || !q) { free(av); free(q); return ORC_EINVAL; }
    for (int64_t i = 0; i < M * K; i++) av[i] = orc_e4m3_to_f64(a[i]);
    for (int64_t n = 0; n < N; n++) {
        for (int64_t kb = 0; kb < K / 8; kb++) {
            uint32_t w = (uint32_t)b[kb * N + n];
            for (int i = 0; i < 8; i++) q[8 * kb + K8_ORDER[i]] = sext4((w >> (4 * i)) & 0xF);
        }
        double s2n = decode_act(s2[n], dtype);
        for (int64_t m = 0; m < M; m++) {
            double sacc = 0.0;
            for (int64_t k = 0; k < K; k++) sacc += av[m * K + k] * (double)q[k];
            if (acc) acc[m * N + n] = sacc;
            if (y) y[m * N + n] = sacc * (double)s1[m] * s2n;
        }
    }
    free(av);
    free(q);
    return ORC_OK;
}

typedef struct {
    const int8_t *a8;
    const int32_t *b;
    const float *s1;
    const uint16_t *s2, *s3;
    int64_t M, N, K;
    int G, dtype;
    int64_t *acc;
    double *y;
    int64_t n0, n1;
    int err;
} w4a8_job;

static void *w4a8_worker(void *arg) {
    w4a8_job *t = (w4a8_job *)arg;
    int64_t K = t->K, N = t->N;
    int *w8 = (int *)malloc(sizeof(int) * (size_t)K);
    if (!w8) { t->err = 1; return NULL; }
    for (int64_t n = t->n0; n < t->n1; n++) {
        /* dequantise column n to int8 weights w8[k] = q[k,n] (* s3[k/G,n]) */
        for (int64_t kb = 0; kb < K / 8; kb++) {
            uint32_t w = (uint32_t)t->b[kb * N + n];
            for (int i = 0; i < 8; i++) {
                int64_t k = 8 * kb + K8_ORDER[i];
                int q = sext4((w >> (4 * i)) & 0xF);
                int mult = 1;
                if (t->s3) {
                    double s3 = decode_act(t->s3[(k / t->G) * N + n], t->dtype);
                    mult = (int)s3;
                    if ((double)mult != s3 || mult < 1 || mult > 16) { t->err = 1; mult = 0; }
                }
                w8[k] = q * mult;
            }
        }
        double s2 = decode_act(t->s2[n], t->dtype);
        for (int64_t m = 0; m < t->M; m++) {
            const int8_t *ar = t->a8 + m * K;
            int64_t acc = 0;
            for (int64_t k = 0; k < K; k++) acc += (int64_t)ar[k] * (int64_t)w8[k];
            if (t->acc) t->acc[m * N + n] = acc;
            if (t->y) t->y[m * N + n] = (double)acc * (double)t->s1[m] * s2;
        }
    }
    free(w8);
    return NULL;
}

/* acc[m,n] = sum_k a8[m,k] * w8[k,n]  (int64), with w8 = q for per-channel
 * weights (s3 == NULL) or w8 = q * s3[k/G, n] for per-group weights, and
 * Y64[m,n] = acc * s1[m] * s2[n] in double; s2 and s3 are fp16 (dtype 0) or
 * bf16 (dtype 1) bit patterns.  Either output may be NULL. */
int orc_w4a8(const int8_t *a8, const int32_t *b, const float *s1, const uint16_t *s2,
             const uint16_t *s3, int64_t M, int64_t N, int64_t K, int G, int dtype, int64_t *acc,
             double *y, int nthreads) {
    if (M < 0 || N <= 0 || K <= 0 || K % 8 || (dtype != 0 && dtype != 1)) return ORC_EINVAL;
    if (s3 && (G <= 0 || K % G)) return ORC_EINVAL;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > N) nthreads = (int)N;
    w4a8_job *jobs = (w4a8_job *)calloc((size_t)nthreads, sizeof(w4a8_job));
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    for (int i = 0; i < nthreads; i++) {
        w4a8_job *t = &jobs[i];
        t->a8 = a8; t->b = b; t->s1 = s1; t->s2 = s2; t->s3 = s3;
        t->M = M; t->N = N; t->K = K; t->G = G; t->dtype = dtype; t->acc = acc; t->y = y;
        t->n0 = N * i / nthreads;
        t->n1 = N * (i + 1) / nthreads;
    }
    for (int i = 1; i < nthreads; i++) pthread_create(&th[i], NULL, w4a8_worker, &jobs[i]);
    w4a8_worker(&jobs[0]);
    int rc = ORC_OK;
    for (int i = 1; i < nthreads; i++) pthread_join(th[i], NULL);
    for (int i = 0; i < nthreads; i++)
        if (jobs[i].err) rc = ORC_EINVAL;
    free(th); free(jobs);
    return rc;
}
