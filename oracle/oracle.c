/*
 * CPU oracle for the k-quant weight matmul.
 *
 * TEST INFRASTRUCTURE ONLY. The tests, the smoke check and the CPU-baseline
 * leg of the benchmark call it; the product library never does, and this file
 * shares no code, header or table with it.
 *
 * Plain C99, plain loops, OpenMP over independent rows, no intrinsics.
 *
 * What it computes:
 *
 *  1. The activation plane. f32 activations are quantized on the fly, per
 *     token row, in blocks of 32 values, to int8 with one f32 scale and one
 *     f32 sum per block. The pages say activations are quantized on the fly
 *     with precomputed per-subblock sums (minfer Support Matrix, "Supported
 *     Quantization Formats") and that the CUDA prefill path feeds a q8 plane
 *     produced by the activation's producer (minfer Features, "GPU — CUDA").
 *     They do not give the rounding rule. Reading taken:
 *         amax = max |x_i|,  d = amax / 127 (f32 division),
 *         q_i  = 0 if d == 0 else clamp(roundf(x_i / d), -127, 127),
 *         s    = d * (float)(sum of q_i)        (one f32 rounding).
 *     d == 0 covers amax == 0 and an amax below 127 * 2^-150, whose
 *     quotient underflows to zero.
 *
 *  2. The matmul. out[t][n] = sum_k w[n][k] * d[t][k/32] * q[t][k], with w
 *     the dequantized weight of GGML's Q4_K, Q5_K or Q6_K 256-value super-block
 *     (minfer Architecture, §6 Quantization & Tensor Layout: blocks match
 *     ggml-common.h) and weights stored [out][in] row-major (minfer
 *     Architecture, §4.5 Core invariants, item 3). It is evaluated as exact
 *     integer dots over each scale group (32 values for Q4_K and Q5_K, 16 for
 *     Q6_K),
 *     combined in double from exact decodes of the f16 fields, and rounded
 *     once to f32. The stored activation sum s is not used: the Q4_K / Q5_K
 *     min term recomputes the exact integer sum of q.
 *
 * Block layouts (all fields little-endian):
 *   Q4_K, 144 B: f16 d | f16 dmin | 12 B of eight 6-bit scale codes and eight
 *     6-bit min codes | 128 B of 4-bit quants. Weight w = 64c + 32h + i lies in
 *     sub-block j = 2c + h and is (qs[32c + i] >> 4h) & 15; its value is
 *     d*sc_j*q - dmin*m_j.
 *   Q6_K, 210 B: 128 B low nibbles | 64 B high bit pairs | 16 int8 scales |
 *     f16 d. Weight w = 128g + 32r + i has low 4 bits
 *     (ql[64g + 32(r%2) + i] >> 4(r/2)) & 15 and high 2 bits
 *     (qh[32g + i] >> 2r) & 3; its value is d*scales[w/16]*(q - 32).
 *   Q5_K, 176 B: f16 d | f16 dmin | the same 12 B of scale and min codes as
 *     Q4_K | 32 B of high bits | 128 B of low nibbles. Weight w = 64c + 32h + i
 *     lies in sub-block j = 2c + h; its 5-bit quant has low 4 bits
 *     (qs[32c + i] >> 4h) & 15 and high bit (qh[i] >> (2c + h)) & 1, and its
 *     value is d*sc_j*q - dmin*m_j (the pages list q5_K among the MMVQ
 *     formats, minfer Support Matrix, "Supported Quantization Formats"; the
 *     layout is GGML's).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Exact IEEE binary16 -> double, subnormals included. */
static double f16_to_double(uint16_t h)
{
    int sign = h >> 15;
    int e = (h >> 10) & 31;
    int m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m + 1024), e - 25);
    return sign ? -v : v;
}

/* ---------------------------------------------------------------------- */
/* Activation quantizer.                                                   */
/* ---------------------------------------------------------------------- */

void oracle_quantize_act(const float *x, int64_t M, int64_t K, int64_t ldx,
                         int8_t *q, float *d, float *s)
{
    const int64_t nb = K / 32;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < M; ++t) {
        for (int64_t b = 0; b < nb; ++b) {
            const float *xb = x + t * ldx + 32 * b;
            float amax = 0.0f;
            for (int i = 0; i < 32; ++i) {
                float a = fabsf(xb[i]);
                if (a > amax)
                    amax = a;
            }
            float db = amax / 127.0f;
            int sum = 0;
            for (int i = 0; i < 32; ++i) {
                int qi = 0;
                if (db != 0.0f) {
                    float r = roundf(xb[i] / db);
                    if (r > 127.0f)
                        r = 127.0f;
                    if (r < -127.0f)
                        r = -127.0f;
                    qi = (int)r;
                }
                q[t * K + 32 * b + i] = (int8_t)qi;
                sum += qi;
            }
            d[t * nb + b] = db;
            s[t * nb + b] = db * (float)sum;
        }
    }
}

/* ---------------------------------------------------------------------- */
/* Block decoders.                                                         */
/* ---------------------------------------------------------------------- */

/* The 12-byte field of eight 6-bit scale codes and eight 6-bit min codes
 * shared by Q4_K and Q5_K: codes 0..3 are the low 6 bits of bytes 0..3
 * (scales) and 4..7 (mins); codes 4..7 take their low 4 bits from the low
 * (scale) or high (min) nibble of bytes 8..11 and their top 2 bits from the
 * top bits of bytes 0..3 (scale) or 4..7 (min). */
static void decode_scale_min(const uint8_t *B, int32_t sc[8], int32_t m[8])
{
    for (int j = 0; j < 4; ++j) {
        sc[j] = B[j] & 63;
        m[j] = B[j + 4] & 63;
    }
    for (int j = 4; j < 8; ++j) {
        sc[j] = (B[j + 4] & 15) | ((B[j - 4] >> 6) << 4);
        m[j] = (B[j + 4] >> 4) | ((B[j] >> 6) << 4);
    }
}

void oracle_q4k_block_decode(const uint8_t *blk, double *d, double *dmin,
                             int32_t sc[8], int32_t m[8], uint8_t q4[256])
{
    *d = f16_to_double((uint16_t)(blk[0] | (blk[1] << 8)));
    *dmin = f16_to_double((uint16_t)(blk[2] | (blk[3] << 8)));
    decode_scale_min(blk + 4, sc, m);
    const uint8_t *qs = blk + 16;
    for (int w = 0; w < 256; ++w) {
        int c = w / 64, h = (w / 32) % 2, i = w % 32;
        q4[w] = (uint8_t)((qs[32 * c + i] >> (4 * h)) & 15);
    }
}

void oracle_q5k_block_decode(const uint8_t *blk, double *d, double *dmin,
                             int32_t sc[8], int32_t m[8], uint8_t q5[256])
{
    *d = f16_to_double((uint16_t)(blk[0] | (blk[1] << 8)));
    *dmin = f16_to_double((uint16_t)(blk[2] | (blk[3] << 8)));
    decode_scale_min(blk + 4, sc, m);
    const uint8_t *qh = blk + 16;
    const uint8_t *qs = blk + 48;
    for (int w = 0; w < 256; ++w) {
        int c = w / 64, h = (w / 32) % 2, i = w % 32;
        int low4 = (qs[32 * c + i] >> (4 * h)) & 15;
        int high1 = (qh[i] >> (2 * c + h)) & 1;
        q5[w] = (uint8_t)(low4 | (high1 << 4));
    }
}

void oracle_q6k_block_decode(const uint8_t *blk, double *d, int32_t sc[16],
                             uint8_t q6[256])
{
    const uint8_t *ql = blk;
    const uint8_t *qh = blk + 128;
    const int8_t *scales = (const int8_t *)(blk + 192);
    *d = f16_to_double((uint16_t)(blk[208] | (blk[209] << 8)));
    for (int j = 0; j < 16; ++j)
        sc[j] = scales[j];
    for (int w = 0; w < 256; ++w) {
        int g = w / 128, r = (w / 32) % 4, i = w % 32;
        int low4 = (ql[64 * g + 32 * (r % 2) + i] >> (4 * (r / 2))) & 15;
        int high2 = (qh[32 * g + i] >> (2 * r)) & 3;
        q6[w] = (uint8_t)(low4 | (high2 << 4));
    }
}

/* ---------------------------------------------------------------------- */
/* Registration-time planes (the pages add weight-expansion planes for    */
/* the q6_K MMQ GEMM and a decoded-scale plane for q4_K at weight         */
/* registration: minfer Features, "GPU — CUDA", the W_exp / W_dsc planes  */
/* and their memory knob). Their contents are not given; readings taken:  */
/*  - Q6_K expansion: every weight's integer p = sc_g * (q - 32) (g its    */
/*    16-value group) as two int8 planes, lo = p mod 64 (0..63) and        */
/*    hi = floor(p / 64) (-64..64), so p = 64 hi + lo; plus d per super-   */
/*    block as f32. Planes are [N][K] and [N][K/256].                      */
/*  - Q4_K decoded scales: d*sc_j and dmin*m_j per 32-value sub-block j as */
/*    f32 (both exact: an f16 times a 6-bit integer), planes [N][K/32].    */
/* ---------------------------------------------------------------------- */

void oracle_expand_q6k(const uint8_t *W, int64_t N, int64_t K, int8_t *lo,
                       int8_t *hi, float *dw)
{
    const int64_t nsb = K / 256;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t sb = 0; sb < nsb; ++sb) {
            double d;
            int32_t sc[16];
            uint8_t q6[256];
            oracle_q6k_block_decode(W + (n * nsb + sb) * 210, &d, sc, q6);
            dw[n * nsb + sb] = (float)d;
            for (int w = 0; w < 256; ++w) {
                const int32_t p = sc[w / 16] * ((int32_t)q6[w] - 32);
                /* floor division and the matching non-negative remainder */
                int32_t h = p / 64;
                if (p % 64 != 0 && p < 0)
                    h -= 1;
                const int64_t k = n * K + sb * 256 + w;
                hi[k] = (int8_t)h;
                lo[k] = (int8_t)(p - 64 * h);
            }
        }
    }
}

void oracle_dsc_q4k(const uint8_t *W, int64_t N, int64_t K, float *fw, float *fm)
{
    const int64_t nsb = K / 256;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t sb = 0; sb < nsb; ++sb) {
            double d, dmin;
            int32_t sc[8], m[8];
            uint8_t q4[256];
            oracle_q4k_block_decode(W + (n * nsb + sb) * 144, &d, &dmin, sc, m, q4);
            for (int j = 0; j < 8; ++j) {
                fw[n * nsb * 8 + sb * 8 + j] = (float)(d * sc[j]);
                fm[n * nsb * 8 + sb * 8 + j] = (float)(dmin * m[j]);
            }
        }
    }
}

/* ---------------------------------------------------------------------- */
/* Matmuls. out is [ntok][N]; token tt is toks[tt] (or tt when toks is    */
/* NULL). Exactly one of out64 / out32 is non-NULL.                        */
/* ---------------------------------------------------------------------- */

/* Q4_K and Q5_K: per 32-value sub-block, d*sc*(exact int dot of the quants
 * with q) - dmin*m*(exact int sum of q), scaled by the activation block's d. */
typedef void (*scale_min_decoder)(const uint8_t *, double *, double *, int32_t *,
                                  int32_t *, uint8_t *);

static void matmul_scale_min(const uint8_t *W, int64_t block_bytes,
                             scale_min_decoder decode, const int8_t *q,
                             const float *dx, int64_t M, int64_t N, int64_t K,
                             const int64_t *toks, int64_t ntok, double *out64,
                             float *out32)
{
    const int64_t nsb = K / 256, nb = K / 32;
    const int64_t rowb = nsb * block_bytes;
    if (!toks)
        ntok = M;
#pragma omp parallel
    {
        uint8_t *qw = (uint8_t *)malloc((size_t)K);
        double *dsc = (double *)malloc(sizeof(double) * (size_t)nb);
        double *dmm = (double *)malloc(sizeof(double) * (size_t)nb);
#pragma omp for schedule(static)
        for (int64_t n = 0; n < N; ++n) {
            for (int64_t sb = 0; sb < nsb; ++sb) {
                double d, dmin;
                int32_t sc[8], m[8];
                decode(W + n * rowb + sb * block_bytes, &d, &dmin, sc, m,
                       qw + 256 * sb);
                for (int j = 0; j < 8; ++j) {
                    dsc[8 * sb + j] = d * sc[j];
                    dmm[8 * sb + j] = dmin * m[j];
                }
            }
            for (int64_t tt = 0; tt < ntok; ++tt) {
                const int64_t t = toks ? toks[tt] : tt;
                const int8_t *qt = q + t * K;
                double acc = 0.0;
                for (int64_t b = 0; b < nb; ++b) {
                    int32_t I = 0, Qs = 0;
                    for (int i = 0; i < 32; ++i) {
                        int32_t xq = qt[32 * b + i];
                        I += (int32_t)qw[32 * b + i] * xq;
                        Qs += xq;
                    }
                    double dxb = (double)dx[t * nb + b];
                    acc += dsc[b] * dxb * (double)I - dmm[b] * dxb * (double)Qs;
                }
                if (out64)
                    out64[tt * N + n] = acc;
                else
                    out32[tt * N + n] = (float)acc;
            }
        }
        free(qw);
        free(dsc);
        free(dmm);
    }
}

void oracle_matmul_q4k(const uint8_t *W, const int8_t *q, const float *dx,
                       int64_t M, int64_t N, int64_t K,
                       const int64_t *toks, int64_t ntok,
                       double *out64, float *out32)
{
    matmul_scale_min(W, 144, oracle_q4k_block_decode, q, dx, M, N, K, toks,
                     ntok, out64, out32);
}

void oracle_matmul_q5k(const uint8_t *W, const int8_t *q, const float *dx,
                       int64_t M, int64_t N, int64_t K,
                       const int64_t *toks, int64_t ntok,
                       double *out64, float *out32)
{
    matmul_scale_min(W, 176, oracle_q5k_block_decode, q, dx, M, N, K, toks,
                     ntok, out64, out32);
}

void oracle_matmul_q6k(const uint8_t *W, const int8_t *q, const float *dx,
                       int64_t M, int64_t N, int64_t K,
                       const int64_t *toks, int64_t ntok,
                       double *out64, float *out32)
{
    const int64_t nsb = K / 256, ng = K / 16, nb = K / 32;
    const int64_t rowb = nsb * 210;
    if (!toks)
        ntok = M;
#pragma omp parallel
    {
        int32_t *qv = (int32_t *)malloc(sizeof(int32_t) * (size_t)K);
        double *dsc = (double *)malloc(sizeof(double) * (size_t)ng);
#pragma omp for schedule(static)
        for (int64_t n = 0; n < N; ++n) {
            for (int64_t sb = 0; sb < nsb; ++sb) {
                double d;
                int32_t sc[16];
                uint8_t q6[256];
                oracle_q6k_block_decode(W + n * rowb + sb * 210, &d, sc, q6);
                for (int j = 0; j < 16; ++j)
                    dsc[16 * sb + j] = d * sc[j];
                for (int w = 0; w < 256; ++w)
                    qv[256 * sb + w] = (int32_t)q6[w] - 32;
            }
            for (int64_t tt = 0; tt < ntok; ++tt) {
                const int64_t t = toks ? toks[tt] : tt;
                const int8_t *qt = q + t * K;
                double acc = 0.0;
                for (int64_t g = 0; g < ng; ++g) {
                    int32_t J = 0;
                    for (int i = 0; i < 16; ++i)
                        J += qv[16 * g + i] * (int32_t)qt[16 * g + i];
                    double dxb = (double)dx[t * nb + g / 2];
                    acc += dsc[g] * dxb * (double)J;
                }
                if (out64)
                    out64[tt * N + n] = acc;
                else
                    out32[tt * N + n] = (float)acc;
            }
        }
        free(qv);
        free(dsc);
    }
}

/* ---------------------------------------------------------------------- */
/* Thread control for the timed CPU baseline.                              */
/* ---------------------------------------------------------------------- */

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}
