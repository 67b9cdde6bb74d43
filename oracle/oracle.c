/*
 * oracle.c -- plain, slow, obviously-correct CPU reference for the quantized
 * GEMV / mmq path.  TEST INFRASTRUCTURE ONLY: it is loaded by the tests, by the
 * smoke check and by the bench's CPU-baseline leg, never by the product path.
 * It shares no code, header or table with the HIP library.
 *
 * What the pages fix and what they leave open:
 *   - blazr README, "Model Formats > GGUF": the types with dedicated GPU dot
 *     kernels are Q4_K, Q6_K and Q8_0, the other GGUF types run on a generic
 *     path; the pages give no byte layout.  Q5_K is one of those others.
 *   - infr page, "Vulkan-first, Metal too": GPU output is checked against a
 *     CPU reference backend -- the role this file plays.
 *   - Block layouts and dequant formulas are GGUF's published ones (the pages
 *     are silent): Q8_0 = fp16 d + 32 int8; Q8_1 = fp16 d + fp16 s + 32 int8;
 *     Q4_K = fp16 d, fp16 dmin, 12 bytes of packed 6-bit scales/mins, 128
 *     bytes of nibbles (w = d*sc*q - dmin*m); Q6_K = 128 bytes low nibbles,
 *     64 bytes high 2-bit pairs, 16 int8 scales, fp16 d (w = d*sc*(q-32));
 *     Q5_K = Q4_K's header, 32 bytes of fifth bits, 128 bytes of nibbles
 *     (w = d*sc*q - dmin*m with q in 0..31); the 32-value types Q4_0 = fp16 d
 *     + 16 bytes of nibbles (w = d*(q - 8)) and Q5_0 = fp16 d + 32 fifth bits
 *     + 16 bytes of nibbles (w = d*(q - 16)), two more of those others.
 *
 * Everything is computed in double from the stored fields.  The dequantizers
 * and the integer block-dot routines decode the fields independently of each
 * other (no shared element-extraction helper), so their agreement is a check.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define QK 32      /* elements per Q8_0 / Q8_1 block */
#define QKK 256    /* elements per K-quant superblock */
#define B_Q8_0 34
#define B_Q8_1 36
#define B_Q4_K 144
#define B_Q6_K 210
#define B_Q5_K 176
#define B_Q4_0 18
#define B_Q5_0 22

/* ------------------------------------------------------------------------ */
/* IEEE-754 binary16 <-> binary32, written from the format definition.       */
/* ------------------------------------------------------------------------ */

/* OpenMP threads the routines below use (the CPU-baseline timing runs them
 * on one thread and on all threads); no arithmetic depends on it. */
void orc_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
int orc_max_threads(void) { return omp_get_max_threads(); }

float orc_f16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);              /* zero or subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m | 0x400), e - 25); /* 1.m * 2^(e-15) */
    return (float)(sign ? -v : v);
}

/* Round-to-nearest-even binary32 -> binary16, subnormals kept, overflow to inf. */
uint16_t orc_f32_to_f16(float f)
{
    uint16_t sign = signbit(f) ? 0x8000 : 0;
    double a = fabs((double)f);
    if (isnan(f))
        return sign | 0x7e00;
    if (a >= 65520.0) /* halfway between 65504 and 2^16 rounds (to even) up to inf */
        return sign | 0x7c00;
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: value = q * 2^-24, q in [0, 1024] */
        double q = rint(a * ldexp(1.0, 24)); /* exact scaling, RNE rounding */
        return sign | (uint16_t)q;           /* q == 1024 is the smallest normal */
    }
    int E;
    frexp(a, &E);       /* a = fr * 2^E, fr in [0.5, 1) */
    int e = E - 1;      /* a = 1.xxx * 2^e */
    double q = rint(ldexp(a, 10 - e)); /* significand scaled to [1024, 2048] */
    if (q >= 2048.0) {
        q = 1024.0;
        e += 1;
    }
    if (e + 15 >= 31)
        return sign | 0x7c00;
    return sign | (uint16_t)(((e + 15) << 10) | ((int)q - 1024));
}

void orc_f16_to_f32_n(const uint16_t *h, float *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_f16_to_f32(h[i]);
}

void orc_f32_to_f16_n(const float *f, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_f32_to_f16(f[i]);
}

static uint16_t rd16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static void wr16(uint8_t *p, uint16_t v) { p[0] = (uint8_t)(v & 0xff); p[1] = (uint8_t)(v >> 8); }
static double h2d(const uint8_t *p) { return (double)orc_f16_to_f32(rd16(p)); }

/* ------------------------------------------------------------------------ */
/* RMS scale of an activation row (the RMSNorm that precedes a projection in  */
/* the model families the infr page runs): r = 1 / sqrt(sum(x^2)/k + eps),    */
/* in double, from the f32 values.  The normalized row is x * r * gamma.      */
/* ------------------------------------------------------------------------ */
void orc_rms_scale(const float *x, double *r, int64_t rows, int64_t k, double eps)
{
    for (int64_t i = 0; i < rows; ++i) {
        double ss = 0.0;
        for (int64_t t = 0; t < k; ++t)
            ss += (double)x[i * k + t] * (double)x[i * k + t];
        r[i] = 1.0 / sqrt(ss / (double)k + eps);
    }
}

/* ------------------------------------------------------------------------ */
/* Activation quantization to Q8_1 (on the path).                             */
/* Per 32-element block: amax; d = amax/127 (fp32, correctly rounded);        */
/* q = round-half-away(x/d) from the fp32 d, clamped to +-127; s = d*sum(q)   */
/* as an fp32 product; d and s are each rounded once to fp16 (RNE).           */
/* All-zero block: d = s = 0, q = 0.                                          */
/* ------------------------------------------------------------------------ */
void orc_quantize_q8_1(const float *x, uint8_t *xq, int64_t rows, int64_t k)
{
    int64_t nb = k / QK;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            const float *xb = x + r * k + b * QK;
            uint8_t *o = xq + (r * nb + b) * B_Q8_1;
            float amax = 0.0f;
            for (int i = 0; i < QK; ++i)
                if (fabsf(xb[i]) > amax)
                    amax = fabsf(xb[i]);
            float d = amax / 127.0f;
            int sum = 0;
            for (int i = 0; i < QK; ++i) {
                int q = 0;
                if (amax != 0.0f) {
                    q = (int)roundf(xb[i] / d);
                    if (q > 127) q = 127;
                    if (q < -127) q = -127;
                }
                o[4 + i] = (uint8_t)(int8_t)q;
                sum += q;
            }
            float s = d * (float)sum;
            wr16(o + 0, orc_f32_to_f16(d));
            wr16(o + 2, orc_f32_to_f16(s));
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Field decoders (exported so tests can check them against hand-built blocks */
/* and against the input generator's packer).                                 */
/* ------------------------------------------------------------------------ */

/* Q4_K: 6-bit scale sc[j] and min m[j] of sub-block j from the 12 packed bytes.
 * j < 4: low 6 bits of bytes j (scale) and j+4 (min).
 * j >= 4: low nibble (scale) / high nibble (min) of byte j+4, with the top two
 * bits taken from the spare top bits of bytes j-4 (scale) and j (min). */
static void q4k_scale_min(const uint8_t *sc12, int j, int *sc, int *m)
{
    if (j < 4) {
        *sc = sc12[j] & 63;
        *m = sc12[j + 4] & 63;
    } else {
        *sc = (sc12[j + 4] & 0x0f) | ((sc12[j - 4] >> 6) << 4);
        *m = (sc12[j + 4] >> 4) | ((sc12[j] >> 6) << 4);
    }
}

/* Decode one Q4_K superblock into its fields. q[i] is element i's 4-bit code. */
void orc_unpack_q4_k(const uint8_t *blk, float *d, float *dmin, int32_t *sc, int32_t *m, int32_t *q)
{
    *d = orc_f16_to_f32(rd16(blk));
    *dmin = orc_f16_to_f32(rd16(blk + 2));
    for (int j = 0; j < 8; ++j) {
        int a, b;
        q4k_scale_min(blk + 4, j, &a, &b);
        sc[j] = a;
        m[j] = b;
    }
    /* 32-byte group g holds elements 64g..64g+31 in its low nibbles and
     * 64g+32..64g+63 in its high nibbles. */
    const uint8_t *qs = blk + 16;
    for (int i = 0; i < QKK; ++i) {
        int g = i / 64, r = i % 64;
        uint8_t byte = qs[32 * g + (r % 32)];
        q[i] = (r < 32) ? (byte & 0x0f) : (byte >> 4);
    }
}

/* Decode one Q5_K superblock: fp16 d, fp16 dmin, the 12 scale bytes packed as
 * Q4_K's, qh[32], qs[128].  Element i (sub-block j = i/32) takes its low four
 * bits from qs by Q4_K's rule and its fifth bit from bit j of qh[i % 32]:
 * q[i] in 0..31. */
void orc_unpack_q5_k(const uint8_t *blk, float *d, float *dmin, int32_t *sc, int32_t *m, int32_t *q)
{
    *d = orc_f16_to_f32(rd16(blk));
    *dmin = orc_f16_to_f32(rd16(blk + 2));
    for (int j = 0; j < 8; ++j) {
        int a, b;
        q4k_scale_min(blk + 4, j, &a, &b);
        sc[j] = a;
        m[j] = b;
    }
    const uint8_t *qh = blk + 16, *qs = blk + 48;
    for (int i = 0; i < QKK; ++i) {
        int g = i / 64, r = i % 64, j = i / 32;
        uint8_t byte = qs[32 * g + (r % 32)];
        int nib = (r < 32) ? (byte & 0x0f) : (byte >> 4);
        q[i] = nib | (((qh[i % 32] >> j) & 1) << 4);
    }
}

/* Decode one Q4_0 block: element i < 16 is the low nibble of qs[i] (bytes
 * 2..17), element 16 + i the high nibble; q in 0..15, w = d*(q - 8). */
void orc_unpack_q4_0(const uint8_t *blk, float *d, int32_t *q)
{
    *d = orc_f16_to_f32(rd16(blk));
    const uint8_t *qs = blk + 2;
    for (int i = 0; i < QK; ++i)
        q[i] = (i < 16) ? (qs[i] & 0x0f) : (qs[i - 16] >> 4);
}

/* Decode one Q5_0 block: fp16 d, then qh (bytes 2..5): bit i of that
 * little-endian 32-bit field is element i's fifth bit; the low four bits are
 * placed as in Q4_0 (qs at bytes 6..21).  q in 0..31, w = d*(q - 16). */
void orc_unpack_q5_0(const uint8_t *blk, float *d, int32_t *q)
{
    *d = orc_f16_to_f32(rd16(blk));
    const uint8_t *qh = blk + 2, *qs = blk + 6;
    for (int i = 0; i < QK; ++i) {
        int nib = (i < 16) ? (qs[i] & 0x0f) : (qs[i - 16] >> 4);
        int hb = (qh[i / 8] >> (i % 8)) & 1;
        q[i] = nib | (hb << 4);
    }
}

/* Decode one Q6_K superblock.  q[i] is element i's 6-bit code (0..63). */
void orc_unpack_q6_k(const uint8_t *blk, float *d, int32_t *sc, int32_t *q)
{
    const uint8_t *ql = blk, *qh = blk + 128;
    const int8_t *scales = (const int8_t *)(blk + 192);
    *d = orc_f16_to_f32(rd16(blk + 208));
    for (int j = 0; j < 16; ++j)
        sc[j] = scales[j];
    /* element 128h + 32g + l: low nibble of ql[64h + l] (g=0), ql[64h+32+l]
     * (g=1), high nibble of ql[64h+l] (g=2), ql[64h+32+l] (g=3); its top two
     * bits are bits 2g..2g+1 of qh[32h + l]. */
    for (int i = 0; i < QKK; ++i) {
        int h = i / 128, g = (i % 128) / 32, l = i % 32;
        uint8_t lo = ql[64 * h + l + 32 * (g & 1)];
        int nib = (g < 2) ? (lo & 0x0f) : (lo >> 4);
        int hi = (qh[32 * h + l] >> (2 * g)) & 3;
        q[i] = nib | (hi << 4);
    }
}

/* ------------------------------------------------------------------------ */
/* Dequantizers: rows of blocks -> double.                                    */
/* ------------------------------------------------------------------------ */

void orc_dequant_q8_0(const uint8_t *w, double *out, int64_t rows, int64_t k)
{
    int64_t nb = k / QK;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t *blk = w + (r * nb + b) * B_Q8_0;
            double d = h2d(blk);
            for (int i = 0; i < QK; ++i)
                out[r * k + b * QK + i] = d * (double)(int8_t)blk[2 + i];
        }
}

void orc_dequant_q8_1(const uint8_t *xq, double *out, int64_t rows, int64_t k)
{
    int64_t nb = k / QK;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t *blk = xq + (r * nb + b) * B_Q8_1;
            double d = h2d(blk);
            for (int i = 0; i < QK; ++i)
                out[r * k + b * QK + i] = d * (double)(int8_t)blk[4 + i];
        }
}

void orc_dequant_q4_k(const uint8_t *w, double *out, int64_t rows, int64_t k)
{
    int64_t ns = k / QKK;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t s = 0; s < ns; ++s) {
            const uint8_t *blk = w + (r * ns + s) * B_Q4_K;
            float d, dmin;
            int32_t sc[8], m[8], q[QKK];
            orc_unpack_q4_k(blk, &d, &dmin, sc, m, q);
            for (int i = 0; i < QKK; ++i) {
                int j = i / 32;
                out[r * k + s * QKK + i] = (double)d * sc[j] * q[i] - (double)dmin * m[j];
            }
        }
}

void orc_dequant_q5_k(const uint8_t *w, double *out, int64_t rows, int64_t k)
{
    int64_t ns = k / QKK;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t s = 0; s < ns; ++s) {
            const uint8_t *blk = w + (r * ns + s) * B_Q5_K;
            float d, dmin;
            int32_t sc[8], m[8], q[QKK];
            orc_unpack_q5_k(blk, &d, &dmin, sc, m, q);
            for (int i = 0; i < QKK; ++i) {
                int j = i / 32;
                out[r * k + s * QKK + i] = (double)d * sc[j] * q[i] - (double)dmin * m[j];
            }
        }
}

void orc_dequant_q4_0(const uint8_t *w, double *out, int64_t rows, int64_t k)
{
    int64_t nb = k / QK;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            float d;
            int32_t q[QK];
            orc_unpack_q4_0(w + (r * nb + b) * B_Q4_0, &d, q);
            for (int i = 0; i < QK; ++i)
                out[r * k + b * QK + i] = (double)d * (q[i] - 8);
        }
}

void orc_dequant_q5_0(const uint8_t *w, double *out, int64_t rows, int64_t k)
{
    int64_t nb = k / QK;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            float d;
            int32_t q[QK];
            orc_unpack_q5_0(w + (r * nb + b) * B_Q5_0, &d, q);
            for (int i = 0; i < QK; ++i)
                out[r * k + b * QK + i] = (double)d * (q[i] - 16);
        }
}

void orc_dequant_q6_k(const uint8_t *w, double *out, int64_t rows, int64_t k)
{
    int64_t ns = k / QKK;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t s = 0; s < ns; ++s) {
            const uint8_t *blk = w + (r * ns + s) * B_Q6_K;
            float d;
            int32_t sc[16], q[QKK];
            orc_unpack_q6_k(blk, &d, sc, q);
            for (int i = 0; i < QKK; ++i)
                out[r * k + s * QKK + i] = (double)d * sc[i / 16] * (q[i] - 32);
        }
}

/* ------------------------------------------------------------------------ */
/* GEMV, plain definition: y[n] = sum_k w^[n,k] * x^[k], both operands        */
/* dequantized exactly to double.  `sel` (nsel entries) picks output rows;    */
/* sel == NULL means all n rows (nsel ignored).  y has one entry per row      */
/* computed.                                                                  */
/* ------------------------------------------------------------------------ */

typedef void (*dequant_fn)(const uint8_t *, double *, int64_t, int64_t);

static void gemv_plain(dequant_fn deq, int64_t row_bytes, const uint8_t *w, const uint8_t *xq,
                       double *y, int64_t n, int64_t k, const int64_t *sel, int64_t nsel)
{
    int64_t cnt = sel ? nsel : n;
    double *xd = (double *)malloc(sizeof(double) * (size_t)(k > 0 ? k : 1));
    orc_dequant_q8_1(xq, xd, 1, k);
#pragma omp parallel
    {
        double *wd = (double *)malloc(sizeof(double) * (size_t)(k > 0 ? k : 1));
#pragma omp for schedule(static)
        for (int64_t i = 0; i < cnt; ++i) {
            int64_t row = sel ? sel[i] : i;
            deq(w + row * row_bytes, wd, 1, k);
            double acc = 0.0;
            for (int64_t c = 0; c < k; ++c)
                acc += wd[c] * xd[c];
            y[i] = acc;
        }
        free(wd);
    }
    free(xd);
}

void orc_qgemv_q8_0(const uint8_t *w, const uint8_t *xq, double *y, int64_t n, int64_t k,
                    const int64_t *sel, int64_t nsel)
{
    gemv_plain(orc_dequant_q8_0, (k / QK) * B_Q8_0, w, xq, y, n, k, sel, nsel);
}

void orc_qgemv_q4_k(const uint8_t *w, const uint8_t *xq, double *y, int64_t n, int64_t k,
                    const int64_t *sel, int64_t nsel)
{
    gemv_plain(orc_dequant_q4_k, (k / QKK) * B_Q4_K, w, xq, y, n, k, sel, nsel);
}

void orc_qgemv_q5_k(const uint8_t *w, const uint8_t *xq, double *y, int64_t n, int64_t k,
                    const int64_t *sel, int64_t nsel)
{
    gemv_plain(orc_dequant_q5_k, (k / QKK) * B_Q5_K, w, xq, y, n, k, sel, nsel);
}

void orc_qgemv_q6_k(const uint8_t *w, const uint8_t *xq, double *y, int64_t n, int64_t k,
                    const int64_t *sel, int64_t nsel)
{
    gemv_plain(orc_dequant_q6_k, (k / QKK) * B_Q6_K, w, xq, y, n, k, sel, nsel);
}

void orc_qgemv_q4_0(const uint8_t *w, const uint8_t *xq, double *y, int64_t n, int64_t k,
                    const int64_t *sel, int64_t nsel)
{
    gemv_plain(orc_dequant_q4_0, (k / QK) * B_Q4_0, w, xq, y, n, k, sel, nsel);
}

void orc_qgemv_q5_0(const uint8_t *w, const uint8_t *xq, double *y, int64_t n, int64_t k,
                    const int64_t *sel, int64_t nsel)
{
    gemv_plain(orc_dequant_q5_0, (k / QK) * B_Q5_0, w, xq, y, n, k, sel, nsel);
}

/* ------------------------------------------------------------------------ */
/* Per-block integer dots (the quantities the GPU must reproduce exactly).    */
/* Decoding here is written directly against the byte layout, separately     */
/* from the dequantizers above.                                               */
/* ------------------------------------------------------------------------ */

/* Q8_0: D[n][b] = sum_{i<32} qw[i] * qa[i]. */
void orc_blockdots_q8_0(const uint8_t *w, const uint8_t *xq, int32_t *D, int64_t n, int64_t k)
{
    int64_t nb = k / QK;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            const int8_t *qw = (const int8_t *)(w + (r * nb + b) * B_Q8_0 + 2);
            const int8_t *qa = (const int8_t *)(xq + b * B_Q8_1 + 4);
            int32_t acc = 0;
            for (int i = 0; i < QK; ++i)
                acc += (int32_t)qw[i] * qa[i];
            D[r * nb + b] = acc;
        }
}

/* Q4_0 and Q5_0: D[n][b] = sum_{i<32} (q[i] - off) * qa[i], off = 8 or 16.
 * Byte j of qs carries elements j (low nibble) and j + 16 (high nibble); for
 * Q5_0 the fifth bits are read as one little-endian 32-bit word. */
static void blockdots_legacy(int five, const uint8_t *w, const uint8_t *xq, int32_t *D, int64_t n, int64_t k)
{
    int64_t nb = k / QK;
    int bytes = five ? B_Q5_0 : B_Q4_0, off = five ? 16 : 8;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t *blk = w + (r * nb + b) * bytes;
            uint32_t qh = 0;
            if (five)
                qh = (uint32_t)blk[2] | ((uint32_t)blk[3] << 8) | ((uint32_t)blk[4] << 16) | ((uint32_t)blk[5] << 24);
            const uint8_t *qs = blk + (five ? 6 : 2);
            const int8_t *qa = (const int8_t *)(xq + b * B_Q8_1 + 4);
            int32_t acc = 0;
            for (int j = 0; j < 16; ++j) {
                int lo = qs[j] & 0x0f, hi = qs[j] >> 4;
                if (five) {
                    lo |= (int)((qh >> j) & 1u) << 4;
                    hi |= (int)((qh >> (j + 16)) & 1u) << 4;
                }
                acc += (lo - off) * qa[j] + (hi - off) * qa[j + 16];
            }
            D[r * nb + b] = acc;
        }
}

void orc_blockdots_q4_0(const uint8_t *w, const uint8_t *xq, int32_t *D, int64_t n, int64_t k)
{
    blockdots_legacy(0, w, xq, D, n, k);
}

void orc_blockdots_q5_0(const uint8_t *w, const uint8_t *xq, int32_t *D, int64_t n, int64_t k)
{
    blockdots_legacy(1, w, xq, D, n, k);
}

/* Q4_K: D[n][8s+j] = sum_{i<32} q[i] * qa[i] over sub-block j of superblock s
 * (q the unsigned nibble), and S[b] = sum_{i<32} qa[i] of activation block b. */
void orc_blockdots_q4_k(const uint8_t *w, const uint8_t *xq, int32_t *D, int32_t *S, int64_t n, int64_t k)
{
    int64_t ns = k / QKK, nb = k / QK;
    for (int64_t b = 0; b < nb; ++b) {
        const int8_t *qa = (const int8_t *)(xq + b * B_Q8_1 + 4);
        int32_t acc = 0;
        for (int i = 0; i < QK; ++i)
            acc += qa[i];
        S[b] = acc;
    }
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r)
        for (int64_t s = 0; s < ns; ++s) {
            const uint8_t *qs = w + (r * ns + s) * B_Q4_K + 16;
            for (int j = 0; j < 8; ++j) {
                /* sub-block j lives in byte group j/2, low nibbles if j even */
                const int8_t *qa = (const int8_t *)(xq + (s * 8 + j) * B_Q8_1 + 4);
                int32_t acc = 0;
                for (int i = 0; i < QK; ++i) {
                    uint8_t byte = qs[32 * (j / 2) + i];
                    int q = (j % 2 == 0) ? (byte & 15) : (byte >> 4);
                    acc += q * qa[i];
                }
                D[r * nb + s * 8 + j] = acc;
            }
        }
}

/* Q5_K: as Q4_K with the 5-bit code: D[n][8s+j] = sum_{i<32} q[i] * qa[i],
 * q = nibble | (bit j of qh[i]) << 4; S[b] = sum of qa over activation block b. */
void orc_blockdots_q5_k(const uint8_t *w, const uint8_t *xq, int32_t *D, int32_t *S, int64_t n, int64_t k)
{
    int64_t ns = k / QKK, nb = k / QK;
    for (int64_t b = 0; b < nb; ++b) {
        const int8_t *qa = (const int8_t *)(xq + b * B_Q8_1 + 4);
        int32_t acc = 0;
        for (int i = 0; i < QK; ++i)
            acc += qa[i];
        S[b] = acc;
    }
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r)
        for (int64_t s = 0; s < ns; ++s) {
            const uint8_t *blk = w + (r * ns + s) * B_Q5_K;
            const uint8_t *qh = blk + 16, *qs = blk + 48;
            for (int j = 0; j < 8; ++j) {
                const int8_t *qa = (const int8_t *)(xq + (s * 8 + j) * B_Q8_1 + 4);
                int32_t acc = 0;
                for (int i = 0; i < QK; ++i) {
                    uint8_t byte = qs[32 * (j / 2) + i];
                    int q = ((j % 2 == 0) ? (byte & 15) : (byte >> 4)) | (((qh[i] >> j) & 1) << 4);
                    acc += q * qa[i];
                }
                D[r * nb + s * 8 + j] = acc;
            }
        }
}

/* Q6_K: D[n][16s+j] = sum_{i<16} (q[i]-32) * qa over 16-element sub-block j of
 * superblock s; its activation is half (j%2) of Q8_1 block 8s + j/2. */
void orc_blockdots_q6_k(const uint8_t *w, const uint8_t *xq, int32_t *D, int64_t n, int64_t k)
{
    int64_t ns = k / QKK;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r)
        for (int64_t s = 0; s < ns; ++s) {
            const uint8_t *blk = w + (r * ns + s) * B_Q6_K;
            for (int j = 0; j < 16; ++j) {
                const int8_t *qa = (const int8_t *)(xq + (s * 8 + j / 2) * B_Q8_1 + 4 + 16 * (j % 2));
                int32_t acc = 0;
                for (int i = 0; i < 16; ++i) {
                    int e = 16 * j + i;         /* element within the superblock */
                    int half = e / 128, rem = e % 128;
                    int grp = rem / 32, l = rem % 32;
                    uint8_t lo = blk[64 * half + l + ((grp == 1 || grp == 3) ? 32 : 0)];
                    int nib = (grp >= 2) ? (lo >> 4) : (lo & 15);
                    int top = (blk[128 + 32 * half + l] >> (2 * grp)) & 3;
                    acc += ((nib | (top << 4)) - 32) * qa[i];
                }
                D[r * ns * 16 + s * 16 + j] = acc;
            }
        }
}

/* GEMV from the integer dots, factored per block:
 *   Q8_0: sum_b dw*da*D;   Q4_K, Q5_K: sum_{s,j} da*(d*sc_j*D - dmin*m_j*S);
 *   Q6_K: sum_{s,j} d*sc_j*da*D;   Q4_0, Q5_0: sum_b dw*da*D.
 *   fmt: 0 Q8_0, 1 Q4_K, 2 Q6_K, 3 Q5_K, 4 Q4_0, 5 Q5_0.
 * Exactly equal (up to double rounding) to the plain definition. */
void orc_qgemv_factored(int fmt, const uint8_t *w, const uint8_t *xq, double *y, int64_t n, int64_t k)
{
    int64_t nb = k / QK, ns = k / QKK;
    int32_t *D = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n * (nb * 2 + 1)));
    int32_t *S = (int32_t *)malloc(sizeof(int32_t) * (size_t)(nb + 1));
    if (fmt == 0)
        orc_blockdots_q8_0(w, xq, D, n, k);
    else if (fmt == 4)
        orc_blockdots_q4_0(w, xq, D, n, k);
    else if (fmt == 5)
        orc_blockdots_q5_0(w, xq, D, n, k);
    else if (fmt == 1)
        orc_blockdots_q4_k(w, xq, D, S, n, k);
    else if (fmt == 3)
        orc_blockdots_q5_k(w, xq, D, S, n, k);
    else
        orc_blockdots_q6_k(w, xq, D, n, k);
    for (int64_t r = 0; r < n; ++r) {
        double acc = 0.0;
        if (fmt == 0 || fmt == 4 || fmt == 5) {
            int bytes = fmt == 0 ? B_Q8_0 : (fmt == 4 ? B_Q4_0 : B_Q5_0);
            for (int64_t b = 0; b < nb; ++b)
                acc += h2d(w + (r * nb + b) * bytes) * h2d(xq + b * B_Q8_1) * D[r * nb + b];
        } else if (fmt == 1 || fmt == 3) {
            for (int64_t s = 0; s < ns; ++s) {
                const uint8_t *blk = w + (r * ns + s) * (fmt == 1 ? B_Q4_K : B_Q5_K);
                double d = h2d(blk), dmin = h2d(blk + 2);
                for (int j = 0; j < 8; ++j) {
                    int sc, m;
                    q4k_scale_min(blk + 4, j, &sc, &m);
                    int64_t b = s * 8 + j;
                    acc += h2d(xq + b * B_Q8_1) * (d * sc * D[r * nb + b] - dmin * m * S[b]);
                }
            }
        } else {
            for (int64_t s = 0; s < ns; ++s) {
                const uint8_t *blk = w + (r * ns + s) * B_Q6_K;
                double d = h2d(blk + 208);
                for (int j = 0; j < 16; ++j)
                    acc += d * (int8_t)blk[192 + j] * h2d(xq + (s * 8 + j / 2) * B_Q8_1) *
                           D[r * ns * 16 + s * 16 + j];
            }
        }
        y[r] = acc;
    }
    free(D);
    free(S);
}

/* ------------------------------------------------------------------------ */
/* Prefill product (mmq), plain definition:                                   */
/*   C[m][n] = sum_k a^[m,k] * w^[n,k]                                        */
/* A is Q8_1 [M][K/32]; B is Q4_K, Q5_K or Q6_K [N][K/256] or Q8_0, Q4_0 or   */
/* Q5_0 [N][K/32];                                                            */
/* C row-major [M][N].  Both operands are dequantized exactly to double and   */
/* dotted in k order.                                                         */
/* `sel` picks (m, n) pairs: sel[2i], sel[2i+1]; NULL means every entry.      */
/* ------------------------------------------------------------------------ */
typedef void (*dequant_fn)(const uint8_t *, double *, int64_t, int64_t);

static void qgemm_plain(dequant_fn deq, int64_t wrow, const uint8_t *w, const uint8_t *aq, double *c, int64_t m,
                        int64_t n, int64_t k, const int64_t *sel, int64_t nsel)
{
    int64_t arow = (k / QK) * B_Q8_1;
    if (sel) {
#pragma omp parallel
        {
            double *wd = (double *)malloc(sizeof(double) * (size_t)(k + 1));
            double *ad = (double *)malloc(sizeof(double) * (size_t)(k + 1));
#pragma omp for schedule(static)
            for (int64_t i = 0; i < nsel; ++i) {
                int64_t mi = sel[2 * i], ni = sel[2 * i + 1];
                deq(w + ni * wrow, wd, 1, k);
                orc_dequant_q8_1(aq + mi * arow, ad, 1, k);
                double acc = 0.0;
                for (int64_t t = 0; t < k; ++t)
                    acc += ad[t] * wd[t];
                c[i] = acc;
            }
            free(wd);
            free(ad);
        }
        return;
    }
    double *W = (double *)malloc(sizeof(double) * (size_t)(n * k + 1));
    double *A = (double *)malloc(sizeof(double) * (size_t)(m * k + 1));
    deq(w, W, n, k);
    orc_dequant_q8_1(aq, A, m, k);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j) {
            double acc = 0.0;
            for (int64_t t = 0; t < k; ++t)
                acc += A[i * k + t] * W[j * k + t];
            c[i * n + j] = acc;
        }
    free(W);
    free(A);
}

void orc_qgemm_q4_k(const uint8_t *w, const uint8_t *aq, double *c, int64_t m, int64_t n, int64_t k,
                    const int64_t *sel, int64_t nsel)
{
    qgemm_plain(orc_dequant_q4_k, (k / QKK) * B_Q4_K, w, aq, c, m, n, k, sel, nsel);
}

void orc_qgemm_q5_k(const uint8_t *w, const uint8_t *aq, double *c, int64_t m, int64_t n, int64_t k,
                    const int64_t *sel, int64_t nsel)
{
    qgemm_plain(orc_dequant_q5_k, (k / QKK) * B_Q5_K, w, aq, c, m, n, k, sel, nsel);
}

void orc_qgemm_q6_k(const uint8_t *w, const uint8_t *aq, double *c, int64_t m, int64_t n, int64_t k,
                    const int64_t *sel, int64_t nsel)
{
    qgemm_plain(orc_dequant_q6_k, (k / QKK) * B_Q6_K, w, aq, c, m, n, k, sel, nsel);
}

void orc_qgemm_q8_0(const uint8_t *w, const uint8_t *aq, double *c, int64_t m, int64_t n, int64_t k,
                    const int64_t *sel, int64_t nsel)
{
    qgemm_plain(orc_dequant_q8_0, (k / QK) * B_Q8_0, w, aq, c, m, n, k, sel, nsel);
}

void orc_qgemm_q4_0(const uint8_t *w, const uint8_t *aq, double *c, int64_t m, int64_t n, int64_t k,
                    const int64_t *sel, int64_t nsel)
{
    qgemm_plain(orc_dequant_q4_0, (k / QK) * B_Q4_0, w, aq, c, m, n, k, sel, nsel);
}

void orc_qgemm_q5_0(const uint8_t *w, const uint8_t *aq, double *c, int64_t m, int64_t n, int64_t k,
                    const int64_t *sel, int64_t nsel)
{
    qgemm_plain(orc_dequant_q5_0, (k / QK) * B_Q5_0, w, aq, c, m, n, k, sel, nsel);
}

/* mmq per-block dots: for every activation row, the GEMV block dots of that  */
/* row against all weight rows.  Q4_K, Q5_K and the 32-value types:          */
/* D[m][n][k/32]; Q6_K: the                                                   */
/* 16-value sub-block dots, D[m][n][k/16].                                    */
void orc_blockdots_q4_k_mmq(const uint8_t *w, const uint8_t *aq, int32_t *D, int64_t m, int64_t n, int64_t k)
{
    int64_t nb = k / QK;
    int32_t *S = (int32_t *)malloc(sizeof(int32_t) * (size_t)(nb + 1));
    int32_t *row = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n * nb + 1));
    for (int64_t i = 0; i < m; ++i) {
        orc_blockdots_q4_k(w, aq + i * nb * B_Q8_1, row, S, n, k);
        memcpy(D + i * n * nb, row, sizeof(int32_t) * (size_t)(n * nb));
    }
    free(S);
    free(row);
}

void orc_blockdots_q5_k_mmq(const uint8_t *w, const uint8_t *aq, int32_t *D, int64_t m, int64_t n, int64_t k)
{
    int64_t nb = k / QK;
    int32_t *S = (int32_t *)malloc(sizeof(int32_t) * (size_t)(nb + 1));
    for (int64_t i = 0; i < m; ++i)
        orc_blockdots_q5_k(w, aq + i * nb * B_Q8_1, D + i * n * nb, S, n, k);
    free(S);
}

void orc_blockdots_q6_k_mmq(const uint8_t *w, const uint8_t *aq, int32_t *D, int64_t m, int64_t n, int64_t k)
{
    int64_t nb = k / QK, per = k / 16;
    for (int64_t i = 0; i < m; ++i)
        orc_blockdots_q6_k(w, aq + i * nb * B_Q8_1, D + i * n * per, n, k);
}

void orc_blockdots_q8_0_mmq(const uint8_t *w, const uint8_t *aq, int32_t *D, int64_t m, int64_t n, int64_t k)
{
    int64_t nb = k / QK;
    for (int64_t i = 0; i < m; ++i)
        orc_blockdots_q8_0(w, aq + i * nb * B_Q8_1, D + i * n * nb, n, k);
}

void orc_blockdots_q4_0_mmq(const uint8_t *w, const uint8_t *aq, int32_t *D, int64_t m, int64_t n, int64_t k)
{
    int64_t nb = k / QK;
    for (int64_t i = 0; i < m; ++i)
        orc_blockdots_q4_0(w, aq + i * nb * B_Q8_1, D + i * n * nb, n, k);
}

void orc_blockdots_q5_0_mmq(const uint8_t *w, const uint8_t *aq, int32_t *D, int64_t m, int64_t n, int64_t k)
{
    int64_t nb = k / QK;
    for (int64_t i = 0; i < m; ++i)
        orc_blockdots_q5_0(w, aq + i * nb * B_Q8_1, D + i * n * nb, n, k);
}

/* ------------------------------------------------------------------------ */
/* MoE router (the step that makes the routing table the expert FFN takes):  */
/*   logits[t][e] = sum_h Wr[e][h] * x[t][h]       (double, from f32 inputs)   */
/* and, from a given table of logits (f32), per token:                       */
/*   ids[t][0..K-1]: the K experts with the largest logits, larger first,     */
/*                   equal logits in increasing expert order                  */
/*   weights[t][i] = exp(l_i - l_0) / sum_j exp(l_j - l_0) over those K       */
/*                   (double)                                                 */
/* The selection takes the logits it is given, so it can be applied to the   */
/* GPU's own f32 logits and compared exactly.                                 */
/* ------------------------------------------------------------------------ */
void orc_router_logits(const float *wr, const float *x, double *logits, int64_t T, int64_t E, int64_t H)
{
    for (int64_t t = 0; t < T; ++t)
        for (int64_t e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int64_t h = 0; h < H; ++h)
                acc += (double)wr[e * H + h] * (double)x[t * H + h];
            logits[t * E + e] = acc;
        }
}

void orc_route_topk(const float *logits, int32_t *ids, double *weights, int64_t T, int64_t E, int64_t K)
{
    unsigned char *taken = (unsigned char *)malloc((size_t)(E > 0 ? E : 1));
    for (int64_t t = 0; t < T; ++t) {
        const float *l = logits + t * E;
        memset(taken, 0, (size_t)(E > 0 ? E : 1));
        for (int64_t i = 0; i < K; ++i) {
            int64_t best = -1;
            for (int64_t e = 0; e < E; ++e)
                if (!taken[e] && (best < 0 || l[e] > l[best]))   /* strict: the lower index keeps a tie */
                    best = e;
            taken[best] = 1;
            ids[t * K + i] = (int32_t)best;
        }
        double sum = 0.0;
        for (int64_t i = 0; i < K; ++i)
            sum += exp((double)l[ids[t * K + i]] - (double)l[ids[t * K]]);
        for (int64_t i = 0; i < K; ++i)
            weights[t * K + i] = exp((double)l[ids[t * K + i]] - (double)l[ids[t * K]]) / sum;
    }
    free(taken);
}

/* ------------------------------------------------------------------------ */
/* MoE expert FFN (Q4_K experts), per token t and routed slot e = ids[t][i]:  */
/*   g = Wgu[e][0:F] . x^_t,  u = Wgu[e][F:2F] . x^_t        (double)          */
/*   h = silu(g) * u, silu(g) = g / (1 + exp(-g)), rounded once to f32         */
/*   h^ = Q8_1(h)                                                              */
/*   z = Wdown[e] . h^                                       (double)          */
/*   out[t] = sum_i weights[t][i] * z                        (double)          */
/* Rows 0..F-1 of an expert's gate/up weight are the gate, F..2F-1 the up.    */
/* If hq_in is non-NULL, the down projection uses that h^ instead (stage-wise */
/* check).  gu (may be NULL) receives g|u per pair, hq_out (may be NULL) h^.  */
/* Pairs whose id lies outside [0, E) contribute nothing.                     */
/* ------------------------------------------------------------------------ */
void orc_moe_q4_k(const uint8_t *w_gu, const uint8_t *w_down, const uint8_t *xq, const int32_t *ids,
                  const float *weights, int64_t T, int64_t topk, int64_t E, int64_t F, int64_t H,
                  double *gu, uint8_t *hq_out, const uint8_t *hq_in, double *out)
{
    int64_t gu_row = (H / QKK) * B_Q4_K, gu_expert = 2 * F * gu_row;
    int64_t dn_row = (F / QKK) * B_Q4_K, dn_expert = H * dn_row;
    int64_t xq_row = (H / QK) * B_Q8_1, hq_row = (F / QK) * B_Q8_1;
    int64_t P = T * topk;
    for (int64_t i = 0; i < T * H; ++i)
        out[i] = 0.0;
    double *z = (double *)malloc(sizeof(double) * (size_t)(P * H));
    for (int64_t p = 0; p < P; ++p) {
        int64_t t = p / topk;
        int32_t e = ids[p];
        if (e < 0 || e >= E) {
            for (int64_t i = 0; i < H; ++i)
                z[p * H + i] = 0.0;
            continue;
        }
        double *g = (double *)malloc(sizeof(double) * (size_t)(2 * F));
        orc_qgemv_q4_k(w_gu + e * gu_expert, xq + t * xq_row, g, 2 * F, H, NULL, 0);
        float *h = (float *)malloc(sizeof(float) * (size_t)F);
        for (int64_t i = 0; i < F; ++i) {
            double gg = g[i], uu = g[F + i];
            double silu = gg / (1.0 + exp(-gg));
            h[i] = (float)(silu * uu);
        }
        uint8_t *hq = (uint8_t *)malloc((size_t)hq_row);
        orc_quantize_q8_1(h, hq, 1, F);
        if (gu)
            memcpy(gu + p * 2 * F, g, sizeof(double) * (size_t)(2 * F));
        if (hq_out)
            memcpy(hq_out + p * hq_row, hq, (size_t)hq_row);
        const uint8_t *hq_use = hq_in ? hq_in + p * hq_row : hq;
        orc_qgemv_q4_k(w_down + e * dn_expert, hq_use, z + p * H, H, F, NULL, 0);
        free(g);
        free(h);
        free(hq);
    }
    for (int64_t p = 0; p < P; ++p) {
        int64_t t = p / topk;
        int32_t e = ids[p];
        if (e < 0 || e >= E)
            continue;
        for (int64_t i = 0; i < H; ++i)
            out[t * H + i] += (double)weights[p] * z[p * H + i];
    }
    free(z);
}
