/*
 * Q4_0 matmul oracle: TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct CPU implementation of
 *     y[t, o] = sum_k w[o, k] * x[t, k],   w[o, k] = d[o, k/32] * (q[o, k] - 8)
 * used to check the GPU library.  Only the tests, the package's smoke check
 * and the benchmark's CPU-baseline leg may load it; the product path never
 * does.  It shares no source with the GPU library.
 *
 * What it follows:
 *  - The weight layout is the "B transposed" one of rembed's matmul
 *    interface (rembed "Architecture", section "The pluggable kernel
 *    interface"): W is [out x in] row-major, so every output is the dot
 *    product of two contiguous rows.
 *  - Weights come in groups of 32 sharing one scale, with small integer
 *    codes stored two to a byte (goinfer primer ch. 10, "Making Go fast
 *    enough" and "Layout, concretely").  Within a group the split-half order
 *    is used: byte i carries weight i in its low four bits (masking the byte
 *    gives it) and weight i+16 in its high four bits (shifting right by four
 *    gives it), per "Layout, concretely".  The pages do not say which order
 *    GGUF's Q4_0 uses; split-half is taken as GGUF's order.
 *  - A block is 18 bytes: the binary16 scale d, little-endian, then the 16
 *    code bytes; each weight decodes to d * (q - 8).  The pages describe a
 *    block only as a scale with small integers; the 18-byte block, the
 *    scale's position and the offset 8 are the GGUF Q4_0 definition.
 *
 * Arithmetic: each row is dequantized to float32 (exact: d has 11
 * significant bits, q - 8 at most 4), every product is formed in float64
 * (exact: at most 15 + 24 significant bits) and summed in float64 in k order.
 * Alongside y the oracle returns den[t, o] = sum_k |w[o, k] * x[t, k]|, the
 * denominator of the acceptance ratio |y - y_ref| / den.
 *
 * Parity pins (tests/test_oracle_pins.py): zero codes, constant codes against
 * an independent row sum, exact rational brute force on tiny shapes, a
 * vectorised numpy decode at full sizes, a hand-built split-half example, the
 * binary16 decoder against numpy on all 65536 bit patterns, and invariants.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define Q4O_BLOCK 32
#define Q4O_BLOCK_BYTES 18

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits with bias 15, 10 fraction
 * bits.  Exponent 0 holds zeros and subnormals (f * 2^-24), exponent 31 holds
 * infinities (f == 0) and NaNs.  Every binary16 value is exact in float32. */
float q4o_half_to_float(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    float v;
    if (e == 0)
        v = ldexpf((float)f, -24);
    else if (e == 31)
        v = (f == 0) ? INFINITY : NAN;
    else
        v = ldexpf((float)(1024 + f), e - 25);
    return sign ? -v : v;
}

/* Code of weight j (0..31) of a block whose 16 code bytes start at qs. */
static int q4o_code(const uint8_t *qs, int j)
{
    return (j < 16) ? (qs[j] & 0x0f) : (qs[j - 16] >> 4);
}

/* Dequantize row o of an [out x in] block matrix to float32. */
static void q4o_dequant_row(const uint8_t *blocks, int64_t in, int64_t o, float *w)
{
    int64_t nb = in / Q4O_BLOCK;
    for (int64_t b = 0; b < nb; ++b) {
        const uint8_t *blk = blocks + (o * nb + b) * Q4O_BLOCK_BYTES;
        float d = q4o_half_to_float((uint16_t)(blk[0] | (blk[1] << 8)));
        const uint8_t *qs = blk + 2;
        for (int j = 0; j < Q4O_BLOCK; ++j)
            w[b * Q4O_BLOCK + j] = d * (float)(q4o_code(qs, j) - 8);
    }
}

/* Whole matrix to float32, [out x in] row-major.  Returns 0, or -1 when in is
 * not a whole number of blocks. */
int q4o_dequantize(const uint8_t *blocks, int64_t out, int64_t in, float *w)
{
    if (in <= 0 || in % Q4O_BLOCK != 0 || out <= 0)
        return -1;
    for (int64_t o = 0; o < out; ++o)
        q4o_dequant_row(blocks, in, o, w + o * in);
    return 0;
}

typedef struct {
    const uint8_t *blocks;
    const float *x;      /* [n x in], float32 */
    int64_t n, out, in;
    const int64_t *rows; /* rows to compute, or NULL for 0..out-1 */
    int64_t nrows;
    double *y, *den;     /* [n x nrows] */
    int64_t lo, hi;      /* this worker's slice of the row list */
} q4o_job;

static void *q4o_worker(void *arg)
{
    q4o_job *j = (q4o_job *)arg;
    float *w = (float *)malloc((size_t)j->in * sizeof(float));
    if (!w)
        return (void *)1;
    for (int64_t i = j->lo; i < j->hi; ++i) {
        int64_t o = j->rows ? j->rows[i] : i;
        q4o_dequant_row(j->blocks, j->in, o, w);
        for (int64_t t = 0; t < j->n; ++t) {
            const float *xt = j->x + t * j->in;
            double acc = 0.0, mag = 0.0;
            for (int64_t k = 0; k < j->in; ++k) {
                double p = (double)w[k] * (double)xt[k];
                acc += p;
                mag += fabs(p);
            }
            j->y[t * j->nrows + i] = acc;
            if (j->den)
                j->den[t * j->nrows + i] = mag;
        }
    }
    free(w);
    return NULL;
}

static int q4o_hw_threads(void)
{
    long c = sysconf(_SC_NPROCESSORS_ONLN);
    return c > 0 ? (int)c : 1;
}

/* y[t, i] (and den[t, i]) for rows[i], i < nrows, or for every row when rows
 * is NULL (then nrows must equal out).  x is float32 (x_is_f16 == 0) or
 * binary16 bit patterns (x_is_f16 == 1), [n x in] row-major.  nthreads <= 0
 * uses every online core.  Returns the number of threads used, or a negative
 * value on a bad argument or allocation failure. */
int q4o_matmul_rows(const uint8_t *blocks, const void *x, int x_is_f16,
                    int64_t n, int64_t out, int64_t in,
                    const int64_t *rows, int64_t nrows,
                    double *y, double *den, int nthreads)
{
    if (!blocks || !x || !y || n <= 0 || out <= 0 || in <= 0 || in % Q4O_BLOCK)
        return -1;
    if (!rows && nrows != out)
        return -1;
    for (int64_t i = 0; rows && i < nrows; ++i)
        if (rows[i] < 0 || rows[i] >= out)
            return -1;

    const float *xf = (const float *)x;
    float *xconv = NULL;
    if (x_is_f16) {
        xconv = (float *)malloc((size_t)(n * in) * sizeof(float));
        if (!xconv)
            return -2;
        const uint16_t *xh = (const uint16_t *)x;
        for (int64_t i = 0; i < n * in; ++i)
            xconv[i] = q4o_half_to_float(xh[i]);
        xf = xconv;
    }

    if (nthreads <= 0)
        nthreads = q4o_hw_threads();
    if (nthreads > nrows)
        nthreads = (int)nrows;
    if (nthreads < 1)
        nthreads = 1;

    pthread_t *tid = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    q4o_job *jobs = (q4o_job *)calloc((size_t)nthreads, sizeof(q4o_job));
    if (!tid || !jobs) {
        free(tid); free(jobs); free(xconv);
        return -2;
    }
    int rc = 0;
    for (int i = 0; i < nthreads; ++i) {
        q4o_job *j = &jobs[i];
        j->blocks = blocks; j->x = xf; j->n = n; j->out = out; j->in = in;
        j->rows = rows; j->nrows = nrows; j->y = y; j->den = den;
        j->lo = nrows * i / nthreads;
        j->hi = nrows * (i + 1) / nthreads;
        if (pthread_create(&tid[i], NULL, q4o_worker, j) != 0) {
            nthreads = i;
            rc = -2;
            break;
        }
    }
    for (int i = 0; i < nthreads; ++i) {
        void *r = NULL;
        pthread_join(tid[i], &r);
        if (r)
            rc = -2;
    }
    free(tid); free(jobs); free(xconv);
    return rc < 0 ? rc : nthreads;
}

/* All rows: y and den are [n x out]. */
int q4o_matmul(const uint8_t *blocks, const void *x, int x_is_f16,
               int64_t n, int64_t out, int64_t in,
               double *y, double *den, int nthreads)
{
    return q4o_matmul_rows(blocks, x, x_is_f16, n, out, in, NULL, out,
                           y, den, nthreads);
}

/*
 * W4A8: int4 weights against int8 activations.
 *
 * What it follows: rembed "Architecture", section "int8 quantization" (full
 * int8: activations quantized to 8-bit integers, an integer dot product per
 * output, an offset correction subtracted in the epilogue, checked bit for
 * bit against an integer reference) and the goinfer primer ch. 10 "Which
 * kernel runs is a runtime decision" (the quantized dot on 8-bit integer
 * dot-product hardware).  The pages do not give the activations' scale
 * granularity; the reading taken here is one scale per 32 activations of a
 * row, the weights' block size, so that every block's integer sum is scaled
 * once: d = max |x| / 127 over the block (float32 division), q = x / d
 * rounded to nearest, ties to even (float32 division, then rint), and q = 0
 * for every value of a block whose d is not a positive finite number.
 */

/* Quantize x [n x in] (float32) per 32-value block: q [n x in] int8 codes,
 * d [n x in/32] float32 scales.  Returns 0, or -1 on a bad shape. */
int q4o_quantize_x8(const float *x, int64_t n, int64_t in, int8_t *q, float *d)
{
    if (!x || !q || !d || n <= 0 || in <= 0 || in % Q4O_BLOCK)
        return -1;
    int64_t nb = in / Q4O_BLOCK;
    for (int64_t t = 0; t < n; ++t)
        for (int64_t b = 0; b < nb; ++b) {
            const float *xb = x + t * in + b * Q4O_BLOCK;
            float amax = 0.0f;
            for (int j = 0; j < Q4O_BLOCK; ++j) {
                float a = fabsf(xb[j]);
                if (a > amax || a != a)      /* a NaN makes the maximum NaN */
                    amax = a;
            }
            float s = amax / 127.0f;
            d[t * nb + b] = s;
            int ok = s > 0.0f && s <= 3.4028234663852886e38f;
            for (int j = 0; j < Q4O_BLOCK; ++j)
                q[t * in + b * Q4O_BLOCK + j] = ok ? (int8_t)rintf(xb[j] / s) : 0;
        }
    return 0;
}

typedef struct {
    const uint8_t *blocks;
    const int8_t *q;     /* [n x in] */
    const float *d;      /* [n x nb] */
    int64_t n, out, in;
    const int64_t *rows;
    int64_t nrows;
    double *y, *den;
    int64_t lo, hi;
} q4o_job8;

static void *q4o_worker8(void *arg)
{
    q4o_job8 *j = (q4o_job8 *)arg;
    int64_t nb = j->in / Q4O_BLOCK;
    for (int64_t i = j->lo; i < j->hi; ++i) {
        int64_t o = j->rows ? j->rows[i] : i;
        for (int64_t t = 0; t < j->n; ++t) {
            double acc = 0.0, mag = 0.0;
            for (int64_t b = 0; b < nb; ++b) {
                const uint8_t *blk = j->blocks + (o * nb + b) * Q4O_BLOCK_BYTES;
                double dw = (double)q4o_half_to_float((uint16_t)(blk[0] | (blk[1] << 8)));
                double dx = (double)j->d[t * nb + b];
                const int8_t *qx = j->q + t * j->in + b * Q4O_BLOCK;
                int64_t isum = 0, iabs = 0;
                for (int k = 0; k < Q4O_BLOCK; ++k) {
                    int64_t p = (int64_t)(q4o_code(blk + 2, k) - 8) * (int64_t)qx[k];
                    isum += p;
                    iabs += p < 0 ? -p : p;
                }
                acc += dw * dx * (double)isum;           /* exact product */
                mag += fabs(dw * dx) * (double)iabs;
            }
            j->y[t * j->nrows + i] = acc;
            if (j->den)
                j->den[t * j->nrows + i] = mag;
        }
    }
    return NULL;
}

/* y[t, i] = sum_b dw[o, b] * d[t, b] * sum_{k in b} (qw[o, k] - 8) * q[t, k]
 * for rows[i] (every row when rows is NULL), with exact integer block sums
 * and float64 scaling; den[t, i] = sum_b |dw d| * sum_k |(qw - 8) q|.
 * Returns the number of threads used, or a negative value on error. */
int q4o_matmul_w4a8_rows(const uint8_t *blocks, const int8_t *q, const float *d,
                         int64_t n, int64_t out, int64_t in,
                         const int64_t *rows, int64_t nrows,
                         double *y, double *den, int nthreads)
{
    if (!blocks || !q || !d || !y || n <= 0 || out <= 0 || in <= 0 || in % Q4O_BLOCK)
        return -1;
    if (!rows && nrows != out)
        return -1;
    for (int64_t i = 0; rows && i < nrows; ++i)
        if (rows[i] < 0 || rows[i] >= out)
            return -1;
    if (nthreads <= 0)
        nthreads = q4o_hw_threads();
    if (nthreads > nrows)
        nthreads = (int)nrows;
    if (nthreads < 1)
        nthreads = 1;
    pthread_t *tid = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    q4o_job8 *jobs = (q4o_job8 *)calloc((size_t)nthreads, sizeof(q4o_job8));
    if (!tid || !jobs) {
        free(tid); free(jobs);
        return -2;
    }
    int rc = 0;
    for (int i = 0; i < nthreads; ++i) {
        q4o_job8 *j = &jobs[i];
        j->blocks = blocks; j->q = q; j->d = d; j->n = n; j->out = out; j->in = in;
        j->rows = rows; j->nrows = nrows; j->y = y; j->den = den;
        j->lo = nrows * i / nthreads;
        j->hi = nrows * (i + 1) / nthreads;
        if (pthread_create(&tid[i], NULL, q4o_worker8, j) != 0) {
            nthreads = i;
            rc = -2;
            break;
        }
    }
    for (int i = 0; i < nthreads; ++i)
        pthread_join(tid[i], NULL);
    free(tid); free(jobs);
    return rc < 0 ? rc : nthreads;
}
