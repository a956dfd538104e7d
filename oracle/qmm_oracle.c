/*
 * qmm_oracle.c -- plain, slow CPU reference for the quantized matmul.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code with the HIP kernels: its own
 * fp16 decoder (from the IEEE 754 binary16 definition), its own bit reader,
 * its own loops.
 *
 * What it computes (the method, stated from the pages):
 *   - Weights are stored with affine quantization at 2 to 8 bits
 *     ("Apple Silicon 로컬 LLM 추론의 새 기준 BaseRT" (thakicloud.com),
 *     section "BaseRT는 무엇인가": the .base format uses affine Q2..Q8).
 *   - Decode multiplies a single activation row (M = 1, a GEMV) and prefill
 *     several rows (M > 1, a GEMM) by those weights, dequantizing inside the
 *     compute loop ("BaseRT claims fastest Apple Silicon inference"
 *     (thetesserapress.com), section "What BaseRT does differently").
 *   - The result the fast kernels must reach is the plain one: unpack every
 *     code, form w = scale * q + min, take the dot product.  This file is that
 *     definition written out, in double precision, in k order.
 *
 * Readings where the pages are silent (the library's format definition):
 *   - W is N x K (output rows x reduction), row-major.
 *   - Code k of row n occupies bits [k*b, k*b + b) of that row's bitstream;
 *     stream bit i is bit (i mod 32) of 32-bit word floor(i / 32) of the row.
 *     Rows are padded to nothing: a row is exactly K*b/32 words (K*b % 32 == 0).
 *   - Codes are unsigned, 0 .. 2^b - 1.
 *   - scale and min are fp16, one of each per group of `group` consecutive k,
 *     stored as [N][K/group] row-major.  w = scale * q + min.
 *   - x is fp16 [M][K]; the result is returned in double, with
 *     a = sum_k |w x| beside it for the tolerance test.
 *
 * Threads: the row loop carries an OpenMP pragma when built with -fopenmp.
 * Every output element is still computed by one thread in k order, so the
 * result does not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <stdlib.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * exponent 0      -> subnormal: (-1)^s * f * 2^-24
 * exponent 1..30  -> normal:    (-1)^s * (1024 + f) * 2^(e - 25)
 * exponent 31     -> f == 0 ? infinity : NaN                                */
double qmo_fp16_to_double(uint16_t h)
{
    int s = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -24);
    } else if (e == 31) {
        v = (f == 0) ? INFINITY : NAN;
    } else {
        v = ldexp((double)(1024 + f), e - 25);
    }
    return s ? -v : v;
}

void qmo_fp16_array_to_double(const uint16_t *h, int64_t count, double *out)
{
    for (int64_t i = 0; i < count; ++i)
        out[i] = qmo_fp16_to_double(h[i]);
}

/* One stream bit of a packed row. */
static unsigned row_bit(const uint32_t *row, int64_t i)
{
    return (row[i / 32] >> (i % 32)) & 1u;
}

/* Code k of a packed row: q = sum_{j<b} bit(k*b + j) << j. */
static unsigned row_code(const uint32_t *row, int64_t k, int bits)
{
    unsigned q = 0;
    for (int j = 0; j < bits; ++j)
        q |= row_bit(row, k * bits + j) << j;
    return q;
}

static int64_t words_per_row(int64_t k, int bits) { return k * bits / 32; }

/* Codes of every row: codes[n*K + k]. */
void qmo_unpack(const uint32_t *w, int64_t n, int64_t k, int bits, uint8_t *codes)
{
    int64_t wpr = words_per_row(k, bits);
    for (int64_t r = 0; r < n; ++r)
        for (int64_t c = 0; c < k; ++c)
            codes[r * k + c] = (uint8_t)row_code(w + r * wpr, c, bits);
}

/* Inverse of qmo_unpack: set stream bit k*b + j of row r to bit j of the code. */
void qmo_pack(const uint8_t *codes, int64_t n, int64_t k, int bits, uint32_t *w)
{
    int64_t wpr = words_per_row(k, bits);
    for (int64_t i = 0; i < n * wpr; ++i)
        w[i] = 0;
    for (int64_t r = 0; r < n; ++r) {
        uint32_t *row = w + r * wpr;
        for (int64_t c = 0; c < k; ++c) {
            unsigned q = codes[r * k + c];
            for (int j = 0; j < bits; ++j) {
                int64_t i = c * bits + j;
                row[i / 32] |= (uint32_t)((q >> j) & 1u) << (i % 32);
            }
        }
    }
}

/* Dequantized weights in double: wd[n*K + k] = scale * q + min. */
void qmo_dequant(const uint32_t *w, const uint16_t *scales, const uint16_t *mins,
                 int64_t n, int64_t k, int bits, int group, double *wd)
{
    int64_t wpr = words_per_row(k, bits);
    int64_t gpr = k / group;
    for (int64_t r = 0; r < n; ++r)
        for (int64_t c = 0; c < k; ++c) {
            double s = qmo_fp16_to_double(scales[r * gpr + c / group]);
            double m = qmo_fp16_to_double(mins[r * gpr + c / group]);
            double q = (double)row_code(w + r * wpr, c, bits);
            wd[r * k + c] = s * q + m;
        }
}

/* y[i*N + r] = sum_k w[r,k] x[i,k];  a[i*N + r] = sum_k |w[r,k] x[i,k]|.
 * x_rows, when not NULL, names the row of x that output row i uses
 * (x_rows[i]); otherwise output row i uses x row i.  a may be NULL.        */
static void qmm_rows(const uint32_t *w, const uint16_t *scales, const uint16_t *mins,
                     const uint16_t *x, const int32_t *x_rows, int64_t m_rows,
                     int64_t n, int64_t k, int bits, int group,
                     double *y, double *a, int64_t y_stride)
{
    int64_t wpr = words_per_row(k, bits);
    int64_t gpr = k / group;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 16)
#endif
    for (int64_t r = 0; r < n; ++r) {
        const uint32_t *row = w + r * wpr;
        for (int64_t i = 0; i < m_rows; ++i) {
            const uint16_t *xr = x + (x_rows ? (int64_t)x_rows[i] : i) * k;
            double acc = 0.0, acc_abs = 0.0;
            for (int64_t c = 0; c < k; ++c) {
                double s = qmo_fp16_to_double(scales[r * gpr + c / group]);
                double m = qmo_fp16_to_double(mins[r * gpr + c / group]);
                double wv = s * (double)row_code(row, c, bits) + m;
                double p = wv * qmo_fp16_to_double(xr[c]);
                acc += p;
                acc_abs += fabs(p);
            }
            y[i * y_stride + r] = acc;
            if (a)
                a[i * y_stride + r] = acc_abs;
        }
    }
}

/* Y = X W^T for M rows of x (M = 1 is the decode GEMV). */
void qmo_qmm(const uint32_t *w, const uint16_t *scales, const uint16_t *mins,
             const uint16_t *x, int64_t m, int64_t n, int64_t k, int bits, int group,
             double *y, double *a)
{
    qmm_rows(w, scales, mins, x, NULL, m, n, k, bits, group, y, a, n);
}

/* Only the listed output rows of Y = X W^T: for each j < count,
 * y[j] = sum_k w[rows_n[j], k] x[rows_m[j], k] (and a[j] likewise).
 * Used to check single elements of full-size problems.                     */
void qmo_qmm_sample(const uint32_t *w, const uint16_t *scales, const uint16_t *mins,
                    const uint16_t *x, int64_t k, int bits, int group,
                    const int64_t *rows_m, const int64_t *rows_n, int64_t count,
                    double *y, double *a)
{
    int64_t wpr = words_per_row(k, bits);
    int64_t gpr = k / group;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 4)
#endif
    for (int64_t j = 0; j < count; ++j) {
        int64_t r = rows_n[j];
        const uint32_t *row = w + r * wpr;
        const uint16_t *xr = x + rows_m[j] * k;
        double acc = 0.0, acc_abs = 0.0;
        for (int64_t c = 0; c < k; ++c) {
            double s = qmo_fp16_to_double(scales[r * gpr + c / group]);
            double m = qmo_fp16_to_double(mins[r * gpr + c / group]);
            double p = (s * (double)row_code(row, c, bits) + m) * qmo_fp16_to_double(xr[c]);
            acc += p;
            acc_abs += fabs(p);
        }
        y[j] = acc;
        if (a)
            a[j] = acc_abs;
    }
}

/* Mixture-of-experts projection over expert-sorted rows.
 * Experts are stacked: expert e's packed rows start at w + e*N*K*b/32, its
 * scales and mins at e*N*(K/group).  Rows p in [offsets[e], offsets[e+1])
 * belong to expert e; row p reads activation row x_rows[p] (or p when
 * x_rows is NULL) and writes y[p*N .. p*N + N).                            */
void qmo_moe(const uint32_t *w, const uint16_t *scales, const uint16_t *mins,
             const uint16_t *x, const int32_t *x_rows, const int32_t *offsets,
             int64_t n_experts, int64_t n, int64_t k, int bits, int group,
             double *y, double *a)
{
    int64_t w_expert = n * words_per_row(k, bits);
    int64_t g_expert = n * (k / group);
    for (int64_t e = 0; e < n_experts; ++e) {
        int64_t p0 = offsets[e], p1 = offsets[e + 1];
        if (p1 <= p0)
            continue;
        const int32_t *rows = x_rows ? x_rows + p0 : NULL;
        /* Without an index, row p of x is activation p: point x at row p0. */
        const uint16_t *xb = x_rows ? x : x + p0 * k;
        qmm_rows(w + e * w_expert, scales + e * g_expert, mins + e * g_expert,
                 xb, rows, p1 - p0, n, k, bits, group,
                 y + p0 * n, a ? a + p0 * n : NULL, n);
    }
}

/* Threads the OpenMP runtime would use (1 without OpenMP). */
int qmo_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void qmo_set_threads(int t)
{
#ifdef _OPENMP
    if (t > 0)
        omp_set_num_threads(t);
#else
    (void)t;
#endif
}
