/*
 * gemm_oracle.c -- CPU reference for C = alpha*A@B + beta*C.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link
 * or call this file.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark use it.  It shares no code, header, table or
 * constant with the GPU library.
 *
 * What it computes (phobos docs, page "gemm, f32", opening paragraph and
 * section "The epilogue"): every element of C becomes alpha times the dot
 * product of row i of A with column j of B, plus beta times the old C[i,j].
 * In the f16r mode (phobos docs, page "gemm on tensor cores", section "What
 * changes") the operands A and B are rounded to binary16 first and the
 * products are summed at higher precision; alpha, beta and C stay f32.
 *
 * Precision: every operand is widened to double.  A product of two f32
 * values (24+24 significant bits) or two f16 values (11+11) is exact in
 * double, so the only rounding is in the double additions, far below the
 * f32 or f16r tolerances.
 *
 * Readings of points the pages leave open:
 *   - rounding to f16 is IEEE 754 roundTiesToEven, subnormals kept, values
 *     at or above 65520 in magnitude become infinities, NaN stays NaN;
 *   - beta == 0 means C is not read (so NaN in C does not leak);
 *   - alpha == 0 or K == 0 means the product term is 0 and A, B are not read;
 *   - matrices are row-major with a leading dimension >= the row length.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC (no -ffast-math: the summation
 * must be plain IEEE double).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_MODE_F32 0
#define ORACLE_MODE_F16R 1

/* ------------------------------------------------------------------------ */
/* IEEE 754 binary32 -> binary16, roundTiesToEven, written from the format   */
/* definitions: binary16 has 1 sign bit, 5 exponent bits (bias 15) and 10    */
/* fraction bits; its largest finite value is 65504 and its smallest         */
/* subnormal is 2^-24.                                                       */
/* ------------------------------------------------------------------------ */
uint16_t oracle_rn_f16_bits(float x)
{
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    uint32_t bexp = (u >> 23) & 0xffu;
    uint32_t frac = u & 0x7fffffu;

    if (bexp == 0xffu) /* infinity or NaN */
        return (uint16_t)(sign | 0x7c00u | (frac ? 0x0200u : 0u));
    if (bexp == 0u) /* zero or f32 subnormal: below 2^-126, rounds to 0 */
        return sign;

    int e = (int)bexp - 127;            /* |x| = sig * 2^(e-23) */
    uint32_t sig = (1u << 23) | frac;   /* 24-bit integer significand */

    if (e > 15) /* |x| >= 2^16 > 65520: overflow */
        return (uint16_t)(sign | 0x7c00u);

    if (e >= -14) { /* result is normal (or overflows after rounding) */
        uint32_t keep = sig >> 13;      /* 11 bits incl. the implicit one */
        uint32_t rem = sig & 0x1fffu;
        if (rem > 0x1000u || (rem == 0x1000u && (keep & 1u)))
            keep += 1u;
        uint32_t hexp = (uint32_t)(e + 15);
        if (keep == 0x800u) { keep = 0x400u; hexp += 1u; }
        if (hexp >= 31u)
            return (uint16_t)(sign | 0x7c00u);
        return (uint16_t)(sign | (hexp << 10) | (keep & 0x3ffu));
    }

    /* subnormal range: result = m * 2^-24 with m = sig * 2^(e+1) */
    int shift = -(e + 1);               /* >= 14 */
    if (shift > 24) /* |x| < 2^-25: below half the smallest subnormal */
        return sign;
    uint32_t keep = sig >> shift;
    uint32_t rem = sig & ((1u << shift) - 1u);
    uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (keep & 1u)))
        keep += 1u;                     /* may carry into the smallest normal */
    return (uint16_t)(sign | keep);
}

/* binary16 bits -> double, exact (every binary16 value is a double). */
double oracle_f16_bits_to_double(uint16_t h)
{
    int s = (h >> 15) & 1;
    int ex = (h >> 10) & 0x1f;
    int fr = h & 0x3ff;
    double v;
    if (ex == 0x1f)
        v = fr ? NAN : INFINITY;
    else if (ex == 0)
        v = ldexp((double)fr, -24);
    else
        v = ldexp((double)(0x400 | fr), ex - 25);
    return s ? -v : v;
}

/* The operand as the method multiplies it: f32 as is, or rounded to f16. */
static double operand(int mode, float x)
{
    if (mode == ORACLE_MODE_F16R)
        return oracle_f16_bits_to_double(oracle_rn_f16_bits(x));
    return (double)x;
}

void oracle_rn_f16_array(const float* x, uint16_t* out, int64_t n)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_rn_f16_bits(x[i]);
}

/* r(X): the operand matrix widened to double, dense (ld = cols). */
static double* rounded_copy(int mode, const float* X, int64_t rows, int64_t cols, int64_t ld)
{
    double* R = (double*)malloc((size_t)(rows * cols > 0 ? rows * cols : 1) * sizeof(double));
    if (!R)
        return NULL;
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            R[r * cols + c] = operand(mode, X[r * ld + c]);
    return R;
}

/*
 * One output row: acc[j] = sum_k r(A[i,k]) r(B[k,j]) and
 * mag[j] = sum_k |r(A[i,k])| |r(B[k,j])|, k ascending.
 */
static void row_products(const double* rA, const double* rB, int64_t i, int64_t N, int64_t K,
                         double* acc, double* mag)
{
    for (int64_t j = 0; j < N; ++j) { acc[j] = 0.0; mag[j] = 0.0; }
    for (int64_t k = 0; k < K; ++k) {
        double a = rA[i * K + k];
        const double* b = rB + k * N;
        for (int64_t j = 0; j < N; ++j) {
            acc[j] += a * b[j];
            mag[j] += fabs(a) * fabs(b[j]);
        }
    }
}

/*
 * Full reference.  Cref[i*N+j] = alpha*sum + beta*C0 (double, not rounded to
 * f32) and W[i*N+j] = |alpha|*sum|a||b| + |beta||C0|, the scale the parity
 * bound is relative to.  Returns 0, or -1 on allocation failure.
 */
int oracle_gemm(int mode, int64_t M, int64_t N, int64_t K, float alpha,
                const float* A, int64_t lda, const float* B, int64_t ldb,
                float beta, const float* C0, int64_t ldc, double* Cref, double* W)
{
    if (M <= 0 || N <= 0)
        return 0;
    int product = (K > 0 && alpha != 0.0f);
    double* rA = NULL;
    double* rB = NULL;
    if (product) {
        rA = rounded_copy(mode, A, M, K, lda);
        rB = rounded_copy(mode, B, K, N, ldb);
        if (!rA || !rB) { free(rA); free(rB); return -1; }
    }
    int fail = 0;
    #pragma omp parallel
    {
        double* acc = (double*)calloc((size_t)N, sizeof(double));
        double* mag = (double*)calloc((size_t)N, sizeof(double));
        if (!acc || !mag) {
            #pragma omp atomic write
            fail = 1;
        } else {
            #pragma omp for schedule(dynamic, 4)
            for (int64_t i = 0; i < M; ++i) {
                if (product)
                    row_products(rA, rB, i, N, K, acc, mag);
                for (int64_t j = 0; j < N; ++j) {
                    double term = product ? (double)alpha * acc[j] : 0.0;
                    double w = product ? fabs((double)alpha) * mag[j] : 0.0;
                    if (beta != 0.0f) {
                        double c = (double)C0[i * ldc + j];
                        term += (double)beta * c;
                        w += fabs((double)beta) * fabs(c);
                    }
                    Cref[i * N + j] = term;
                    W[i * N + j] = w;
                }
            }
        }
        free(acc);
        free(mag);
    }
    free(rA);
    free(rB);
    return fail ? -1 : 0;
}

/*
 * Sampled entries: for each (rows[s], cols[s]) the same sum as oracle_gemm,
 * computed on its own (k ascending), for checks at sizes where the full
 * product is too slow on the CPU.
 */
void oracle_gemm_entries(int mode, int64_t K, float alpha,
                         const float* A, int64_t lda, const float* B, int64_t ldb,
                         float beta, const float* C0, int64_t ldc,
                         const int64_t* rows, const int64_t* cols, int64_t n,
                         double* ref, double* W)
{
    int product = (K > 0 && alpha != 0.0f);
    #pragma omp parallel for schedule(dynamic, 16)
    for (int64_t s = 0; s < n; ++s) {
        int64_t i = rows[s], j = cols[s];
        double acc = 0.0, mag = 0.0;
        if (product) {
            for (int64_t k = 0; k < K; ++k) {
                double a = operand(mode, A[i * lda + k]);
                double b = operand(mode, B[k * ldb + j]);
                acc += a * b;
                mag += fabs(a) * fabs(b);
            }
        }
        double term = product ? (double)alpha * acc : 0.0;
        double w = product ? fabs((double)alpha) * mag : 0.0;
        if (beta != 0.0f) {
            double c = (double)C0[i * ldc + j];
            term += (double)beta * c;
            w += fabs((double)beta) * fabs(c);
        }
        ref[s] = term;
        W[s] = w;
    }
}

/*
 * Streaming comparison of a result Cgot (row-major, ld ldg) with the
 * reference, row by row, without storing the whole reference.
 * stats[0] = max |err|/W (inf if an element with W == 0 is not exact),
 * stats[1] = number of elements with NOT(|err| <= tol*W) (NaN fails),
 * stats[2] = max |err|, stats[3] = max |ref|,
 * stats[4] = sum err^2,  stats[5] = sum ref^2.
 * rows_lo..rows_hi restricts the check to a band of rows.
 * Returns 0, or -1 on allocation failure.
 */
int oracle_check(int mode, int64_t M, int64_t N, int64_t K, float alpha,
                 const float* A, int64_t lda, const float* B, int64_t ldb,
                 float beta, const float* C0, int64_t ldc,
                 const float* Cgot, int64_t ldg, double tol,
                 int64_t rows_lo, int64_t rows_hi, double* stats)
{
    for (int s = 0; s < 6; ++s) stats[s] = 0.0;
    if (M <= 0 || N <= 0)
        return 0;
    if (rows_lo < 0) rows_lo = 0;
    if (rows_hi > M) rows_hi = M;
    int product = (K > 0 && alpha != 0.0f);
    double* rA = NULL;
    double* rB = NULL;
    if (product) {
        rA = rounded_copy(mode, A, M, K, lda);
        rB = rounded_copy(mode, B, K, N, ldb);
        if (!rA || !rB) { free(rA); free(rB); return -1; }
    }
    double max_ratio = 0.0, n_fail = 0.0, max_err = 0.0, max_ref = 0.0, se = 0.0, sr = 0.0;
    int fail = 0;
    #pragma omp parallel reduction(max : max_ratio, max_err, max_ref) reduction(+ : n_fail, se, sr)
    {
        double* acc = (double*)calloc((size_t)N, sizeof(double));
        double* mag = (double*)calloc((size_t)N, sizeof(double));
        if (!acc || !mag) {
            #pragma omp atomic write
            fail = 1;
        } else {
            #pragma omp for schedule(dynamic, 4)
            for (int64_t i = rows_lo; i < rows_hi; ++i) {
                if (product)
                    row_products(rA, rB, i, N, K, acc, mag);
                for (int64_t j = 0; j < N; ++j) {
                    double term = product ? (double)alpha * acc[j] : 0.0;
                    double w = product ? fabs((double)alpha) * mag[j] : 0.0;
                    if (beta != 0.0f) {
                        double c = (double)C0[i * ldc + j];
                        term += (double)beta * c;
                        w += fabs((double)beta) * fabs(c);
                    }
                    double got = (double)Cgot[i * ldg + j];
                    double err = fabs(got - term);
                    if (!(err <= tol * w))
                        n_fail += 1.0;
                    double ratio;
                    if (err != err)
                        ratio = INFINITY;
                    else if (w > 0.0)
                        ratio = err / w;
                    else
                        ratio = (err == 0.0) ? 0.0 : INFINITY;
                    if (ratio > max_ratio) max_ratio = ratio;
                    if (err > max_err || err != err) max_err = (err != err) ? INFINITY : err;
                    if (fabs(term) > max_ref) max_ref = fabs(term);
                    se += (err != err) ? INFINITY : err * err;
                    sr += term * term;
                }
            }
        }
        free(acc);
        free(mag);
    }
    free(rA);
    free(rB);
    stats[0] = max_ratio; stats[1] = n_fail; stats[2] = max_err;
    stats[3] = max_ref;   stats[4] = se;     stats[5] = sr;
    return fail ? -1 : 0;
}
