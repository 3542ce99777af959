/*
 * nvfp4_oracle.c -- plain CPU oracle for NVFP4 block-scaled GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU product path
 * never calls it, and the two share no code, headers, tables or constants.
 *
 * What is computed (kernelbot pages nvfp4-group-gemm-498453 and
 * nvfp4-gemm-125598: the `custom_kernel` docstrings and the MMA loop, which
 * state C = A * SFA * B * SFB with one scale per 16 consecutive K elements):
 *
 *   a_k      = E2M1(nibble of A[m] at k) * E4M3(SFA[m][k/16])
 *   b_k      = E2M1(nibble of B[n] at k) * E4M3(SFB[n][k/16])
 *   C64[m,n] = sum_{k<K} a_k * b_k                 (fp64, k ascending)
 *   bound    = sum_{k<K} |a_k * b_k|               (fp64, for the tolerance)
 *   C16[m,n] = binary16 round-to-nearest-even of C64 (overflow -> +-inf)
 *
 * Readings taken where the pages are silent (each is listed in the design
 * notes): low nibble of a byte holds the even k; the scale type is the OCP
 * e4m3 "fn" variant (bias 7, max 448, no inf, NaN = S.1111.111); e2m1 is the
 * OCP MX fp4 format; rounding to fp16 is round-to-nearest-even as the raw-CUDA
 * page's epilogue (`__floats2half2_rn`) does.
 *
 * Layouts (all row-major, contiguous):
 *   A   [M][K/2]  bytes, two e2m1 codes per byte, low nibble = even k
 *   SFA [M][K/16] e4m3fn codes
 *   B   [N][K/2], SFB [N][K/16] likewise
 *   C16 [M][N] binary16 bit patterns; C64 and bound [M][N] doubles
 *
 * Parallelism: OpenMP over output rows only; every output is one plain
 * ascending-k loop, so the result does not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

/* e2m1 (OCP MX fp4): 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit.
 * Exponent field 0 is subnormal: value = m * 2^-1.  Otherwise
 * value = 2^(e-1) * (1 + m/2).  There is no inf or NaN. */
double oracle_e2m1_value(int code)
{
    int s = (code >> 3) & 1;
    int e = (code >> 1) & 3;
    int m = code & 1;
    double mag;
    if (e == 0)
        mag = m * 0.5;
    else
        mag = ldexp(1.0 + m / 2.0, e - 1);
    return s ? -mag : mag;
}

/* e4m3fn (OCP fp8 E4M3): 1 sign bit, 4 exponent bits (bias 7), 3 mantissa
 * bits.  Exponent field 0 is subnormal: value = (m/8) * 2^-6.  S.1111.111 is
 * NaN; there is no inf, so S.1111.110 = 448 is the largest finite value. */
double oracle_e4m3_value(int code)
{
    int s = (code >> 7) & 1;
    int e = (code >> 3) & 15;
    int m = code & 7;
    double mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = ldexp(m / 8.0, -6);
    else
        mag = ldexp(1.0 + m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* Round a non-negative double q to an integer, ties to even.  q < 2^52, so
 * the fraction q - floor(q) is exact. */
static double round_half_even(double q)
{
    double f = floor(q);
    double d = q - f;
    if (d > 0.5)
        return f + 1.0;
    if (d < 0.5)
        return f;
    return (fmod(f, 2.0) == 0.0) ? f : f + 1.0;
}

/* IEEE 754 binary16 encoding of x, round to nearest, ties to even.
 * binary16: 1 sign, 5 exponent bits (bias 15), 10 fraction bits; normals
 * span [2^-14, 65504]; subnormals are multiples of 2^-24; a magnitude that
 * rounds above 65504 (that is, >= 65520) becomes inf. NaN maps to a quiet NaN. */
uint16_t oracle_fp16_rne(double x)
{
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    double ax = fabs(x);
    if (isnan(x))
        return (uint16_t)(sign | 0x7E00u);
    if (ax >= 65520.0)
        return (uint16_t)(sign | 0x7C00u);
    if (ax < ldexp(1.0, -14)) {
        /* subnormal range: integer multiple of 2^-24 (q == 1024 is the
         * smallest normal, whose encoding 0x0400 is exactly q) */
        double q = round_half_even(ldexp(ax, 24));
        return (uint16_t)(sign | (uint16_t)q);
    }
    int e;
    frexp(ax, &e);          /* ax = f * 2^e with f in [0.5, 1) */
    e -= 1;                 /* now ax = g * 2^e with g in [1, 2) */
    double q = round_half_even(ldexp(ax, 10 - e)); /* 11-bit significand */
    if (q >= 2048.0) {      /* carried into the next binade */
        q /= 2.0;
        e += 1;
    }
    if (e > 15)             /* unreachable below 65520, kept for clarity */
        return (uint16_t)(sign | 0x7C00u);
    return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)(q - 1024.0));
}

/* Element k of row r of a packed operand X with row length K (in elements),
 * scaled by its block scale from SF. */
static double scaled_element(const uint8_t *X, const uint8_t *SF, long r, long k, long K)
{
    uint8_t byte = X[r * (K / 2) + k / 2];
    int code = (k % 2 == 0) ? (byte & 0xF) : (byte >> 4);
    return oracle_e2m1_value(code) * oracle_e4m3_value(SF[r * (K / 16) + k / 16]);
}

/* Decode R rows of a packed operand into doubles: out[r][k] = element * scale. */
void oracle_decode_rows(const uint8_t *X, const uint8_t *SF, long R, long K, double *out)
{
#pragma omp parallel for schedule(static)
    for (long r = 0; r < R; ++r)
        for (long k = 0; k < K; ++k)
            out[r * K + k] = scaled_element(X, SF, r, k, K);
}

/* Full product.  Any of C16, C64, bound may be NULL. K must be a multiple
 * of 16 (one scale per 16 elements). */
int oracle_gemm(const uint8_t *A, const uint8_t *SFA, const uint8_t *B, const uint8_t *SFB,
                long M, long N, long K, uint16_t *C16, double *C64, double *bound)
{
    if (M < 0 || N < 0 || K < 0 || K % 16 != 0)
        return 1;
    double *Ad = (double *)malloc(sizeof(double) * (size_t)(M * K > 0 ? M * K : 1));
    double *Bd = (double *)malloc(sizeof(double) * (size_t)(N * K > 0 ? N * K : 1));
    if (!Ad || !Bd) {
        free(Ad);
        free(Bd);
        return 2;
    }
    oracle_decode_rows(A, SFA, M, K, Ad);
    oracle_decode_rows(B, SFB, N, K, Bd);
#pragma omp parallel for schedule(dynamic, 1)
    for (long m = 0; m < M; ++m) {
        for (long n = 0; n < N; ++n) {
            double acc = 0.0, mag = 0.0;
            for (long k = 0; k < K; ++k) {
                double p = Ad[m * K + k] * Bd[n * K + k];
                acc += p;
                mag += fabs(p);
            }
            if (C64)
                C64[m * N + n] = acc;
            if (bound)
                bound[m * N + n] = mag;
            if (C16)
                C16[m * N + n] = oracle_fp16_rne(acc);
        }
    }
    free(Ad);
    free(Bd);
    return 0;
}

/* Selected outputs only, each computed on its own straight from the packed
 * codes: entry i is (rows[i], cols[i]).  Used to check a few outputs of a
 * product too large to compute whole. */
int oracle_gemm_entries(const uint8_t *A, const uint8_t *SFA, const uint8_t *B, const uint8_t *SFB,
                        long M, long N, long K, long count, const long *rows, const long *cols,
                        uint16_t *C16, double *C64, double *bound)
{
    if (K % 16 != 0)
        return 1;
    for (long i = 0; i < count; ++i)
        if (rows[i] < 0 || rows[i] >= M || cols[i] < 0 || cols[i] >= N)
            return 1;
#pragma omp parallel for schedule(dynamic, 4)
    for (long i = 0; i < count; ++i) {
        double acc = 0.0, mag = 0.0;
        for (long k = 0; k < K; ++k) {
            double p = scaled_element(A, SFA, rows[i], k, K) * scaled_element(B, SFB, cols[i], k, K);
            acc += p;
            mag += fabs(p);
        }
        if (C64)
            C64[i] = acc;
        if (bound)
            bound[i] = mag;
        if (C16)
            C16[i] = oracle_fp16_rne(acc);
    }
    return 0;
}

/* Number of OpenMP threads a parallel region uses (reported with timings). */
int oracle_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            extern int omp_get_num_threads(void);
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}
