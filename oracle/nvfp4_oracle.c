/*
 * nvfp4_oracle.c -- CPU oracle for the NVFP4 grouped GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: it exists so that tests, the smoke check and the benchmark's
 * CPU-baseline leg can compare the GPU result with a plain, slow, obviously
 * correct computation.  It shares no code, header or table with the HIP
 * library.
 *
 * What it computes (pages: "nvfp4 group gemm" submissions 474067, 482269 and
 * 496386 on kernelindex.com; the header comment of submission 474067 states
 * FP4 E2M1 operands, E4M3FN scale factors and FP16 output; its MMA helper
 * issues the block-scaled MMA of kind mxf4nvf4 with one scale per 16
 * elements ("block16"); its epilogue converts the fp32 accumulator to fp16
 * with round-to-nearest-even):
 *
 *   for every group g, m < M_g, n < N_g:
 *     C_g[m][n] = fp16_rne( sum_{k < K_g}  E2M1(A_g[m][k]) * E4M3FN(SFA_g[m][k/16])
 *                                       * E2M1(B_g[n][k]) * E4M3FN(SFB_g[n][k/16]) )
 *
 * The sum is taken in fp64, in plain k order, starting from +0.0, and rounded
 * once to fp16.  Every product of two decoded operands is an exact multiple
 * of 2**-20 (E2M1 quantum 2**-1 times E4M3FN quantum 2**-9, squared), so the
 * fp64 sum is exact whenever K * max|term| < 2**33; for the benchmark
 * workloads it is, and the oracle then returns the correctly rounded fp16 of
 * the exact real sum.
 *
 * Layouts (plain reading of the pages plus the benchmark spec):
 *   A_g  [M][K/2]  bytes, row-major; element k in byte k/2, even k in the low
 *                  nibble, odd k in the high nibble.
 *   B_g  [N][K/2]  bytes, same packing (C = A * B^T, both operands K-major,
 *                  as in the pages' tensor-map view of A and B).
 *   SFA  [M][K/16] E4M3FN bytes, row-major.   SFB [N][K/16] likewise.
 *   C_g  [M][N]    fp16 bits, row-major.
 *
 * Number formats (OCP 8-bit floating point spec for E4M3FN; OCP Microscaling
 * Formats spec v1.0 for E2M1):
 *   E2M1:   s | e(2) | m(1), exponent bias 1, subnormal when e == 0,
 *           no inf or NaN.  Magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.
 *   E4M3FN: s | E(4) | M(3), exponent bias 7, subnormal when E == 0,
 *           no infinities, NaN only for E == 15 && M == 7 (0x7F, 0xFF).
 *   fp16:   IEEE binary16.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- format decoding (lookup tables filled from the format definitions) ---- */

static double g_e2m1[16];
static double g_e4m3[256];
static int g_tables_ready = 0;

static double e2m1_from_fields(unsigned code)
{
    unsigned s = (code >> 3) & 1u, e = (code >> 1) & 3u, m = code & 1u;
    double mag = (e == 0) ? 0.5 * (double)m                       /* subnormal: m * 2^-1 */
                          : ldexp(1.0 + 0.5 * (double)m, (int)e - 1); /* 2^(e-1) * (1 + m/2) */
    return s ? -mag : mag;
}

static double e4m3fn_from_fields(unsigned byte)
{
    unsigned s = (byte >> 7) & 1u, E = (byte >> 3) & 15u, M = byte & 7u;
    double mag;
    if (E == 15u && M == 7u)
        return NAN;
    if (E == 0u)
        mag = ldexp((double)M / 8.0, -6);                  /* subnormal: (M/8) * 2^-6 */
    else
        mag = ldexp(1.0 + (double)M / 8.0, (int)E - 7);    /* (1 + M/8) * 2^(E-7) */
    return s ? -mag : mag;
}

static void build_tables(void)
{
    if (g_tables_ready)
        return;
    for (unsigned c = 0; c < 16; ++c)
        g_e2m1[c] = e2m1_from_fields(c);
    for (unsigned b = 0; b < 256; ++b)
        g_e4m3[b] = e4m3fn_from_fields(b);
    g_tables_ready = 1;
}

double oracle_e2m1_value(unsigned code)
{
    build_tables();
    return g_e2m1[code & 15u];
}

double oracle_e4m3fn_value(unsigned byte)
{
    build_tables();
    return g_e4m3[byte & 255u];
}

/* ---- one rounding: fp64 -> IEEE binary16, round to nearest, ties to even ---- */

uint16_t oracle_fp16_rne(double x)
{
    uint16_t sign;
    double ax, q, fl, frac;
    int e, ulp_exp;
    uint64_t r;

    if (isnan(x))
        return 0x7E00u;
    sign = signbit(x) ? 0x8000u : 0u;
    ax = fabs(x);
    if (ax == 0.0)
        return sign;
    /* 65520 is halfway between the largest finite fp16 (65504) and 2^16; the
       tie goes to the even neighbour 2^16, which overflows to infinity. */
    if (ax >= 65520.0)
        return (uint16_t)(sign | 0x7C00u);
    frexp(ax, &e);                       /* ax = f * 2^e, f in [0.5, 1) */
    /* binade exponent is e-1; normal fp16 has 10 fraction bits, subnormal
       fp16 has a fixed quantum of 2^-24 */
    ulp_exp = (e - 1 >= -14) ? (e - 1 - 10) : -24;
    q = ldexp(ax, -ulp_exp);             /* value in units of the fp16 quantum (exact) */
    fl = floor(q);
    frac = q - fl;
    r = (uint64_t)fl;
    if (frac > 0.5 || (frac == 0.5 && (r & 1u)))
        r += 1u;
    if (ulp_exp == -24)                  /* subnormal (r == 1024 becomes the smallest normal) */
        return (uint16_t)(sign | (uint16_t)r);
    /* normal: r in [1024, 2048]; a carry to 2048 bumps the exponent field */
    return (uint16_t)(sign | (uint16_t)((((uint64_t)(e - 1 + 15)) << 10) + (r - 1024u)));
}

/* ---- element access ---- */

static unsigned nibble_at(const uint8_t *row, int64_t k)
{
    uint8_t byte = row[k >> 1];
    return (k & 1) ? (unsigned)(byte >> 4) : (unsigned)(byte & 15u);
}

/* decoded operand value x = code * scale, exact in fp64 */
static double operand_value(const uint8_t *codes_row, const uint8_t *scale_row, int64_t k)
{
    return g_e2m1[nibble_at(codes_row, k)] * g_e4m3[scale_row[k >> 4]];
}

/* ---- one output element of one group, straight from the definition ---- */

double oracle_dot(const uint8_t *a, const uint8_t *sfa, const uint8_t *b, const uint8_t *sfb,
                  int64_t k_len, int64_t m, int64_t n)
{
    const uint8_t *a_row = a + m * (k_len / 2), *sa_row = sfa + m * (k_len / 16);
    const uint8_t *b_row = b + n * (k_len / 2), *sb_row = sfb + n * (k_len / 16);
    double acc = +0.0;
    build_tables();
    for (int64_t k = 0; k < k_len; ++k)
        acc += operand_value(a_row, sa_row, k) * operand_value(b_row, sb_row, k);
    return acc;
}

/*
 * Full GEMM of one group.  c16 (M*N fp16 bits) and/or c64 (M*N doubles, the
 * unrounded sums) may be NULL.  B's rows are decoded once into an fp64 matrix
 * (each entry is the exact product code*scale of the definition); the sum over
 * k is still the plain k-ordered loop.  nthreads <= 0 uses the OpenMP default.
 * Returns 0, or -1 if memory for the decoded B could not be obtained.
 */
int oracle_gemm_group(const uint8_t *a, const uint8_t *sfa, const uint8_t *b, const uint8_t *sfb,
                      int64_t m_len, int64_t n_len, int64_t k_len,
                      uint16_t *c16, double *c64, int nthreads)
{
    double *bdec;
    int failed = 0;
    build_tables();
    if (m_len <= 0 || n_len <= 0)
        return 0;
    if (k_len <= 0) {
        for (int64_t i = 0; i < m_len * n_len; ++i) {
            if (c16) c16[i] = 0;
            if (c64) c64[i] = 0.0;
        }
        return 0;
    }
    bdec = (double *)malloc((size_t)n_len * (size_t)k_len * sizeof(double));
    if (!bdec)
        return -1;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel
    {
        double *arow = (double *)malloc((size_t)k_len * sizeof(double));
#pragma omp for schedule(static)
        for (int64_t n = 0; n < n_len; ++n)
            for (int64_t k = 0; k < k_len; ++k)
                bdec[n * k_len + k] = operand_value(b + n * (k_len / 2), sfb + n * (k_len / 16), k);
#pragma omp for schedule(dynamic, 1)
        for (int64_t m = 0; m < m_len; ++m) {
            if (!arow) {
#pragma omp atomic write
                failed = 1;
                continue;
            }
            for (int64_t k = 0; k < k_len; ++k)
                arow[k] = operand_value(a + m * (k_len / 2), sfa + m * (k_len / 16), k);
            for (int64_t n = 0; n < n_len; ++n) {
                const double *brow = bdec + n * k_len;
                double acc = +0.0;
                for (int64_t k = 0; k < k_len; ++k)
                    acc += arow[k] * brow[k];
                if (c16) c16[m * n_len + n] = oracle_fp16_rne(acc);
                if (c64) c64[m * n_len + n] = acc;
            }
        }
        free(arow);
    }
    free(bdec);
    return failed ? -1 : 0;
}

/*
 * Sampled outputs of one group: for i < count, element (rows[i], cols[i]).
 * Used at full benchmark sizes, where only a sample is checked.
 */
void oracle_gemm_entries(const uint8_t *a, const uint8_t *sfa, const uint8_t *b, const uint8_t *sfb,
                         int64_t k_len, const int32_t *rows, const int32_t *cols, int64_t count,
                         uint16_t *out16, double *out64, int nthreads)
{
    build_tables();
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        double v = oracle_dot(a, sfa, b, sfb, k_len, rows[i], cols[i]);
        if (out16) out16[i] = oracle_fp16_rne(v);
        if (out64) out64[i] = v;
    }
}

/* threads an OpenMP region would use (for reporting the CPU baseline) */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
