/*
 * Oracle for the software-pipelined tiled GEMM and the streaming elementwise
 * pipeline.  TEST INFRASTRUCTURE ONLY: nothing on the product path links,
 * loads or calls this file; only the tests, the package smoke check and the
 * CPU-baseline leg of the benchmark do.  It shares no code, header, table or
 * helper with the HIP library.
 *
 * Everything here is the plain definition of what the pipelined kernels
 * compute, written as slow, obviously correct loops:
 *
 *  - GEMM.  The Pallas "Quickstart: GPU" page (section "Pipelining: a matmul
 *    kernel") and its Chinese rewrite (section "Hopper 上的矩阵乘法内核")
 *    compute C = A @ B for a of shape (m, k) and b of shape (k, n), fp16
 *    inputs, an fp32 accumulator and an fp16 output obtained with
 *    astype(float16).  Tiling, multi-buffering and the accumulation order
 *    change nothing but rounding, so the oracle is the mathematical product:
 *    every fp16*fp16 product is exact in binary64, the products are summed in
 *    ascending k in binary64, and the sum is rounded ONCE to binary16 with
 *    round-to-nearest-even.
 *  - Streaming add.  The software-pipelining guide (lmnt.cn), section 6
 *    "pipelined elementwise kernel", adds two f32 arrays block by block and
 *    checks the result for exact equality with x + y; section 4 adds 1 to
 *    every element.  The oracle is one IEEE-754 binary32 addition per element.
 *  - fill and iota.  Quickstart "Your first kernel" writes 42.0 into 128 f32
 *    elements; "Parallel work with a grid" writes 0.0, 1.0, ..., 1023.0.
 *  - Reduction along the last grid axis.  The guide, section 7.2
 *    "reductions and accumulation", sums an (R, M, N) f32 array over its
 *    first array axis by making that axis the last (sequential) grid axis:
 *    the output block is zeroed at the first step and x[i] is added to it
 *    at step i, in f32.  The oracle is that loop: start from +0.0f and add
 *    x[0], x[1], ..., x[R-1] in this order, one binary32 addition each.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC (no fast-math, so
 * the x86-64 SSE2 arithmetic is IEEE binary32/binary64 with RNE and no
 * flush-to-zero).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- binary16 <-> binary64 ------------------------------------------------ */

/* Decode one IEEE binary16 bit pattern to the binary64 value it denotes
 * (exact: every binary16 value is representable in binary64). */
double oracle_f64_from_f16(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int m = h & 0x3FF;
    double v;
    if (e == 0) {
        v = ldexp((double)m, -24); /* zero or subnormal: m * 2^-24 */
    } else if (e == 31) {
        v = (m == 0) ? INFINITY : NAN;
    } else {
        v = ldexp((double)(1024 + m), e - 25); /* (1.m) * 2^(e-15) */
    }
    return sign ? -v : v;
}

/* Round a binary64 value to the nearest binary16, ties to even, in one step
 * (no intermediate binary32, so no double rounding).  Magnitudes from 65520
 * up become infinity; binary16 subnormals are produced, never flushed. */
uint16_t oracle_f16_from_f64(double x)
{
    uint64_t b;
    memcpy(&b, &x, sizeof b);
    uint16_t sign = (uint16_t)((b >> 48) & 0x8000u);
    uint64_t mag = b & 0x7FFFFFFFFFFFFFFFull;
    int biased = (int)(mag >> 52);
    uint64_t frac = mag & 0xFFFFFFFFFFFFFull;

    if (biased == 0x7FF) {
        if (frac == 0)
            return sign | 0x7C00u; /* infinity */
        uint16_t payload = (uint16_t)(frac >> 42);
        return sign | 0x7C00u | (payload ? payload : 1u) | 0x200u; /* quiet NaN */
    }
    if (biased == 0)
        return sign; /* zero or binary64 subnormal: far below 2^-25 */

    int E = biased - 1023;              /* unbiased exponent */
    uint64_t m = frac | (1ull << 52);   /* 53-bit significand, value m*2^(E-52) */

    if (E >= -14) {
        /* binary16 normal range: keep 11 significant bits. */
        uint64_t q = m >> 42;
        uint64_t rem = m & ((1ull << 42) - 1);
        uint64_t half = 1ull << 41;
        if (rem > half || (rem == half && (q & 1)))
            q += 1;
        if (q == 2048) { /* carried into the next binade */
            q = 1024;
            E += 1;
        }
        if (E > 15)
            return sign | 0x7C00u;
        return sign | (uint16_t)(((E + 15) << 10) | (q & 0x3FF));
    }

    /* binary16 subnormal range: value in units of 2^-24 is m * 2^(E-28). */
    int s = 28 - E; /* > 42 */
    if (s >= 64)
        return sign; /* below a quarter of 2^-24: rounds to zero */
    uint64_t q = m >> s;
    uint64_t rem = m & ((1ull << s) - 1);
    uint64_t half = 1ull << (s - 1);
    if (rem > half || (rem == half && (q & 1)))
        q += 1;
    /* q == 1024 encodes the smallest normal, which is the right bit pattern. */
    return sign | (uint16_t)q;
}

void oracle_f16_from_f64_array(const double* x, uint16_t* h, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        h[i] = oracle_f16_from_f64(x[i]);
}

void oracle_f64_from_f16_array(const uint16_t* h, double* x, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        x[i] = oracle_f64_from_f16(h[i]);
}

/* ---- GEMM ------------------------------------------------------------------ */

static double g_dec[65536];
static int g_dec_ready = 0;

static void init_decode_table(void)
{
    if (g_dec_ready)
        return;
    for (int h = 0; h < 65536; ++h)
        g_dec[h] = oracle_f64_from_f16((uint16_t)h);
    g_dec_ready = 1;
}

/* One output element: C[i,j] = sum over ascending k of A[i,k]*B[k,j] in
 * binary64, then one rounding to binary16.  A is row-major [M,K], B is
 * row-major [K,N]. */
static void one_element(const uint16_t* A, const uint16_t* B, int64_t N, int64_t K,
                        int64_t i, int64_t j, uint16_t* c, double* s_out)
{
    double s = 0.0;
    for (int64_t k = 0; k < K; ++k)
        s += g_dec[A[i * K + k]] * g_dec[B[k * N + j]];
    *c = oracle_f16_from_f64(s);
    if (s_out)
        *s_out = s;
}

int oracle_threads(void)
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

/* Full product.  C is row-major [M,N] binary16; S (optional, may be NULL)
 * receives the unrounded binary64 sums.  Rows are distributed over OpenMP
 * threads; each element is still one ascending-k sum. */
void oracle_gemm_f16(const uint16_t* A, const uint16_t* B, uint16_t* C, double* S,
                     int64_t M, int64_t N, int64_t K)
{
    init_decode_table();
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j)
            one_element(A, B, N, K, i, j, &C[i * N + j], S ? &S[i * N + j] : NULL);
}

/* Selected elements (I[p], J[p]) of the same product, for shapes where the
 * full triple loop is too slow. */
void oracle_gemm_f16_points(const uint16_t* A, const uint16_t* B, int64_t M, int64_t N,
                            int64_t K, const int64_t* I, const int64_t* J, int64_t P,
                            uint16_t* C, double* S)
{
    (void)M;
    init_decode_table();
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t p = 0; p < P; ++p)
        one_element(A, B, N, K, I[p], J[p], &C[p], S ? &S[p] : NULL);
}

/* ---- streaming elementwise ----------------------------------------------- */

void oracle_add_f32(const float* x, const float* y, float* z, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        z[i] = x[i] + y[i];
}

void oracle_add_scalar_f32(const float* x, float c, float* z, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        z[i] = x[i] + c;
}

/* o[j] = (((0 + x[0][j]) + x[1][j]) + ...) + x[R-1][j], binary32, ascending
 * i.  x is [R][n] row-major. */
void oracle_sum_axis0_f32(const float* x, float* o, int64_t R, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j) {
        float s = 0.0f;
        for (int64_t i = 0; i < R; ++i)
            s = s + x[i * n + j];
        o[j] = s;
    }
}

void oracle_fill_f32(float* o, float v, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        o[i] = v;
}

void oracle_iota_f32(float* o, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        o[i] = (float)i;
}
