/*
 * oracle.c - plain CPU reference for the planned dense GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this library.  It shares no
 * code, header, table or helper with the HIP library, and the HIP library
 * never calls it.
 *
 * Page citations use two keys:
 *   [overview] the DeepGEMM overview article (lqnn.cn, mirrored at discosf.com)
 *   [generator] the DeepGEMM generator article (kwkr.cn)
 *
 * What is computed is the plain definition of the operation the pages build
 * kernels for:
 *
 *   r[i][j] = act( alpha * sum_k a[i][k] * b[k][j] + beta * d[i][j] + bias[j] )
 *
 *   - the GEMM with the "alpha * C + beta * D" epilogue: [generator] section 3.2,
 *     step 3 (the --epilogue argument of the code generator);
 *   - a bias term added in the epilogue: [generator] section 2.2, third layer
 *     (Epilogue Generator), whose example adds a per-column bias vector;
 *   - act = GELU fused after the GEMM: [overview] section 6.1 (op_type "gelu");
 *     the exact erf form is used: GELU(x) = x/2 * (1 + erf(x / sqrt 2));
 *   - accumulation wider than the 16-bit inputs, result cast to the output
 *     type: [overview] section 3.5, second lesson (fp32 accumulate, cast_output);
 *   - integer accumulation into 32 bits and round-to-nearest conversion of the
 *     integer result: [overview] section 4.3 (INT32 output, cvt.rn.f16.s32);
 *   - the 4-bit e2m1 code (sign, 2-bit exponent, 1-bit mantissa): [overview]
 *     section 2.2, second layer.
 *
 * Floating-point results are summed in binary64 with k ascending and returned
 * unrounded; the comparison rule lives in the tests.  Integer results are exact
 * in int64 and also returned wrapped to 32 bits.  The per-element summation
 * order does not depend on the thread count, so results are bit-identical for
 * any number of threads.
 *
 * Build: gcc -O2 -fopenmp -fPIC -shared -ffp-contract=off oracle.c -lm
 * (contraction is off so every product and sum is rounded on its own).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* element kinds understood by the oracle (its own numbering) */
enum { ORC_F16 = 0, ORC_BF16 = 1, ORC_F32 = 2, ORC_I8 = 3, ORC_I32 = 4, ORC_E2M1 = 5 };

/* ---------------------------------------------------------------- codecs */

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double orc_f16_value(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);                 /* zero or subnormal: f * 2^-24 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp(1024.0 + (double)f, e - 25);     /* (1 + f/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16 is the upper half of an IEEE binary32. */
double orc_bf16_value(uint16_t h)
{
    uint32_t w = (uint32_t)h << 16;
    float x;
    memcpy(&x, &w, sizeof x);
    return (double)x;
}

/*
 * e2m1: bit 3 sign, bits 2..1 exponent E, bit 0 mantissa M, exponent bias 1.
 * E = 0 is the subnormal range: value = M * 0.5.
 * E > 0: value = 2^(E-1) * (1 + M/2).
 * Codes 0..7 give 0, 0.5, 1, 1.5, 2, 3, 4, 6; codes 8..15 are their negatives.
 */
double orc_e2m1_value(uint8_t code)
{
    int s = (code >> 3) & 1;
    int E = (code >> 1) & 3;
    int M = code & 1;
    double v = (E == 0) ? 0.5 * M : ldexp(1.0 + 0.5 * M, E - 1);
    return s ? -v : v;
}

/*
 * Round a binary64 value to the nearest value of a binary format with p
 * significand bits (including the hidden one), minimum normal exponent emin and
 * largest finite value maxv, ties to even; return the rounded value (or +-inf
 * past the overflow threshold).  rint() rounds to nearest-even in the default
 * rounding mode, and x / ulp is exact because ulp is a power of two.
 */
static double round_to_format(double x, int p, int emin, double maxv, double *ulp_out)
{
    if (x == 0.0 || isnan(x) || isinf(x)) {
        *ulp_out = 0.0;
        return x;
    }
    int e;
    frexp(fabs(x), &e);            /* |x| = m * 2^e, m in [0.5, 1)  => exponent e-1 */
    int ex = e - 1;
    if (ex < emin) ex = emin;      /* subnormal range shares the minimum-normal ulp */
    double ulp = ldexp(1.0, ex - (p - 1));
    double q = rint(x / ulp) * ulp;
    /* overflow: anything that rounds beyond maxv goes to infinity */
    if (fabs(q) > maxv) q = copysign(INFINITY, x);
    *ulp_out = ulp;
    return q;
}

/* binary64 -> binary16 bits, round to nearest even. */
uint16_t orc_f16_rne(double x)
{
    if (isnan(x)) return 0x7e00;
    double ulp;
    double q = round_to_format(x, 11, -14, 65504.0, &ulp);
    uint16_t sign = signbit(q) ? 0x8000 : 0;
    double a = fabs(q);
    if (isinf(a)) return sign | 0x7c00;
    if (a == 0.0) return sign;
    if (a < ldexp(1.0, -14))                       /* subnormal: a = f * 2^-24 */
        return sign | (uint16_t)ldexp(a, 24);
    int e;
    double m = frexp(a, &e);                       /* a = m * 2^e, m in [0.5,1) */
    int E = e - 1 + 15;
    uint16_t f = (uint16_t)((m * 2.0 - 1.0) * 1024.0);
    return sign | (uint16_t)(E << 10) | f;
}

/* binary64 -> bfloat16 bits, round to nearest even (8 significand bits). */
uint16_t orc_bf16_rne(double x)
{
    if (isnan(x)) return 0x7fc0;
    double ulp;
    /* largest finite bfloat16: (2 - 2^-7) * 2^127 */
    double q = round_to_format(x, 8, -126, ldexp(2.0 - ldexp(1.0, -7), 127), &ulp);
    /* q is exactly representable in binary32 (or is +-inf/0) */
    float f = (float)q;
    uint32_t w;
    memcpy(&w, &f, sizeof w);
    return (uint16_t)(w >> 16);
}

/* GELU with the exact error function: x/2 * (1 + erf(x / sqrt 2)). */
double orc_gelu_erf(double x)
{
    return 0.5 * x * (1.0 + erf(x * M_SQRT1_2));
}

static double load_real(int kind, const void *p, int64_t idx)
{
    switch (kind) {
    case ORC_F16:  return orc_f16_value(((const uint16_t *)p)[idx]);
    case ORC_BF16: return orc_bf16_value(((const uint16_t *)p)[idx]);
    case ORC_F32:  return (double)((const float *)p)[idx];
    case ORC_I8:   return (double)((const int8_t *)p)[idx];
    case ORC_I32:  return (double)((const int32_t *)p)[idx];
    case ORC_E2M1: return orc_e2m1_value(((const uint8_t *)p)[idx] & 0xf);
    default:       return NAN;
    }
}

static int set_threads(int nthreads)
{
#ifdef _OPENMP
    int n = nthreads > 0 ? nthreads : omp_get_max_threads();
    return n;
#else
    (void)nthreads;
    return 1;
#endif
}

/* --------------------------------------------------------- real-valued GEMM */

/*
 * r = act(alpha * A.B + beta * D + bias), all in binary64.
 *
 *   A      logical M x K, row-major, contiguous; kind F16 / BF16 / F32
 *   B      logical K x N, row-major, contiguous; kind F16 / BF16 / F32 / E2M1
 *          (E2M1: one code per byte, low 4 bits)
 *   scale  E2M1 only: binary16 bits, logical [K/group_k][N]; the weight is
 *          w[k][n] = e2m1(code[k][n]) * scale[k/group_k][n]  (exact in binary64:
 *          a 2-bit significand times an 11-bit one)
 *   D      logical M x N row-major (nullable when beta == 0; not read then)
 *   bias   [N] (nullable)
 *   act    0 identity, 1 GELU (erf form)
 *   R      out, M x N binary64, unrounded
 *
 * Returns 0, or -1 on a bad argument.
 */
int orc_gemm_real(int64_t M, int64_t N, int64_t K,
                  int a_kind, const void *A,
                  int b_kind, const void *B,
                  const uint16_t *scale, int64_t group_k,
                  double alpha,
                  double beta, int d_kind, const void *D,
                  int bias_kind, const void *bias,
                  int act, double *R, int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || !R) return -1;
    if (M == 0 || N == 0) return 0;
    if (K > 0 && (!A || !B)) return -1;
    if (b_kind == ORC_E2M1 && (!scale || group_k <= 0 || K % group_k)) return -1;
    if (beta != 0.0 && !D) return -1;

    /* decode B once: w[k][n] */
    double *w = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1) * (size_t)N);
    if (!w) return -1;
    int nt = set_threads(nthreads);
    #pragma omp parallel for num_threads(nt) schedule(static)
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n) {
            double v = load_real(b_kind, B, k * N + n);
            if (b_kind == ORC_E2M1)
                v = v * orc_f16_value(scale[(k / group_k) * N + n]);
            w[k * N + n] = v;
        }

    #pragma omp parallel num_threads(nt)
    {
        double *acc = (double *)malloc(sizeof(double) * (size_t)N);
        #pragma omp for schedule(static)
        for (int64_t i = 0; i < M; ++i) {
            for (int64_t n = 0; n < N; ++n) acc[n] = 0.0;
            /* k ascending for every element */
            for (int64_t k = 0; k < K; ++k) {
                double a = load_real(a_kind, A, i * K + k);
                const double *wk = w + k * N;
                for (int64_t n = 0; n < N; ++n) acc[n] += a * wk[n];
            }
            for (int64_t n = 0; n < N; ++n) {
                double v = alpha * acc[n];
                if (beta != 0.0) v += beta * load_real(d_kind, D, i * N + n);
                if (bias) v += load_real(bias_kind, bias, n);
                if (act == 1) v = orc_gelu_erf(v);
                R[i * N + n] = v;
            }
        }
        free(acc);
    }
    free(w);
    return 0;
}

/* -------------------------------------------------------------- integer GEMM */

/*
 * acc[i][j] = sum_k a[i][k] * b[k][j] over int8 inputs, exact in int64;
 * R = alpha * acc + beta * d (exact, int64), C = R wrapped modulo 2^32.
 * Because wrapping is a ring homomorphism, C equals what a 32-bit two's
 * complement accumulator computes step by step.
 *
 * Returns the number of elements for which acc, alpha*acc, beta*d or R left
 * the int32 range (0 when the 32-bit result is the true one), or -1 on a bad
 * argument.  Either output pointer may be NULL.
 */
int64_t orc_gemm_int(int64_t M, int64_t N, int64_t K,
                     const int8_t *A, const int8_t *B,
                     int64_t alpha, int64_t beta, const int32_t *D,
                     int64_t *R, int32_t *C, int nthreads)
{
    if (M < 0 || N < 0 || K < 0) return -1;
    if (M == 0 || N == 0) return 0;
    if (K > 0 && (!A || !B)) return -1;
    if (beta != 0 && !D) return -1;
    int nt = set_threads(nthreads);
    int64_t overflow = 0;
    #pragma omp parallel num_threads(nt) reduction(+ : overflow)
    {
        int64_t *acc = (int64_t *)malloc(sizeof(int64_t) * (size_t)N);
        #pragma omp for schedule(static)
        for (int64_t i = 0; i < M; ++i) {
            for (int64_t n = 0; n < N; ++n) acc[n] = 0;
            for (int64_t k = 0; k < K; ++k) {
                int64_t a = A[i * K + k];
                const int8_t *bk = B + k * N;
                for (int64_t n = 0; n < N; ++n) acc[n] += a * (int64_t)bk[n];
            }
            for (int64_t n = 0; n < N; ++n) {
                int64_t s = alpha * acc[n];
                int64_t t = beta != 0 ? beta * (int64_t)D[i * N + n] : 0;
                int64_t r = s + t;
                if (acc[n] != (int32_t)acc[n] || s != (int32_t)s || t != (int32_t)t ||
                    r != (int32_t)r)
                    overflow += 1;
                if (R) R[i * N + n] = r;
                if (C) C[i * N + n] = (int32_t)(uint32_t)(uint64_t)r;
            }
        }
        free(acc);
    }
    return overflow;
}

/*
 * Requantise an integer accumulator ([overview] section 4.3: the INT32 result
 * converted with round-to-nearest).  The decision is taken in binary32, in this
 * exact order, each step rounded to nearest even:
 *   v = f32( f32( f32(acc) * alpha ) + bias[j] )        (bias term only if given)
 *   out_kind ORC_I8 : q = clamp(rint(v), -128, 127)     (saturating int8)
 *   out_kind ORC_F16: binary16 bits of v, round to nearest even
 * acc is the 32-bit accumulator value (wrapped), as the integer GEMM leaves it.
 */
int orc_requant(int64_t M, int64_t N, const int32_t *acc, float alpha,
                const float *bias, int out_kind, void *out)
{
    if (M < 0 || N < 0 || (M * N > 0 && (!acc || !out))) return -1;
    if (out_kind != ORC_I8 && out_kind != ORC_F16) return -1;
    for (int64_t i = 0; i < M; ++i)
        for (int64_t n = 0; n < N; ++n) {
            volatile float a = (float)acc[i * N + n];
            volatile float v = a * alpha;
            if (bias) v = v + bias[n];
            if (out_kind == ORC_I8) {
                float r = rintf(v);
                int q = r > 127.0f ? 127 : (r < -128.0f ? -128 : (int)r);
                ((int8_t *)out)[i * N + n] = (int8_t)q;
            } else {
                ((uint16_t *)out)[i * N + n] = orc_f16_rne((double)v);
            }
        }
    return 0;
}

/* --------------------------------------------------- vectorised codec helpers */

void orc_f16_values(int64_t n, const uint16_t *h, double *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_f16_value(h[i]);
}

void orc_bf16_values(int64_t n, const uint16_t *h, double *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_value(h[i]);
}

void orc_e2m1_values(int64_t n, const uint8_t *c, double *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e2m1_value(c[i] & 0xf);
}

void orc_f16_rne_array(int64_t n, const double *x, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_f16_rne(x[i]);
}

void orc_bf16_rne_array(int64_t n, const double *x, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_rne(x[i]);
}

void orc_gelu_erf_array(int64_t n, const double *x, double *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_gelu_erf(x[i]);
}

int orc_max_threads(void)
{
    return set_threads(0);
}
