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
 *     section 2.2, second layer;
 *   - the block-scaled variant of that 4-bit scheme (fp8 e4m3 activations and
 *     e2m1 weights, one power-of-two e8m0 scale per 32 values along K): the
 *     pages' precision scheme ([overview] section 2.2, second layer, and the
 *     e2m1 weight unpack of [overview] section 4.3) run on the OCP Microscaling
 *     (MX) v1.0 element and scale formats.  The formats are that published
 *     specification's, not the pages'; the block size 32 and the fp8
 *     activation are this oracle's reading.
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
 * fp8 e4m3 (OCP MX "E4M3"): bit 7 sign, bits 6..3 exponent E (bias 7), bits 2..0
 * mantissa M.  E = 0 is the subnormal range: value = M/8 * 2^-6.  Otherwise
 * value = (1 + M/8) * 2^(E-7), except E = 15 with M = 7, which is NaN.  There
 * are no infinities; the largest finite magnitude is 1.75 * 2^8 = 448.
 */
double orc_fp8e4m3_value(uint8_t code)
{
    int s = (code >> 7) & 1;
    int E = (code >> 3) & 15;
    int M = code & 7;
    double v;
    if (E == 15 && M == 7)
        v = NAN;
    else if (E == 0)
        v = ldexp((double)M, -9);                  /* M/8 * 2^-6 */
    else
        v = ldexp(8.0 + (double)M, E - 10);        /* (1 + M/8) * 2^(E-7) */
    return s ? -v : v;
}

/* e8m0 block scale (OCP MX): an 8-bit biased exponent, value 2^(code - 127);
 * code 255 is NaN.  No sign, no mantissa. */
double orc_e8m0_value(uint8_t code)
{
    return code == 255 ? NAN : ldexp(1.0, (int)code - 127);
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

/* ------------------------------------------------------ MX block-scaled GEMM */

/*
 * r = act(alpha * sum_k a[i][k] * w[k][j] + bias[j]), all in binary64, with
 *   a[i][k] = fp8e4m3(A[i][k]) * e8m0(SA[i][k/32])
 *   w[k][j] = e2m1(B[k][j])    * e8m0(SB[k/32][j])
 *
 *   A   fp8 e4m3 codes, logical M x K row-major
 *   SA  e8m0 codes, [M][K/32]
 *   B   e2m1 codes, logical K x N row-major, one code per byte (low 4 bits)
 *   SB  e8m0 codes, [K/32][N]
 *   bias [N] of bias_kind (nullable); act 0 identity, 1 GELU (erf form)
 *   R   out, M x N binary64, unrounded
 *
 * Every a and w is exact in binary64 (4- and 2-bit significands times powers of
 * two within binary64's range), and so is every product.  Sums run with k
 * ascending.  Returns 0, or -1 on a bad argument (K not a multiple of 32).
 */
int orc_gemm_mx(int64_t M, int64_t N, int64_t K,
                const uint8_t *A, const uint8_t *SA,
                const uint8_t *B, const uint8_t *SB,
                double alpha, int bias_kind, const void *bias,
                int act, double *R, int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || K % 32 || !R) return -1;
    if (M == 0 || N == 0) return 0;
    if (K > 0 && (!A || !SA || !B || !SB)) return -1;
    const int64_t G = K / 32;
    double *w = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1) * (size_t)N);
    double *a = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1) * (size_t)M);
    if (!w || !a) {
        free(w);
        free(a);
        return -1;
    }
    int nt = set_threads(nthreads);
    #pragma omp parallel for num_threads(nt) schedule(static)
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n)
            w[k * N + n] = orc_e2m1_value(B[k * N + n] & 0xf) * orc_e8m0_value(SB[(k / 32) * N + n]);
    #pragma omp parallel for num_threads(nt) schedule(static)
    for (int64_t i = 0; i < M; ++i)
        for (int64_t k = 0; k < K; ++k)
            a[i * K + k] = orc_fp8e4m3_value(A[i * K + k]) * orc_e8m0_value(SA[i * G + k / 32]);

    #pragma omp parallel num_threads(nt)
    {
        double *acc = (double *)malloc(sizeof(double) * (size_t)N);
        #pragma omp for schedule(static)
        for (int64_t i = 0; i < M; ++i) {
            for (int64_t n = 0; n < N; ++n) acc[n] = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const double ak = a[i * K + k];
                const double *wk = w + k * N;
                for (int64_t n = 0; n < N; ++n) acc[n] += ak * wk[n];
            }
            for (int64_t n = 0; n < N; ++n) {
                double v = alpha * acc[n];
                if (bias) v += load_real(bias_kind, bias, n);
                if (act == 1) v = orc_gelu_erf(v);
                R[i * N + n] = v;
            }
        }
        free(acc);
    }
    free(w);
    free(a);
    return 0;
}

/*
 * binary64 -> fp8 e4m3 code, round to nearest even, saturating: magnitudes that
 * round past 448 give +-448 (the MX conversion clamps to the largest normal
 * rather than producing NaN).  NaN input gives code 0x7f.
 */
uint8_t orc_fp8e4m3_rne_sat(double x)
{
    if (isnan(x)) return 0x7f;
    uint8_t sign = signbit(x) ? 0x80 : 0;
    double ulp;
    double q = fabs(round_to_format(fabs(x), 4, -6, INFINITY, &ulp));
    if (q > 448.0) q = 448.0;
    if (q == 0.0) return sign;
    if (q < ldexp(1.0, -6))                        /* subnormal: q = M * 2^-9 */
        return sign | (uint8_t)ldexp(q, 9);
    int e;
    double m = frexp(q, &e);                       /* q = m * 2^e, m in [0.5,1) */
    int E = e - 1 + 7;
    uint8_t M = (uint8_t)((m * 2.0 - 1.0) * 8.0);
    return sign | (uint8_t)(E << 3) | M;
}

/*
 * Quantise binary16 activations to MX fp8 e4m3 with one e8m0 scale per 32
 * consecutive values of a row (the OCP MX v1.0 conversion):
 *   amax  = max |x| over the block
 *   e     = floor(log2(amax)) - 8          (8 = exponent of e4m3's largest normal)
 *   scale = 2^e, stored as code e + 127 (clamped to 0..254); amax = 0 gives code 0
 *   code  = fp8e4m3_rne_sat(x / scale)
 *   X   binary16 bits, M x K row-major;  codes M x K;  scales [M][K/32]
 * x / scale is exact (a power of two within range), so the only rounding is the
 * conversion to e4m3.  Returns 0, or -1 on a bad argument or a non-finite input.
 */
int orc_quant_mx_e4m3(int64_t M, int64_t K, const uint16_t *X, uint8_t *codes, uint8_t *scales)
{
    if (M < 0 || K < 0 || K % 32) return -1;
    if (M * K > 0 && (!X || !codes || !scales)) return -1;
    for (int64_t i = 0; i < M; ++i)
        for (int64_t g = 0; g < K / 32; ++g) {
            const uint16_t *xb = X + i * K + g * 32;
            double amax = 0.0;
            for (int t = 0; t < 32; ++t) {
                double v = orc_f16_value(xb[t]);
                if (!isfinite(v)) return -1;
                if (fabs(v) > amax) amax = fabs(v);
            }
            int sc;
            if (amax == 0.0) {
                sc = 0;
            } else {
                int e2;
                frexp(amax, &e2);                  /* amax in [2^(e2-1), 2^e2) */
                sc = (e2 - 1) - 8 + 127;
                if (sc < 0) sc = 0;
                if (sc > 254) sc = 254;
            }
            scales[i * (K / 32) + g] = (uint8_t)sc;
            for (int t = 0; t < 32; ++t)
                codes[i * K + g * 32 + t] =
                    orc_fp8e4m3_rne_sat(orc_f16_value(xb[t]) / orc_e8m0_value((uint8_t)sc));
        }
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

void orc_fp8e4m3_values(int64_t n, const uint8_t *c, double *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_fp8e4m3_value(c[i]);
}

void orc_e8m0_values(int64_t n, const uint8_t *c, double *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e8m0_value(c[i]);
}

void orc_fp8e4m3_rne_sat_array(int64_t n, const double *x, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_fp8e4m3_rne_sat(x[i]);
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
