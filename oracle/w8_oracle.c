/*
 * Plain CPU oracle for the small-M 8-bit quantized linear-layer GEMM
 *     Y = dequant(Xq) . dequant(Wq)^T
 * in the three formats FP8_Dynamic, W8A8_INT8 and Block_FP8.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU library never
 * links, loads or calls it, and the two share no code.
 *
 * Source of the method: ai-radar.it, "Helion nel backend vLLM: un solo GEMM,
 * tuning per forma e guadagni fino al 10%".  Paragraph 1 names the three
 * 8-bit formats; paragraph 2 states that Standard, Split-K and Swap-AB are the
 * same GEMM computed three ways.  The page gives no formulas, granularities or
 * rounding rules, so this file writes out the plainest definitions:
 *
 *   - FP8_Dynamic: activations quantized per token (row) to OCP E4M3FN at run
 *     time, weights E4M3FN with one fp32 scale per output channel.
 *   - W8A8_INT8:   activations quantized per token to int8, weights int8 with
 *     one fp32 scale per output channel, exact integer accumulation.
 *   - Block_FP8:   activations quantized per 1x128 group along K, weights per
 *     128x128 block, both E4M3FN; each group's partial dot product is scaled
 *     before the groups are summed.
 *
 * Scale rule (all formats): s = amax / Qmax (fp32, correctly rounded), with
 * Qmax = 448 for E4M3FN and 127 for int8; an all-zero group takes s = 1.
 * Code rule: v = x / s (fp32, correctly rounded true division), then
 * E4M3FN: clamp v to [-448, 448] and round to nearest, ties to even;
 * int8:   round to nearest, ties to even, and clamp to [-127, 127].
 *
 * Everything downstream of the codes is exact or fp64:
 *   - int8 dot products in int64;
 *   - E4M3FN dot products in int64 after scaling every decoded value by 2^9
 *     (every finite E4M3FN value times 2^9 is an integer of magnitude at most
 *     229376), so the sum is exact and only the final 2^-18 is applied;
 *   - scale application in fp64.
 *
 * This file must be compiled without -ffast-math and with -ffp-contract=off:
 * float division and nearbyint() are then the IEEE-754 operations the
 * definitions above name (x86-64 evaluates float expressions in float).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_FP8_DYNAMIC 0
#define OR_W8A8_INT8   1
#define OR_BLOCK_FP8   2

#define OR_OK          0
#define OR_E_ARG       1
#define OR_E_NONFINITE 2
#define OR_E_RANGE     3

#define OR_GROUP 128 /* Block_FP8 group / block edge */

/* ------------------------------------------------------------------------ */
/* OCP 8-bit floating point, E4M3FN variant: 1 sign bit, 4 exponent bits with
 * bias 7, 3 mantissa bits; no infinities; S.1111.111 is NaN; the largest
 * finite magnitude is S.1111.110 = 448; exponent field 0 holds subnormals
 * m * 2^-9, m = 0..7.                                                       */

double or_e4m3_decode(uint8_t code)
{
    int sign = (code >> 7) & 1;
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    double mag;
    if (e == 0xF && m == 0x7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m, -9);                 /* m/8 * 2^(1-7) */
    else
        mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -mag : mag;
}

uint8_t or_e4m3_encode(float v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs((double)v);
    double step, n, r;
    int e;

    if (a > 448.0)
        a = 448.0;                                  /* saturate */
    /* Spacing of E4M3FN values around a: 2^-9 below the smallest normal
     * 2^-6, else 2^(E-3) in the binade [2^E, 2^(E+1)).                     */
    if (a < ldexp(1.0, -6)) {
        step = ldexp(1.0, -9);
    } else {
        frexp(a, &e);                               /* a = f * 2^e, f in [0.5,1) */
        step = ldexp(1.0, (e - 1) - 3);
    }
    n = nearbyint(a / step);                        /* a/step is exact; ties to even */
    r = n * step;                                   /* the nearest value, maybe 2^(E+1) */

    if (r == 0.0)
        return sign;
    if (r < ldexp(1.0, -6))
        return (uint8_t)(sign | (uint8_t)ldexp(r, 9));          /* subnormal */
    frexp(r, &e);
    {
        int E = e - 1;                              /* r in [2^E, 2^(E+1)) */
        int mant = (int)((ldexp(r, -E) - 1.0) * 8.0);
        return (uint8_t)(sign | (uint8_t)((E + 7) << 3) | (uint8_t)mant);
    }
}

int8_t or_int8_encode(float v)
{
    float r = nearbyintf(v);                        /* ties to even */
    if (r > 127.0f)
        r = 127.0f;
    if (r < -127.0f)
        r = -127.0f;
    return (int8_t)r;
}

/* Array forms of the two encoders (element-wise, same rules). */
void or_e4m3_encode_n(const float *v, int64_t n, uint8_t *out)
{
    int64_t i;
    for (i = 0; i < n; ++i)
        out[i] = or_e4m3_encode(v[i]);
}

void or_int8_encode_n(const float *v, int64_t n, int8_t *out)
{
    int64_t i;
    for (i = 0; i < n; ++i)
        out[i] = or_int8_encode(v[i]);
}

float or_bf16_to_float(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* ------------------------------------------------------------------------ */
/* One quantization group: n values at x[0], x[stride], ...  Writes the codes
 * at q[0], q[qstride], ... and returns the scale through *s.  is_int8 picks
 * int8 (Qmax 127) or E4M3FN (Qmax 448).                                     */
static int quantize_group(const float *x, int64_t n, int64_t stride,
                          int is_int8, uint8_t *q, int64_t qstride, float *s)
{
    float amax = 0.0f, scale;
    const float qmax = is_int8 ? 127.0f : 448.0f;
    int64_t i;

    for (i = 0; i < n; ++i) {
        float a = fabsf(x[i * stride]);
        if (!isfinite(a))
            return OR_E_NONFINITE;
        if (a > amax)
            amax = a;
    }
    scale = (amax == 0.0f) ? 1.0f : amax / qmax;
    for (i = 0; i < n; ++i) {
        float v = x[i * stride] / scale;
        q[i * qstride] = is_int8 ? (uint8_t)or_int8_encode(v) : or_e4m3_encode(v);
    }
    *s = scale;
    return OR_OK;
}

/* Quantize one group of n contiguous fp32 values (exposed for the tests). */
int or_quantize_group(const float *x, int64_t n, int is_int8, uint8_t *q, float *s)
{
    if (n <= 0)
        return OR_E_ARG;
    return quantize_group(x, n, 1, is_int8, q, 1, s);
}

/* ------------------------------------------------------------------------ */
/* Activation quantization.  X is bf16 [M, K] (row stride ldx elements).
 *   FP8_Dynamic, W8A8_INT8: one scale per row, sx[M].
 *   Block_FP8: one scale per row and 128-wide K group, sx[M, K/128];
 *              K must be a multiple of 128.
 * Xq is [M, K] bytes with row stride ldq.                                   */
int or_quantize_act(int fmt, int M, int K, const uint16_t *x, int64_t ldx,
                    uint8_t *xq, int64_t ldq, float *sx)
{
    int m, g, rc;
    float row[OR_GROUP];

    if (M <= 0 || K <= 0 || ldx < K || ldq < K)
        return OR_E_ARG;
    if (fmt == OR_FP8_DYNAMIC || fmt == OR_W8A8_INT8) {
        for (m = 0; m < M; ++m) {
            /* widen the bf16 row to fp32 (exact), then quantize it as one group */
            float *wide = (float *)malloc(sizeof(float) * (size_t)K);
            int k;
            if (!wide)
                return OR_E_ARG;
            for (k = 0; k < K; ++k)
                wide[k] = or_bf16_to_float(x[(int64_t)m * ldx + k]);
            rc = quantize_group(wide, K, 1, fmt == OR_W8A8_INT8,
                                xq + (int64_t)m * ldq, 1, &sx[m]);
            free(wide);
            if (rc)
                return rc;
        }
        return OR_OK;
    }
    if (fmt == OR_BLOCK_FP8) {
        int G;
        if (K % OR_GROUP)
            return OR_E_ARG;
        G = K / OR_GROUP;
        for (m = 0; m < M; ++m)
            for (g = 0; g < G; ++g) {
                int k;
                for (k = 0; k < OR_GROUP; ++k)
                    row[k] = or_bf16_to_float(x[(int64_t)m * ldx + g * OR_GROUP + k]);
                rc = quantize_group(row, OR_GROUP, 1, 0,
                                    xq + (int64_t)m * ldq + g * OR_GROUP, 1,
                                    &sx[(int64_t)m * G + g]);
                if (rc)
                    return rc;
            }
        return OR_OK;
    }
    return OR_E_ARG;
}

/* ------------------------------------------------------------------------ */
/* Offline weight quantization from fp32 W [N, K] (row stride ldw).
 *   FP8_Dynamic: E4M3FN codes, one scale per output row, sw[N].
 *   Block_FP8:   E4M3FN codes, one scale per 128x128 block,
 *                sw[ceil(N/128), ceil(K/128)]; edge blocks may be partial.
 * W8A8_INT8 weights are given as codes and scales directly (not quantized
 * here).  Wq is [N, K] bytes with row stride ldq.                           */
int or_quantize_weight(int fmt, int N, int K, const float *w, int64_t ldw,
                       uint8_t *wq, int64_t ldq, float *sw)
{
    int n;
    if (N <= 0 || K <= 0 || ldw < K || ldq < K)
        return OR_E_ARG;
    if (fmt == OR_FP8_DYNAMIC) {
        int bad = 0;
        /* rows are independent groups; running them on several threads
         * changes no arithmetic */
#pragma omp parallel for schedule(static) reduction(| : bad)
        for (n = 0; n < N; ++n)
            bad |= quantize_group(w + (int64_t)n * ldw, K, 1, 0, wq + (int64_t)n * ldq, 1, &sw[n]);
        return bad ? OR_E_NONFINITE : OR_OK;
    }
    if (fmt == OR_BLOCK_FP8) {
        int NB = (N + OR_GROUP - 1) / OR_GROUP, KB = (K + OR_GROUP - 1) / OR_GROUP;
        int bn, bad = 0;
        /* blocks are independent groups (see above) */
#pragma omp parallel for schedule(static) reduction(| : bad)
        for (bn = 0; bn < NB; ++bn) {
            int bk;
            for (bk = 0; bk < KB; ++bk) {
                int n0 = bn * OR_GROUP, k0 = bk * OR_GROUP;
                int nr = (N - n0 < OR_GROUP) ? N - n0 : OR_GROUP;
                int kc = (K - k0 < OR_GROUP) ? K - k0 : OR_GROUP;
                float amax = 0.0f, scale;
                int i, j;
                for (i = 0; i < nr; ++i)
                    for (j = 0; j < kc; ++j) {
                        float a = fabsf(w[(int64_t)(n0 + i) * ldw + k0 + j]);
                        if (!isfinite(a))
                            bad = 1;
                        else if (a > amax)
                            amax = a;
                    }
                scale = (amax == 0.0f) ? 1.0f : amax / 448.0f;
                for (i = 0; i < nr; ++i)
                    for (j = 0; j < kc; ++j)
                        wq[(int64_t)(n0 + i) * ldq + k0 + j] =
                            or_e4m3_encode(w[(int64_t)(n0 + i) * ldw + k0 + j] / scale);
                sw[(int64_t)bn * KB + bk] = scale;
            }
        }
        return bad ? OR_E_NONFINITE : OR_OK;
    }
    return OR_E_ARG;
}

/* ------------------------------------------------------------------------ */
/* Exact accumulators.
 * or_acc_int8: C[m*N + n] = sum_k xq[m,k] * wq[n,k] over k in [k0, k1), int64.
 * or_acc_fp8:  D[m*N + n] = sum_k dec(xq[m,k]) * dec(wq[n,k]) over [k0, k1),
 *              computed exactly as 2^-18 * sum of int64 products of
 *              dec()*2^9; returns OR_E_ARG if a NaN code is met.              */
int or_acc_int8(int M, int N, int k0, int k1, const int8_t *xq, int64_t ldq,
                const int8_t *wq, int64_t ldw, int64_t *C)
{
    int m, n;
    if (M <= 0 || N <= 0 || k0 < 0 || k1 < k0)
        return OR_E_ARG;
#pragma omp parallel for private(n) schedule(static)
    for (m = 0; m < M; ++m)
        for (n = 0; n < N; ++n) {
            int64_t acc = 0;
            int k;
            for (k = k0; k < k1; ++k)
                acc += (int64_t)xq[(int64_t)m * ldq + k] * (int64_t)wq[(int64_t)n * ldw + k];
            C[(int64_t)m * N + n] = acc;
        }
    return OR_OK;
}

static int64_t e4m3_int[256];   /* dec(c) * 2^9, an exact integer; NaN codes flagged */
static int e4m3_int_ready;

static void init_e4m3_int(void)
{
    int c;
    if (e4m3_int_ready)
        return;
    for (c = 0; c < 256; ++c) {
        double d = or_e4m3_decode((uint8_t)c);
        e4m3_int[c] = isnan(d) ? INT64_MIN : (int64_t)ldexp(d, 9);
    }
    e4m3_int_ready = 1;
}

int or_acc_fp8(int M, int N, int k0, int k1, const uint8_t *xq, int64_t ldq,
               const uint8_t *wq, int64_t ldw, double *D)
{
    int m, n, bad = 0;
    if (M <= 0 || N <= 0 || k0 < 0 || k1 < k0)
        return OR_E_ARG;
    init_e4m3_int();
#pragma omp parallel for private(n) schedule(static) reduction(| : bad)
    for (m = 0; m < M; ++m)
        for (n = 0; n < N; ++n) {
            int64_t acc = 0;
            int k;
            for (k = k0; k < k1; ++k) {
                int64_t a = e4m3_int[xq[(int64_t)m * ldq + k]];
                int64_t b = e4m3_int[wq[(int64_t)n * ldw + k]];
                if (a == INT64_MIN || b == INT64_MIN)
                    bad = 1;
                else
                    acc += a * b;
            }
            D[(int64_t)m * N + n] = ldexp((double)acc, -18);
        }
    return bad ? OR_E_ARG : OR_OK;
}

/* ------------------------------------------------------------------------ */
/* The whole GEMM from codes and scales, result in fp64 (not rounded to bf16).
 *   W8A8_INT8:   Y[m,n] = C[m,n] * sx[m] * sw[n]
 *   FP8_Dynamic: Y[m,n] = D[m,n] * sx[m] * sw[n]
 *   Block_FP8:   Y[m,n] = sum_g sx[m,g] * sw[n/128, g] * D_g[m,n],
 *                D_g the exact dot product over k in [128g, 128g+128),
 *                groups summed in increasing g.
 * Scale layouts are those written by or_quantize_act / or_quantize_weight.
 * Y is [M, N] row-major.  Returns OR_E_RANGE if an int8 accumulator falls
 * outside int32 (the GPU accumulates in int32).                            */
int or_gemm(int fmt, int M, int N, int K,
            const uint8_t *xq, int64_t ldq, const float *sx,
            const uint8_t *wq, int64_t ldw, const float *sw, double *Y)
{
    const int64_t total = (int64_t)M * N;
    int64_t i;
    int rc = OR_OK;

    if (M <= 0 || N <= 0 || K <= 0)
        return OR_E_ARG;

    if (fmt == OR_W8A8_INT8) {
        int64_t *C = (int64_t *)malloc(sizeof(int64_t) * (size_t)total);
        if (!C)
            return OR_E_ARG;
        rc = or_acc_int8(M, N, 0, K, (const int8_t *)xq, ldq, (const int8_t *)wq, ldw, C);
        for (i = 0; rc == OR_OK && i < total; ++i) {
            int m = (int)(i / N), n = (int)(i % N);
            if (C[i] > INT32_MAX || C[i] < INT32_MIN)
                rc = OR_E_RANGE;
            else
                Y[i] = (double)C[i] * (double)sx[m] * (double)sw[n];
        }
        free(C);
        return rc;
    }

    if (fmt == OR_FP8_DYNAMIC) {
        double *D = (double *)malloc(sizeof(double) * (size_t)total);
        if (!D)
            return OR_E_ARG;
        rc = or_acc_fp8(M, N, 0, K, xq, ldq, wq, ldw, D);
        for (i = 0; rc == OR_OK && i < total; ++i) {
            int m = (int)(i / N), n = (int)(i % N);
            Y[i] = D[i] * (double)sx[m] * (double)sw[n];
        }
        free(D);
        return rc;
    }

    if (fmt == OR_BLOCK_FP8) {
        int G, KB, g;
        double *D;
        if (K % OR_GROUP)
            return OR_E_ARG;
        G = K / OR_GROUP;
        KB = G;                                    /* weight blocks along K */
        D = (double *)malloc(sizeof(double) * (size_t)total);
        if (!D)
            return OR_E_ARG;
        for (i = 0; i < total; ++i)
            Y[i] = 0.0;
        for (g = 0; rc == OR_OK && g < G; ++g) {
            rc = or_acc_fp8(M, N, g * OR_GROUP, (g + 1) * OR_GROUP, xq, ldq, wq, ldw, D);
            for (i = 0; rc == OR_OK && i < total; ++i) {
                int m = (int)(i / N), n = (int)(i % N);
                Y[i] += (double)sx[(int64_t)m * G + g] *
                        (double)sw[(int64_t)(n / OR_GROUP) * KB + g] * D[i];
            }
        }
        free(D);
        return rc;
    }
    return OR_E_ARG;
}

/* Number of OpenMP threads the accumulator loops use (1 without OpenMP). */
int or_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Sets the OpenMP thread count of the loops above (n >= 1; ignored without
 * OpenMP).  Timing only: the results do not depend on it, since each thread
 * computes whole, independent rows or blocks. */
void or_set_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
