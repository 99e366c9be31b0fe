/*
 * oracle.c -- plain, slow, obviously-correct CPU oracle for the W2A8 ternary
 * linear layer and the role-dependent (FP8 / bf16) projections.  TEST
 * INFRASTRUCTURE ONLY: the tests, the smoke check and the
 * CPU-baseline leg of the benchmark may call it; the product path never does.
 * It shares no code, header, table or constant with the HIP library.
 *
 * What it follows (page: "BitMTP: When Multi-Token Prediction Meets Low-Bit
 * Large Language Models", ai.info AI summary):
 *   - "What This Paper Is About": the backbone is BitNet b1.58, i.e. ternary
 *     (1.58-bit) weights.
 *   - "Main Findings", first bullet: the low-bit setting is W2A8, two-bit
 *     weights and eight-bit activations.
 *   - "Methodology in Plain English", paragraph 3: M1 runs packed low-bit
 *     operators chosen by replay width and input/output dimensions;
 *     paragraph 4: evaluation uses packed W2A8 execution.
 * The pages print no formula for the quantizers, no packed layout and no
 * worked example.  The readings taken here (each one is listed with its
 * reason in the design notes) are:
 *   ternarize : gamma = mean|W| per tensor (or per fused segment), summed in
 *               double in row-major order, divided by N*K in double, rounded
 *               once to fp32; t = clamp(rint(W / gamma), -1, 1) with an fp32
 *               IEEE division and round-half-to-even; gamma == 0 gives t == 0.
 *   quantize  : per token row, a = max|x| (bf16 widened exactly to fp32);
 *               inv = 127 / a (fp32 division); q = clamp(rint(x * inv),
 *               -127, 127) (fp32 multiply, round-half-to-even); s = a / 127
 *               (fp32 division); a == 0 gives q == 0 and s == 0.
 *   contract  : acc[m][n] = sum_k q[m][k] * t[n][k], int32 accumulation.
 *   dequant   : y[m][n] = acc * s_m * gamma(n), evaluated in double.
 *   format    : code c = t + 1 (0, 1, 2; 3 is invalid), 2 bits per weight.
 *               Row n holds K/16 little-endian 32-bit words; word i holds the
 *               sixteen weights k = 16 i + e, e = 4 j + b (j, b in 0..3), the
 *               code of element e sitting at bit 8 b + 2 j.  In byte terms,
 *               byte 4 i + b of the row holds elements 16 i + 4 j + b at bits
 *               2 j.  Rows are contiguous, K/4 bytes each.
 *
 * Role-dependent projections (same page, "Methodology in Plain English",
 * the paragraph on M1: cheaper "fast" projections for drafting, careful
 * "critical" ones for autoregressive steps and verification, and FP8 draft
 * projections on H20).  The pages give no formula; the readings are:
 *   e4m3      : the OCP 8-bit floating-point format E4M3 ("FN": 4 exponent
 *               bits with bias 7, 3 mantissa bits, no infinities, S.1111.111
 *               is NaN, largest finite 448, subnormals down to 2^-9);
 *               encoding rounds to nearest, ties to even.
 *   fast      : per output row (weights) and per token (activations) an
 *               absmax scale: inv = 448 / a (fp32 division), code =
 *               e4m3(x * inv) (fp32 multiply, then the rounding above),
 *               s = a / 448 (fp32 division); a == 0 gives zero codes and
 *               s == 0.  y[m][n] = (sum_k dec(xq) dec(wq)) * s_m * s_n.
 *   critical  : y[m][n] = sum_k x[m][k] w[n][k] over bf16 x and w.
 *
 * Build: plain C11, no fast-math, no FP contraction (gcc -O2
 * -ffp-contract=off).  The OpenMP pragma on the contraction only spreads the
 * independent output rows over threads for timing; integer results do not
 * depend on it.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* bf16 -> fp32 is exact: the bf16 bits are the top half of the fp32 bits. */
static float orc_bf16_to_float(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/*
 * Absmean ternarization of one tensor W[N][K] (BitNet b1.58 reading).
 * Returns 0 on success, -1 if a value is not finite (outside the contract).
 */
int orc_ternarize_absmean(const float *W, int64_t N, int64_t K,
                          int8_t *t, float *gamma_out)
{
    int64_t count = N * K;
    double sum = 0.0;
    for (int64_t i = 0; i < count; i++) {
        if (!isfinite(W[i]))
            return -1;
        sum += fabs((double)W[i]);
    }
    float gamma = count > 0 ? (float)(sum / (double)count) : 0.0f;
    *gamma_out = gamma;
    for (int64_t i = 0; i < count; i++) {
        if (gamma == 0.0f) {
            t[i] = 0;
            continue;
        }
        float r = rintf(W[i] / gamma);
        if (r > 1.0f)
            r = 1.0f;
        if (r < -1.0f)
            r = -1.0f;
        t[i] = (int8_t)r;
    }
    return 0;
}

/*
 * Per-token absmax int8 quantization of x[M][K] given as bf16 bit patterns.
 * Returns 0 on success, -1 if a value is not finite.
 */
int orc_quantize_act(const uint16_t *x_bf16, int64_t M, int64_t K,
                     int8_t *q, float *scale)
{
    for (int64_t m = 0; m < M; m++) {
        const uint16_t *row = x_bf16 + m * K;
        float a = 0.0f;
        for (int64_t k = 0; k < K; k++) {
            float v = orc_bf16_to_float(row[k]);
            if (!isfinite(v))
                return -1;
            float av = fabsf(v);
            if (av > a)
                a = av;
        }
        if (a == 0.0f) {
            for (int64_t k = 0; k < K; k++)
                q[m * K + k] = 0;
            scale[m] = 0.0f;
            continue;
        }
        float inv = 127.0f / a;
        for (int64_t k = 0; k < K; k++) {
            float r = rintf(orc_bf16_to_float(row[k]) * inv);
            if (r > 127.0f)
                r = 127.0f;
            if (r < -127.0f)
                r = -127.0f;
            q[m * K + k] = (int8_t)r;
        }
        scale[m] = a / 127.0f;
    }
    return 0;
}

/*
 * Decode the packed format into ternary values t[N][K].  K must be a
 * multiple of 16.  Returns 0, or -1 at the first field holding the invalid
 * code 3.
 */
int orc_unpack(const uint8_t *packed, int64_t N, int64_t K, int8_t *t)
{
    if (K % 16 != 0)
        return -2;
    int64_t row_bytes = K / 4;
    for (int64_t n = 0; n < N; n++) {
        for (int64_t k = 0; k < K; k++) {
            int64_t i = k / 16;          /* 32-bit word within the row */
            int64_t e = k % 16;          /* element within the word    */
            int64_t j = e / 4, b = e % 4;
            uint8_t byte = packed[n * row_bytes + 4 * i + b];
            int code = (byte >> (2 * j)) & 3;
            if (code == 3)
                return -1;
            t[n * K + k] = (int8_t)(code - 1);
        }
    }
    return 0;
}

/* acc[m][n] = sum_k q[m][k] * t[n][k], exact in int32 for |acc| < 2^31. */
void orc_linear(const int8_t *q, const int8_t *t, int64_t M, int64_t N,
                int64_t K, int32_t *acc, int threads)
{
#ifdef _OPENMP
    if (threads < 1)
        threads = 1;
#pragma omp parallel for num_threads(threads) schedule(static)
#endif
    for (int64_t n = 0; n < N; n++) {
        const int8_t *w = t + n * K;
        for (int64_t m = 0; m < M; m++) {
            const int8_t *x = q + m * K;
            int32_t s = 0;
            for (int64_t k = 0; k < K; k++)
                s += (int32_t)x[k] * (int32_t)w[k];
            acc[m * N + n] = s;
        }
    }
    (void)threads;
}

/* y[m][n] = acc[m][n] * scale[m] * gamma_row[n], in double. */
void orc_dequant(const int32_t *acc, const float *scale, const float *gamma_row,
                 int64_t M, int64_t N, double *y)
{
    for (int64_t m = 0; m < M; m++)
        for (int64_t n = 0; n < N; n++)
            y[m * N + n] = (double)acc[m * N + n] * (double)scale[m] *
                           (double)gamma_row[n];
}

int orc_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------
 * Role-dependent projections: the OCP E4M3 format, the FP8 quantizers, the
 * fast (FP8) and critical (bf16) contractions.
 * ---------------------------------------------------------------------- */

/* Value of an E4M3 code as an integer multiple of 2^-9 (the smallest
 * subnormal), so that sums of products can be formed exactly in int64.
 * Normal codes: (1 + m/8) 2^(e-7) = (8 + m) 2^(e-10) = (8 + m) 2^(e-1) units;
 * subnormal codes (e == 0): (m/8) 2^-6 = m units.  Returns 0 for NaN codes
 * and sets *nan. */
static int64_t orc_e4m3_units(uint8_t c, int *nan)
{
    int e = (c >> 3) & 15, m = c & 7;
    int64_t v;
    if (e == 15 && m == 7) {
        *nan = 1;
        return 0;
    }
    v = e == 0 ? (int64_t)m : (int64_t)(8 + m) << (e - 1);
    return (c & 0x80) ? -v : v;
}

/* Decoded value (NaN for the two NaN codes). */
double orc_e4m3_decode(uint8_t c)
{
    int nan = 0;
    int64_t u = orc_e4m3_units(c, &nan);
    if (nan)
        return NAN;
    if (u == 0 && (c & 0x80))
        return -0.0;
    return ldexp((double)u, -9);
}

/* Round a finite fp32 value to E4M3, nearest with ties to even.  Returns
 * 0 and the code, or -1 if v is not finite or rounds beyond 448. */
int orc_e4m3_encode(float v, uint8_t *out)
{
    double a, q, r;
    int E = -6, ex;
    uint8_t c;
    if (!isfinite(v))
        return -1;
    a = fabs((double)v);
    /* spacing of the representable magnitudes: 2^-9 below 2^-6
     * (subnormals), 2^(E-3) within the binade [2^E, 2^(E+1)) */
    if (a >= ldexp(1.0, -6)) {
        frexp(a, &ex);
        E = ex - 1;
    }
    q = ldexp(1.0, E - 3);
    r = nearbyint(a / q) * q; /* a / q is exact; default mode: ties to even */
    if (r > 448.0)
        return -1;
    if (r < ldexp(1.0, -6)) {
        c = (uint8_t)(r / ldexp(1.0, -9)); /* 0 .. 7 */
    } else {
        double f = frexp(r, &ex); /* r = f 2^ex, f in [0.5, 1) */
        c = (uint8_t)(((ex - 1 + 7) << 3) | ((int)(f * 16.0) - 8));
    }
    *out = (uint8_t)((signbit(v) ? 0x80 : 0) | c);
    return 0;
}

/* Absmax FP8 quantization of one row of K fp32 values. */
static int orc_fp8_row(const float *x, int64_t K, uint8_t *codes, float *scale)
{
    float a = 0.0f, inv;
    for (int64_t k = 0; k < K; k++) {
        if (!isfinite(x[k]))
            return -1;
        if (fabsf(x[k]) > a)
            a = fabsf(x[k]);
    }
    if (a == 0.0f) {
        memset(codes, 0, (size_t)K);
        *scale = 0.0f;
        return 0;
    }
    inv = 448.0f / a;
    for (int64_t k = 0; k < K; k++) {
        float p = x[k] * inv;
        if (orc_e4m3_encode(p, &codes[k]) != 0)
            return -1;
    }
    *scale = a / 448.0f;
    return 0;
}

/* Per-output-row FP8 quantization of weights W[N][K] (fp32). */
int orc_quantize_fp8_rows(const float *W, int64_t N, int64_t K, uint8_t *codes,
                          float *scale)
{
    for (int64_t n = 0; n < N; n++)
        if (orc_fp8_row(W + n * K, K, codes + n * K, &scale[n]) != 0)
            return -1;
    return 0;
}

/* Per-token FP8 quantization of activations x[M][K] (bf16 bit patterns,
 * widened exactly to fp32 first). */
int orc_quantize_act_fp8(const uint16_t *x_bf16, int64_t M, int64_t K,
                         uint8_t *codes, float *scale)
{
    float row[8192];
    if (K > 8192)
        return -2;
    for (int64_t m = 0; m < M; m++) {
        for (int64_t k = 0; k < K; k++)
            row[k] = orc_bf16_to_float(x_bf16[m * K + k]);
        if (orc_fp8_row(row, K, codes + m * K, &scale[m]) != 0)
            return -1;
    }
    return 0;
}

/* Fast contraction: dot[m][n] = sum_k dec(xq[m][k]) dec(wq[n][k]), exact.
 * In units of 2^-9 each factor is an integer below 2^18 in magnitude, a
 * product below 2^36, and K <= 8192 products sum below 2^49: the int64 sum
 * is exact and so is its conversion to double (times 2^-18).  absdot is the
 * same sum over |products| (the scale of the rounding-error bound).
 * Returns -1 on a NaN code. */
int orc_fp8_linear(const uint8_t *xq, const uint8_t *wq, int64_t M, int64_t N,
                   int64_t K, double *dot, double *absdot)
{
    int nan = 0;
    for (int64_t m = 0; m < M; m++)
        for (int64_t n = 0; n < N; n++) {
            int64_t s = 0, sa = 0;
            for (int64_t k = 0; k < K; k++) {
                int64_t p = orc_e4m3_units(xq[m * K + k], &nan) *
                            orc_e4m3_units(wq[n * K + k], &nan);
                s += p;
                sa += p < 0 ? -p : p;
            }
            dot[m * N + n] = ldexp((double)s, -18);
            absdot[m * N + n] = ldexp((double)sa, -18);
        }
    return nan ? -1 : 0;
}

/* Critical contraction: dot[m][n] = sum_k x[m][k] w[n][k] over bf16 values,
 * accumulated in double (each product of two bf16 values is exact in double;
 * the sum's rounding error is at most K 2^-53 absdot). */
void orc_bf16_linear(const uint16_t *x, const uint16_t *w, int64_t M, int64_t N,
                     int64_t K, double *dot, double *absdot)
{
    for (int64_t m = 0; m < M; m++)
        for (int64_t n = 0; n < N; n++) {
            double s = 0.0, sa = 0.0;
            for (int64_t k = 0; k < K; k++) {
                double p = (double)orc_bf16_to_float(x[m * K + k]) *
                           (double)orc_bf16_to_float(w[n * K + k]);
                s += p;
                sa += fabs(p);
            }
            dot[m * N + n] = s;
            absdot[m * N + n] = sa;
        }
}
