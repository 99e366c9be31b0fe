/* Exercises every function of oracle.c on small seeded inputs and on the
 * edge cases (empty shapes, zero rows, ties, the invalid code, non-finite
 * input), for the AddressSanitizer / UndefinedBehaviorSanitizer build.
 * Test infrastructure only. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int orc_ternarize_absmean(const float *W, int64_t N, int64_t K, int8_t *t, float *gamma);
int orc_quantize_act(const uint16_t *x, int64_t M, int64_t K, int8_t *q, float *s);
int orc_unpack(const uint8_t *packed, int64_t N, int64_t K, int8_t *t);
void orc_linear(const int8_t *q, const int8_t *t, int64_t M, int64_t N, int64_t K, int32_t *acc,
                int threads);
void orc_dequant(const int32_t *acc, const float *s, const float *g, int64_t M, int64_t N,
                 double *y);
double orc_e4m3_decode(uint8_t c);
int orc_e4m3_encode(float v, uint8_t *out);
int orc_quantize_fp8_rows(const float *W, int64_t N, int64_t K, uint8_t *codes, float *s);
int orc_quantize_act_fp8(const uint16_t *x, int64_t M, int64_t K, uint8_t *codes, float *s);
int orc_fp8_linear(const uint8_t *xq, const uint8_t *wq, int64_t M, int64_t N, int64_t K,
                   double *dot, double *absdot);
void orc_bf16_linear(const uint16_t *x, const uint16_t *w, int64_t M, int64_t N, int64_t K,
                     double *dot, double *absdot);

static uint32_t rng = 12345u;
static float frand(void) {
    rng = rng * 1664525u + 1013904223u;
    return ((float)(rng >> 8) / 16777216.0f - 0.5f) * 4.0f;
}
static uint16_t bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

int main(void) {
    enum { M = 3, N = 7, K = 64 };
    float W[N * K];
    uint16_t x[M * K], wb[N * K];
    int8_t t[N * K], q[M * K];
    float s[M], g = 0.0f, grow[N];
    int32_t acc[M * N];
    double y[M * N], d[M * N], a[M * N];
    uint8_t packed[N * K / 4], wq[N * K], xq[M * K];
    float ws[N], xs[M];
    for (int i = 0; i < N * K; ++i) {
        W[i] = frand();
        wb[i] = bf16(W[i]);
    }
    for (int i = 0; i < M * K; ++i)
        x[i] = bf16(frand());
    for (int i = 0; i < K; ++i)
        x[K + i] = 0; /* a zero row */
    if (orc_ternarize_absmean(W, N, K, t, &g) != 0)
        return 1;
    if (orc_ternarize_absmean(W, 0, K, t, &g) != 0 || g != 0.0f)
        return 2;
    if (orc_quantize_act(x, M, K, q, s) != 0 || s[1] != 0.0f)
        return 3;
    for (int i = 0; i < N; ++i)
        grow[i] = 0.5f;
    orc_linear(q, t, M, N, K, acc, 1);
    orc_linear(q, t, M, N, K, acc, 2);
    orc_dequant(acc, s, grow, M, N, y);
    /* packed codes: every byte valid (fields 0..2), then one invalid field */
    for (int i = 0; i < N * K / 4; ++i)
        packed[i] = (uint8_t)(0x24 + (i % 3));
    if (orc_unpack(packed, N, K, t) != 0)
        return 4;
    packed[5] = 0xFF;
    if (orc_unpack(packed, N, K, t) != -1)
        return 5;
    for (int c = 0; c < 256; ++c)
        (void)orc_e4m3_decode((uint8_t)c);
    uint8_t code;
    if (orc_e4m3_encode(1.0f, &code) != 0 || orc_e4m3_encode(NAN, &code) == 0)
        return 6;
    if (orc_quantize_fp8_rows(W, N, K, wq, ws) != 0)
        return 7;
    if (orc_quantize_act_fp8(x, M, K, xq, xs) != 0)
        return 8;
    if (orc_fp8_linear(xq, wq, M, N, K, d, a) != 0)
        return 9;
    orc_bf16_linear(x, wb, M, N, K, d, a);
    W[3] = INFINITY;
    if (orc_ternarize_absmean(W, N, K, t, &g) == 0)
        return 10;
    puts("oracle driver: ok");
    return 0;
}
