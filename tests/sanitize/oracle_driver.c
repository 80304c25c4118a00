/* The oracle's C functions under AddressSanitizer and
 * UndefinedBehaviorSanitizer: plans over a grid of shapes, the bf16
 * conversions over every bit pattern, 4-bit dequantisation, the naive GEMM
 * and its sampled form, and the ordered sums, on small inputs, with cross
 * checks (sampled GEMM = full GEMM; row shards' partials add up to the full
 * product).  Exits 0 when every check holds. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_plan(int32_t hidden, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                int32_t ffn, int32_t tp, int32_t group, int64_t *out, int64_t out_len);
int oracle_plan_linear(int64_t K, int64_t N, int32_t tp, int32_t strategy, int32_t group,
                       int64_t *out, int64_t out_len);
int oracle_plan_vocab(int64_t vocab, int64_t hidden, int32_t tp, int32_t group, int64_t *out,
                      int64_t out_len);
int64_t oracle_plan_experts(int32_t n_experts, int64_t hidden, int64_t ffn, int32_t tp,
                            int32_t mode, int32_t group, int64_t *out, int64_t out_len);
void oracle_bf16_to_f64(const uint16_t *in, double *out, int64_t n);
void oracle_f64_to_bf16_rne(const double *in, uint16_t *out, int64_t n);
void oracle_dequant_q4(const uint8_t *codes, const uint16_t *scales, const uint16_t *biases,
                       int64_t K, int64_t N, int64_t group, double *W);
void oracle_gemm(const double *X, const double *W, double *Y, int64_t M, int64_t K, int64_t N);
void oracle_gemm_at(const double *X, const double *W, int64_t K, int64_t N, const int64_t *rows,
                    const int64_t *cols, int64_t count, double *out);
void oracle_sum(const double *P, int64_t R, int64_t count, double *Y);
void oracle_sum_f32_seq(const float *P, int64_t R, int64_t count, float *Y);

static int failures;
#define EXPECT(c)                                                                                  \
    do {                                                                                           \
        if (!(c)) {                                                                                \
            fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, #c);                                \
            ++failures;                                                                            \
        }                                                                                          \
    } while (0)

static uint32_t lcg = 7;
static double rnd(void)
{
    lcg = lcg * 1664525u + 1013904223u;
    return (double)(lcg >> 8) / 16777216.0 - 0.5;
}

int main(void)
{
    /* plans */
    int64_t rec[16 * 7 * 12];
    for (int tp = 1; tp <= 16; ++tp)
        for (int hkv = 1; hkv <= 8; hkv *= 2) {
            int st = oracle_plan(512, 8, hkv, 64, 1024, tp, (tp & 1) ? 0 : 64, rec,
                                 (int64_t)(sizeof rec / sizeof rec[0]));
            (void)st;
        }
    EXPECT(oracle_plan(512, 8, 2, 64, 1024, 4, 0, rec, 4 * 7 * 12 - 1) != 0);
    EXPECT(oracle_plan_linear(1024, 2048, 2, 0, 0, rec, 2 * 12) == 0);
    EXPECT(oracle_plan_vocab(1024, 256, 4, 64, rec, 8 * 12) == 0);
    {
        int64_t *ex = malloc(sizeof(int64_t) * 64 * 4 * 40);
        EXPECT(oracle_plan_experts(64, 256, 128, 4, 0, 64, ex, 64 * 4 * 40) > 0);
        EXPECT(oracle_plan_experts(64, 256, 256, 4, 1, 64, ex, 64 * 4 * 40) > 0);
        free(ex);
    }
    /* bf16 conversions over every bit pattern, and back */
    {
        uint16_t *b = malloc(65536 * sizeof *b), *b2 = malloc(65536 * sizeof *b2);
        double *d = malloc(65536 * sizeof *d);
        for (int i = 0; i < 65536; ++i)
            b[i] = (uint16_t)i;
        oracle_bf16_to_f64(b, d, 65536);
        oracle_f64_to_bf16_rne(d, b2, 65536);
        for (int i = 0; i < 65536; ++i)
            if (!isnan(d[i]))
                EXPECT(b2[i] == b[i]);
        free(b);
        free(b2);
        free(d);
    }
    /* dequantise, multiply, sample, sum */
    {
        enum { M = 5, K = 128, N = 7, G = 64 };
        uint8_t codes[K * N];
        uint16_t sc[(K / G) * N], bi[(K / G) * N];
        double W[K * N], X[M * K], Y[M * N], Yh[2][M * N], Ysum[M * N];
        for (int i = 0; i < K * N; ++i)
            codes[i] = (uint8_t)((lcg = lcg * 1664525u + 1013904223u) >> 28);
        for (int i = 0; i < (K / G) * N; ++i) {
            double s = 0.01 + 0.01 * (rnd() + 0.5), b = 0.05 * rnd();
            oracle_f64_to_bf16_rne(&s, &sc[i], 1);
            oracle_f64_to_bf16_rne(&b, &bi[i], 1);
        }
        for (int i = 0; i < M * K; ++i)
            X[i] = rnd();
        oracle_dequant_q4(codes, sc, bi, K, N, G, W);
        oracle_gemm(X, W, Y, M, K, N);
        int64_t rows[M * N], cols[M * N];
        double s[M * N];
        for (int i = 0; i < M * N; ++i) {
            rows[i] = i / N;
            cols[i] = i % N;
        }
        oracle_gemm_at(X, W, K, N, rows, cols, M * N, s);
        for (int i = 0; i < M * N; ++i)
            EXPECT(fabs(s[i] - Y[i]) <= 1e-12 * (1.0 + fabs(Y[i])));
        /* two row shards of k: X[:, half] W[half, :], summed */
        for (int h = 0; h < 2; ++h) {
            double Xh[M * (K / 2)];
            for (int m = 0; m < M; ++m)
                memcpy(&Xh[m * (K / 2)], &X[m * K + h * (K / 2)], sizeof(double) * (K / 2));
            oracle_gemm(Xh, &W[h * (K / 2) * N], Yh[h], M, K / 2, N);
        }
        oracle_sum(&Yh[0][0], 2, M * N, Ysum);
        for (int i = 0; i < M * N; ++i)
            EXPECT(fabs(Ysum[i] - Y[i]) <= 1e-12 * (1.0 + fabs(Y[i])));
        float pf[3 * 4] = {1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12}, yf[4];
        oracle_sum_f32_seq(pf, 3, 4, yf);
        EXPECT(yf[0] == 15.0f && yf[3] == 24.0f);
    }
    if (failures)
        fprintf(stderr, "%d checks failed\n", failures);
    else
        printf("oracle driver: all checks passed\n");
    return failures ? 1 : 0;
}
