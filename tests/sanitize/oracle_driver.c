/* Drives every function of the CPU oracle on small inputs and edge cases
 * (empty and ragged shapes, pad rows, row strides, every group size, both
 * input dtypes, producers, special values), built with the host compiler's
 * address and undefined-behaviour sanitizers.  Prints "oracle ok" and exits
 * 0 unless a call fails; a sanitizer report aborts it.  Test infrastructure. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int64_t oracle_packed_bytes(int64_t M, int64_t K);
int oracle_rotate_rows_f32(const float *X, int64_t M, int64_t K, int G, float *Y);
int oracle_rotate_rows_f64(const double *X, int64_t M, int64_t K, int G, double *Y);
int oracle_quantize_rows(const void *X, int x_dtype, int64_t M, int64_t K, int64_t ldx, int G, float alpha,
                         void *packed, int threads);
int oracle_modulate_rows(const void *X, int x_dtype, int64_t M, int64_t K, int64_t ldx, const float *scale,
                         const float *shift, float *Y, int threads);
int oracle_rmsnorm_rows(const void *X, int x_dtype, int64_t M, int64_t K, int64_t ldx, float eps,
                        const float *weight, float *Y, int threads);
float oracle_expf(float x);
int oracle_expf_array(const float *x, float *y, int64_t n, int threads);
int oracle_gated_act_rows(const void *X, int x_dtype, int64_t M, int64_t K, int64_t ldx, const void *U,
                          int64_t ldu, int act, float *Y, int threads);
int oracle_unpack_int4(const uint8_t *W4, int64_t N, int64_t K, int8_t *Qw);
int oracle_gated_residual(const float *Y, int64_t M, int64_t N, float scale, const float *gate,
                          const void *R, int r_dtype, int64_t ldr, int z_dtype, void *Z, int64_t ldz,
                          int threads);
int oracle_gemm_i32(const int8_t *Qx, const int8_t *Qw, int64_t M, int64_t K, int64_t N, int32_t *A,
                    int threads);
int oracle_epilogue(const int32_t *A, int64_t M, int64_t N, const float *s_x, const float *s_w,
                    const float *bias, float alpha, int y_dtype, void *Y, int64_t ldy, int threads);
int oracle_linear(const void *X, int x_dtype, int64_t M, int64_t K, int64_t ldx, int G, float alpha,
                  const int8_t *Qw, const float *s_w, const float *bias, int64_t N, void *Y, int y_dtype,
                  int64_t ldy, int threads);

static uint64_t state = 88172645463325252ull;
static double rnd(void)   /* xorshift64, uniform in [-1, 1) */
{
    state ^= state << 13;
    state ^= state >> 7;
    state ^= state << 17;
    return (double)(state >> 11) / 4503599627370496.0 - 1.0;
}

static int fails = 0;
#define OK(call)                                                       \
    do {                                                               \
        int rc_ = (call);                                              \
        if (rc_ != 0) {                                                \
            fprintf(stderr, "%s:%d: %s -> %d\n", __FILE__, __LINE__, #call, rc_); \
            ++fails;                                                   \
        }                                                              \
    } while (0)

int main(void)
{
    const int Gs[5] = {1, 4, 16, 64, 256};
    const int64_t shapes[][2] = {{1, 256}, {3, 256}, {5, 512}, {7, 1024}, {0, 256}};
    for (size_t si = 0; si < sizeof shapes / sizeof shapes[0]; ++si) {
        const int64_t M = shapes[si][0], K = shapes[si][1], ldx = K + 64, N = 37;
        float *X = malloc(sizeof(float) * (size_t)(M > 0 ? M : 1) * ldx);
        uint16_t *Xb = malloc(sizeof(uint16_t) * (size_t)(M > 0 ? M : 1) * ldx);
        for (int64_t i = 0; i < M * ldx; ++i) {
            X[i] = (float)(rnd() * (i % 97 == 0 ? 40.0 : 1.0));
            uint32_t u;
            memcpy(&u, &X[i], 4);
            Xb[i] = (uint16_t)(u >> 16);
        }
        if (M > 0)
            memset(X + (M - 1) * ldx, 0, sizeof(float) * (size_t)K);    /* a zero row */
        const int64_t pb = oracle_packed_bytes(M, K);
        uint8_t *packed = malloc((size_t)(pb > 0 ? pb : 1));
        int8_t *Qw = malloc((size_t)(N * K));
        float *sw = malloc(sizeof(float) * (size_t)N), *b = malloc(sizeof(float) * (size_t)N);
        for (int64_t i = 0; i < N * K; ++i)
            Qw[i] = (int8_t)(int)(rnd() * 127.0);
        for (int64_t i = 0; i < N; ++i) {
            sw[i] = (float)(0.01 + 0.005 * rnd());
            b[i] = (float)(0.1 * rnd());
        }
        float *Y = malloc(sizeof(float) * (size_t)(M > 0 ? M : 1) * (N + 3));
        for (int g = 0; g < 5; ++g) {
            OK(oracle_quantize_rows(X, 0, M, K, ldx, Gs[g], 1.0f, packed, 2));
            OK(oracle_quantize_rows(Xb, 1, M, K, ldx, Gs[g], 0.3f, packed, 1));
            OK(oracle_linear(X, 0, M, K, ldx, Gs[g], 0.5f, Qw, sw, b, N, Y, 0, N + 3, 2));
            OK(oracle_linear(Xb, 1, M, K, ldx, Gs[g], 1.0f, Qw, NULL, NULL, N, Y, 1, N + 3, 1));
        }
        if (M > 0) {
            float *Xr = malloc(sizeof(float) * (size_t)M * K);
            double *Xd = malloc(sizeof(double) * (size_t)M * K), *Yd = malloc(sizeof(double) * (size_t)M * K);
            for (int64_t i = 0; i < M * K; ++i)
                Xd[i] = rnd();
            OK(oracle_rotate_rows_f32(X, M, K, 256, Xr));
            OK(oracle_rotate_rows_f64(Xd, M, K, 64, Yd));
            float *sc = malloc(sizeof(float) * (size_t)K), *sh = malloc(sizeof(float) * (size_t)K);
            for (int64_t i = 0; i < K; ++i) {
                sc[i] = (float)(0.3 * rnd());
                sh[i] = (float)(0.3 * rnd());
            }
            OK(oracle_modulate_rows(Xb, 1, M, K, ldx, sc, sh, Xr, 2));
            OK(oracle_modulate_rows(X, 0, M, K, ldx, sc, NULL, Xr, 1));
            OK(oracle_rmsnorm_rows(X, 0, M, K, ldx, 1e-6f, sc, Xr, 2));
            OK(oracle_rmsnorm_rows(Xb, 1, M, K, ldx, 0.0f, NULL, Xr, 1));
            OK(oracle_gated_act_rows(X, 0, M, K, ldx, X, ldx, 1, Xr, 2));
            OK(oracle_gated_act_rows(Xb, 1, M, K, ldx, Xb, ldx, 2, Xr, 1));
            int32_t *A = malloc(sizeof(int32_t) * (size_t)M * N);
            OK(oracle_gemm_i32((const int8_t *)packed, Qw, M, K, N, A, 2));
            const int64_t m_pad = (M + 3) / 4 * 4;
            const float *s_x = (const float *)(packed + m_pad * K);
            OK(oracle_epilogue(A, M, N, s_x, sw, b, 0.3f, 1, Y, N + 3, 2));
            float *gate = malloc(sizeof(float) * (size_t)N);
            for (int64_t i = 0; i < N; ++i)
                gate[i] = (float)rnd();
            float *Yf = malloc(sizeof(float) * (size_t)M * N);
            OK(oracle_epilogue(A, M, N, s_x, sw, b, 1.0f, 0, Yf, N, 1));
            uint16_t *Zb = malloc(sizeof(uint16_t) * (size_t)M * (N + 5));
            OK(oracle_gated_residual(Yf, M, N, 0.37f, gate, Y, 0, N + 3, 1, Zb, N + 5, 2));
            OK(oracle_gated_residual(Yf, M, N, 1.0f, gate, Zb, 1, N + 5, 0, Y, N + 3, 1));
            free(Zb);
            uint8_t *W4 = malloc((size_t)(N * K / 2));
            for (int64_t i = 0; i < N * K / 2; ++i)
                W4[i] = (uint8_t)(i * 37 + 11);
            OK(oracle_unpack_int4(W4, N, K, Qw));
            free(W4);
            free(Yf);
            free(gate);
            free(A);
            free(sc);
            free(sh);
            free(Xd);
            free(Yd);
            free(Xr);
        }
        free(X);
        free(Xb);
        free(packed);
        free(Qw);
        free(sw);
        free(b);
        free(Y);
    }
    const float specials[] = {0.0f, -0.0f, 1e-30f, -104.5f, -87.0f, 88.7f, 89.5f, 1.0f, -1.0f, 3.0e38f};
    float e[10];
    for (int i = 0; i < 10; ++i)
        (void)oracle_expf(specials[i]);
    OK(oracle_expf_array(specials, e, 10, 2));
    if (fails) {
        fprintf(stderr, "%d call(s) failed\n", fails);
        return 1;
    }
    printf("oracle ok\n");
    return 0;
}
