/*
 * CPU oracle for the INT8 convrot linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow reference that the
 * HIP path is checked against.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load it; the product library never links,
 * calls or falls back to it, and the two share no code.
 *
 * Source of truth: the "INT8 Convrot Safetensors" page (sd.cpp
 * docs/int8_convrot.md), section "How INT8 convrot works" and its
 * subsections "Weight quantization" and "Runtime activation quantization";
 * and the "ggml operator extensions" page (sd.cpp docs/ggml_extensions.md),
 * section "sd.cpp integration" (reconstruction order, packed ConvRot layout).
 *
 * Every floating-point step is one IEEE-754 binary32 operation rounded to
 * nearest-even, in the order written.  Build with -ffp-contract=off and
 * without -ffast-math (x86-64 SSE evaluates float expressions in float).
 *
 * Readings where the pages leave a detail open (each is also listed in the
 * design notes):
 *   - rotation order: H4 is applied along base-4 digit 0 first (stride 1),
 *     then digit 1 (stride 4), ...; each 4-point application computes
 *     s = (x0 + x1) + (x2 + x3), h = s * 0.5, y_j = h - x_{3-j}.
 *   - "round" is round-half-to-even (rintf in the default rounding mode).
 *   - "X_rot / s" is evaluated as X_rot * fl(127 / max): one correctly
 *     rounded reciprocal per row, then a product per element.  The stored
 *     scale is still fl(max / 127).
 *   - an all-zero row gets scale 0 and codes 0.
 *   - the packed tensor is int8 [M_pad][K] (M_pad = M rounded up to a
 *     multiple of 4, pad rows zero) followed by float [M_pad] (pad zero).
 *   - the per-linear input scale alpha pre-multiplies the activation (one
 *     rounding) and divides the output after the weight scale, before bias.
 *   - packed 4-bit weights (page "INT8 Convrot Safetensors", section
 *     "Packed INT4 convrot", format convrot_w4a4): two signed 4-bit values per
 *     byte, the low nibble holding the even input feature; they are decoded
 *     to int8 and then take the same contraction and reconstruction as INT8
 *     weights (the activations use the INT8 convrot quantization unchanged).
 *   - the gated-residual epilogue (page "ggml operator extensions", section
 *     "sd.cpp integration": INT8 GEMM -> [Scale] -> Mul(gate) -> Add(residual))
 *     continues from the binary32 reconstruction: an optional scalar scale,
 *     then a per-channel gate vector of length N shared by every row, then a
 *     residual of the output's shape and dtype, each a separately rounded
 *     binary32 operation; the result takes the output cast.
 *   - the Modulate producer (page "ggml operator extensions", section
 *     "sd.cpp integration", the Modulate operator and its ConvRot fusion) is
 *     applied to the widened binary32 input with per-channel vectors of
 *     length K shared by every row: (x + x * scale) + shift, three separately
 *     rounded operations, the shift being optional.  Its binary32 output is
 *     the input of the quantizer above.
 *   - RMSNorm -> Mul(weight) ahead of the Modulate producer (same page and
 *     section, the RMSNorm -> Mul(weight) -> Mul(modulation) -> Add ->
 *     Add(shift) -> ConvRot fusion; the page does not spell out RMSNorm's
 *     arithmetic): per row, the squares fl(x * x) are summed pairwise within
 *     each block of 64 consecutive features (adjacent pairs, then pairs of
 *     those sums, ...) and the K/64 block sums are added left to right; then
 *     mean = fl(S / K), d = fl(sqrt(fl(mean + eps))), r = fl(1 / d) (each
 *     correctly rounded), y = fl(x * r) and, with a weight, fl(y * w[i]).
 *   - Norm -> Mul(weight) ahead of the quantizer (same page and section, the
 *     Norm -> Mul -> ConvRot fusion; the page names the chain only): Norm is
 *     the normalization by mean and variance with no affine part, and Mul
 *     multiplies by a weight vector of length K shared by every row, as in
 *     the RMSNorm chain.  Per row, the features x are summed in the tree
 *     above (pairwise within 64-feature blocks, block sums left to right),
 *     mean = fl(S1 / K); then the deviations d = fl(x - mean) give
 *     fl(d * d), summed in the same tree, var = fl(S2 / K),
 *     r = fl(1 / fl(sqrt(fl(var + eps)))) (correctly rounded), y = fl(d * r)
 *     and, with a weight, fl(y * w[i]).
 *   - the gated activation ahead of the quantizer (same page and section:
 *     SiLU/Sigmoid -> Mul -> ConvRot, and SwiGLU -> ConvRot with its gate and
 *     up halves): z = fl(act(g) * u) with g the quantizer's input and u a
 *     second tensor of the same shape; sigmoid(g) = fl(1 / fl(1 + e)) with
 *     e = exp(-g) correctly rounded to binary32, and silu(g) =
 *     fl(g * sigmoid(g)).  exp is evaluated in x87 extended precision
 *     (64-bit significand, error a few units in 2^-64) and rounded once to
 *     binary32: the binary32 arguments whose exp lies closest to a binary32
 *     rounding boundary are still far above that error, so the result is the
 *     correctly rounded exp.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)
#define ORACLE_EUNSUPPORTED (-2)
#define ORACLE_EOVERFLOW (-3)

#define ORACLE_F32 0
#define ORACLE_BF16 1

/* G must be a power of four (4^0 = 1 allowed) dividing K: the page's checkpoint
 * format section states the group size rule. */
static int group_size_ok(int64_t K, int G)
{
    if (G < 1 || K < 1 || K % G != 0)
        return 0;
    int g = G;
    while (g > 1) {
        if (g % 4 != 0)
            return 0;
        g /= 4;
    }
    return 1;
}

int64_t oracle_packed_bytes(int64_t M, int64_t K)
{
    int64_t m_pad = (M + 3) / 4 * 4;
    return m_pad * K + 4 * m_pad;
}

/* ---------------------------------------------------------------- rotation */

/*
 * One application of H4 along base-4 digit k (stride st = 4^k) of a G-element
 * group.  H4 = [[1,1,1,-1],[1,1,-1,1],[1,-1,1,1],[-1,1,1,1]] / 2 (page "How
 * INT8 convrot works"): row j is 1/2 everywhere except -1/2 in column 3-j, so
 * (H4 x)_j = (x0 + x1 + x2 + x3) / 2 - x_{3-j}.
 */
static void h4_stage_f32(float *g, int G, int st)
{
    for (int i = 0; i < G; ++i) {
        if ((i / st) % 4 != 0)
            continue;
        float x0 = g[i], x1 = g[i + st], x2 = g[i + 2 * st], x3 = g[i + 3 * st];
        float s = (x0 + x1) + (x2 + x3);
        float h = s * 0.5f;
        g[i] = h - x3;
        g[i + st] = h - x2;
        g[i + 2 * st] = h - x1;
        g[i + 3 * st] = h - x0;
    }
}

/* R_G = H4 (x) H4 (x) ... (x) H4 (n factors, G = 4^n): one H4 stage per digit. */
static void rotate_group_f32(float *g, int G)
{
    for (int st = 1; st < G; st *= 4)
        h4_stage_f32(g, G, st);
}

static void h4_stage_f64(double *g, int G, int st)
{
    for (int i = 0; i < G; ++i) {
        if ((i / st) % 4 != 0)
            continue;
        double x0 = g[i], x1 = g[i + st], x2 = g[i + 2 * st], x3 = g[i + 3 * st];
        double s = (x0 + x1) + (x2 + x3);
        double h = s * 0.5;
        g[i] = h - x3;
        g[i + st] = h - x2;
        g[i + 2 * st] = h - x1;
        g[i + 3 * st] = h - x0;
    }
}

static void rotate_group_f64(double *g, int G)
{
    for (int st = 1; st < G; st *= 4)
        h4_stage_f64(g, G, st);
}

/* Y = X R: the group rotation of every row (X, Y contiguous [M][K] fp32). */
int oracle_rotate_rows_f32(const float *X, int64_t M, int64_t K, int G, float *Y)
{
    if (!X || !Y || M < 0)
        return ORACLE_EINVAL;
    if (!group_size_ok(K, G))
        return ORACLE_EUNSUPPORTED;
    memmove(Y, X, (size_t)(M * K) * sizeof(float));
    for (int64_t r = 0; r < M; ++r)
        for (int64_t g0 = 0; g0 < K; g0 += G)
            rotate_group_f32(Y + r * K + g0, G);
    return ORACLE_OK;
}

/* The same rotation carried out in binary64 (for the exact-identity checks). */
int oracle_rotate_rows_f64(const double *X, int64_t M, int64_t K, int G, double *Y)
{
    if (!X || !Y || M < 0)
        return ORACLE_EINVAL;
    if (!group_size_ok(K, G))
        return ORACLE_EUNSUPPORTED;
    memmove(Y, X, (size_t)(M * K) * sizeof(double));
    for (int64_t r = 0; r < M; ++r)
        for (int64_t g0 = 0; g0 < K; g0 += G)
            rotate_group_f64(Y + r * K + g0, G);
    return ORACLE_OK;
}

/* ------------------------------------------------------------ quantization */

static float load_widened(const void *X, int dtype, int64_t idx)
{
    if (dtype == ORACLE_F32)
        return ((const float *)X)[idx];
    /* bf16 is the upper half of a binary32: widening is exact. */
    uint32_t u = (uint32_t)((const uint16_t *)X)[idx] << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/*
 * One activation row, page "Runtime activation quantization":
 *   x = widen(X[r, :]);  x *= alpha (only when alpha != 1);
 *   y = rotate each contiguous G-group;
 *   m = max_i |y_i| over the whole row;
 *   s = m / 127;  q_i = clamp(round(y_i / s), -127, 127)   (see readings above).
 */
static void quantize_one_row(const void *X, int dtype, int64_t row_off, int64_t K, int G,
                             float alpha, float *y, int8_t *q, float *s_out)
{
    for (int64_t i = 0; i < K; ++i)
        y[i] = load_widened(X, dtype, row_off + i);
    if (alpha != 1.0f)
        for (int64_t i = 0; i < K; ++i)
            y[i] = y[i] * alpha;
    for (int64_t g0 = 0; g0 < K; g0 += G)
        rotate_group_f32(y + g0, G);

    float m = 0.0f;
    for (int64_t i = 0; i < K; ++i) {
        float a = fabsf(y[i]);
        if (a > m)
            m = a;
    }
    if (m == 0.0f) {
        *s_out = 0.0f;
        memset(q, 0, (size_t)K);
        return;
    }
    *s_out = m / 127.0f;
    float inv = 127.0f / m;
    for (int64_t i = 0; i < K; ++i) {
        float t = rintf(y[i] * inv);
        if (t > 127.0f)
            t = 127.0f;
        if (t < -127.0f)
            t = -127.0f;
        q[i] = (int8_t)t;
    }
}

/*
 * Quantize M rows of X (row stride ldx elements) into the packed tensor:
 * int8 [M_pad][K] codes followed by float [M_pad] row scales.
 */
int oracle_quantize_rows(const void *X, int x_dtype, int64_t M, int64_t K, int64_t ldx, int G,
                         float alpha, uint8_t *packed, int threads)
{
    if (!X || !packed || M < 0 || ldx < K)
        return ORACLE_EINVAL;
    if (x_dtype != ORACLE_F32 && x_dtype != ORACLE_BF16)
        return ORACLE_EUNSUPPORTED;
    if (!group_size_ok(K, G))
        return ORACLE_EUNSUPPORTED;
    if (!(alpha > 0.0f) || isinf(alpha))
        return ORACLE_EINVAL;
    int64_t m_pad = (M + 3) / 4 * 4;
    int8_t *Q = (int8_t *)packed;
    uint8_t *tail = packed + m_pad * K;
    int failed = 0;

#pragma omp parallel num_threads(threads > 0 ? threads : 1)
    {
        float *y = (float *)malloc((size_t)K * sizeof(float));
        if (!y) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(static)
        for (int64_t r = 0; r < m_pad; ++r) {
            float s = 0.0f;
            if (r < M && y)
                quantize_one_row(X, x_dtype, r * ldx, K, G, alpha, y, Q + r * K, &s);
            else
                memset(Q + r * K, 0, (size_t)K);
            memcpy(tail + 4 * r, &s, sizeof s);
        }
        free(y);
    }
    return failed ? ORACLE_EINVAL : ORACLE_OK;
}

/* ---------------------------------------------------------------- producer */

/*
 * Modulate (page "ggml operator extensions", section "sd.cpp integration"):
 * Y[r, i] = (x + x * scale[i]) + shift[i] with x = widen(X[r, i]); shift may
 * be NULL (scale-only modulation).  Y is binary32 [M][K], contiguous.
 */
int oracle_modulate_rows(const void *X, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                         const float *scale, const float *shift, float *Y, int threads)
{
    if (!X || !scale || !Y || M < 0 || K < 1 || ldx < K)
        return ORACLE_EINVAL;
    if (x_dtype != ORACLE_F32 && x_dtype != ORACLE_BF16)
        return ORACLE_EUNSUPPORTED;
#pragma omp parallel for schedule(static) num_threads(threads > 0 ? threads : 1)
    for (int64_t r = 0; r < M; ++r) {
        for (int64_t i = 0; i < K; ++i) {
            const float x = load_widened(X, x_dtype, r * ldx + i);
            const float xs = x * scale[i];
            float y = x + xs;
            if (shift)
                y = y + shift[i];
            Y[r * K + i] = y;
        }
    }
    return ORACLE_OK;
}

/*
 * RMSNorm -> Mul(weight) (page "ggml operator extensions", section "sd.cpp
 * integration", the fusion chain that starts RMSNorm -> Mul(weight) and ends
 * in ConvRot), in the reading stated at the top of this file.  weight may be
 * NULL (no multiplication).  K must be a multiple of 64.  Y is binary32
 * [M][K], contiguous.
 */
static float pairwise_sum64(const float *q)
{
    float t[64];
    memcpy(t, q, sizeof t);
    for (int n = 64; n > 1; n /= 2)
        for (int i = 0; i < n / 2; ++i)
            t[i] = t[2 * i] + t[2 * i + 1];
    return t[0];
}

int oracle_rmsnorm_rows(const void *X, int x_dtype, int64_t M, int64_t K, int64_t ldx, float eps,
                        const float *weight, float *Y, int threads)
{
    if (!X || !Y || M < 0 || K < 64 || K % 64 != 0 || ldx < K || !(eps >= 0.0f) || isinf(eps))
        return ORACLE_EINVAL;
    if (x_dtype != ORACLE_F32 && x_dtype != ORACLE_BF16)
        return ORACLE_EUNSUPPORTED;
#pragma omp parallel for schedule(static) num_threads(threads > 0 ? threads : 1)
    for (int64_t r = 0; r < M; ++r) {
        float sq[64];
        float S = 0.0f;
        for (int64_t b = 0; b < K; b += 64) {
            for (int i = 0; i < 64; ++i) {
                const float x = load_widened(X, x_dtype, r * ldx + b + i);
                sq[i] = x * x;
            }
            const float block = pairwise_sum64(sq);
            S = b == 0 ? block : S + block;
        }
        const float mean = S / (float)K;
        const float d = sqrtf(mean + eps);
        const float rs = 1.0f / d;
        for (int64_t i = 0; i < K; ++i) {
            float y = load_widened(X, x_dtype, r * ldx + i) * rs;
            if (weight)
                y = y * weight[i];
            Y[r * K + i] = y;
        }
    }
    return ORACLE_OK;
}

/*
 * Norm -> Mul(weight) (page "ggml operator extensions", section "sd.cpp
 * integration", the Norm -> Mul -> ConvRot fusion), in the reading stated at
 * the top of this file: the row mean, then the mean of the squared
 * deviations, both summed in RMSNorm's tree.  weight may be NULL (no
 * multiplication).  K must be a multiple of 64.  Y is binary32 [M][K],
 * contiguous.
 */
int oracle_norm_rows(const void *X, int x_dtype, int64_t M, int64_t K, int64_t ldx, float eps,
                     const float *weight, float *Y, int threads)
{
    if (!X || !Y || M < 0 || K < 64 || K % 64 != 0 || ldx < K || !(eps >= 0.0f) || isinf(eps))
        return ORACLE_EINVAL;
    if (x_dtype != ORACLE_F32 && x_dtype != ORACLE_BF16)
        return ORACLE_EUNSUPPORTED;
#pragma omp parallel for schedule(static) num_threads(threads > 0 ? threads : 1)
    for (int64_t r = 0; r < M; ++r) {
        float t[64];
        float S1 = 0.0f;
        for (int64_t b = 0; b < K; b += 64) {
            for (int i = 0; i < 64; ++i)
                t[i] = load_widened(X, x_dtype, r * ldx + b + i);
            const float block = pairwise_sum64(t);
            S1 = b == 0 ? block : S1 + block;
        }
        const float mean = S1 / (float)K;
        float S2 = 0.0f;
        for (int64_t b = 0; b < K; b += 64) {
            for (int i = 0; i < 64; ++i) {
                const float dv = load_widened(X, x_dtype, r * ldx + b + i) - mean;
                t[i] = dv * dv;
            }
            const float block = pairwise_sum64(t);
            S2 = b == 0 ? block : S2 + block;
        }
        const float var = S2 / (float)K;
        const float sd = sqrtf(var + eps);
        const float rs = 1.0f / sd;
        for (int64_t i = 0; i < K; ++i) {
            const float dv = load_widened(X, x_dtype, r * ldx + i) - mean;
            float y = dv * rs;
            if (weight)
                y = y * weight[i];
            Y[r * K + i] = y;
        }
    }
    return ORACLE_OK;
}

/*
 * exp(x) rounded once to binary32 from x87 extended precision (the reading
 * stated at the top of this file).
 */
float oracle_expf(float x)
{
    return (float)expl((long double)x);
}

/* oracle_expf over n values (for checking other builds of exp in bulk). */
int oracle_expf_array(const float *x, float *y, int64_t n, int threads)
{
    if (n < 0 || (n > 0 && (!x || !y)))
        return ORACLE_EINVAL;
#pragma omp parallel for schedule(static) num_threads(threads > 0 ? threads : 1)
    for (int64_t i = 0; i < n; ++i)
        y[i] = oracle_expf(x[i]);
    return ORACLE_OK;
}

#define ORACLE_ACT_SILU 1
#define ORACLE_ACT_SIGMOID 2

/*
 * The gated activation (page "ggml operator extensions", section "sd.cpp
 * integration": SiLU/Sigmoid -> Mul -> ConvRot and SwiGLU -> ConvRot), in the
 * reading stated at the top of this file: Y[r, i] = fl(act(g) * u) with
 * g = widen(X[r, i]) and u = widen(U[r, i]) (both of dtype x_dtype, row
 * strides ldx and ldu).  Y is binary32 [M][K], contiguous.
 */
int oracle_gated_act_rows(const void *X, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                          const void *U, int64_t ldu, int act, float *Y, int threads)
{
    if (!X || !U || !Y || M < 0 || K < 1 || ldx < K || ldu < K)
        return ORACLE_EINVAL;
    if ((x_dtype != ORACLE_F32 && x_dtype != ORACLE_BF16) ||
        (act != ORACLE_ACT_SILU && act != ORACLE_ACT_SIGMOID))
        return ORACLE_EUNSUPPORTED;
#pragma omp parallel for schedule(static) num_threads(threads > 0 ? threads : 1)
    for (int64_t r = 0; r < M; ++r) {
        for (int64_t i = 0; i < K; ++i) {
            const float g = load_widened(X, x_dtype, r * ldx + i);
            const float u = load_widened(U, x_dtype, r * ldu + i);
            const float e = oracle_expf(-g);
            const float d = 1.0f + e;
            const float sg = 1.0f / d;
            const float a = act == ORACLE_ACT_SILU ? g * sg : sg;
            Y[r * K + i] = a * u;
        }
    }
    return ORACLE_OK;
}

/* ---------------------------------------------------------- 4-bit weights */

/*
 * convrot_w4a4 weights (page "INT8 Convrot Safetensors", section "Packed INT4
 * convrot"): W4 is [N][K/2] bytes; feature k of output o sits in byte
 * o * K/2 + k/2, in the low nibble when k is even and the high nibble when k
 * is odd, as a two's-complement 4-bit value (-8 .. 7).  Writes int8 [N][K].
 */
int oracle_unpack_int4(const uint8_t *W4, int64_t N, int64_t K, int8_t *Qw)
{
    if (!W4 || !Qw || N < 0 || K < 2 || K % 2 != 0)
        return ORACLE_EINVAL;
    for (int64_t o = 0; o < N; ++o) {
        for (int64_t k = 0; k < K; ++k) {
            const uint8_t byte = W4[o * (K / 2) + k / 2];
            const int nib = (k % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
            Qw[o * K + k] = (int8_t)(nib >= 8 ? nib - 16 : nib);
        }
    }
    return ORACLE_OK;
}

/* ------------------------------------------------------------- contraction */

/*
 * A[r, o] = sum_i Q_x[r, i] * Q_w[o, i]  (page "Runtime activation
 * quantization": signed 32-bit accumulation).  Accumulated in int64; returns
 * ORACLE_EOVERFLOW if any result does not fit int32 (it is then truncated).
 */
int oracle_gemm_i32(const int8_t *Qx, const int8_t *Qw, int64_t M, int64_t K, int64_t N,
                    int32_t *A, int threads)
{
    if (!Qx || !Qw || !A || M < 0 || N < 0 || K < 0)
        return ORACLE_EINVAL;
    int overflow = 0;
#pragma omp parallel for schedule(static) num_threads(threads > 0 ? threads : 1)
    for (int64_t r = 0; r < M; ++r) {
        for (int64_t o = 0; o < N; ++o) {
            int64_t acc = 0;
            for (int64_t i = 0; i < K; ++i)
                acc += (int64_t)Qx[r * K + i] * (int64_t)Qw[o * K + i];
            if (acc > INT32_MAX || acc < INT32_MIN) {
#pragma omp atomic write
                overflow = 1;
            }
            A[r * N + o] = (int32_t)acc;
        }
    }
    return overflow ? ORACLE_EOVERFLOW : ORACLE_OK;
}

/* ---------------------------------------------------------- reconstruction */

static uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/*
 * Y[r, o] = float(A[r, o]) * s_x[r] * s_w[o] / alpha + b[o], each operation
 * rounded separately and in that order (the operator-extensions page states
 * the order for the INT8 GEMM; the convrot page adds the unscale before the
 * bias for input scales other than 1).  s_w and bias may be NULL (1 and 0).
 * Output fp32, or bf16 rounded to nearest-even from the fp32 result.
 */
int oracle_epilogue(const int32_t *A, int64_t M, int64_t N, const float *s_x, const float *s_w,
                    const float *bias, float alpha, int y_dtype, void *Y, int64_t ldy, int threads)
{
    if (!A || !s_x || !Y || M < 0 || N < 0 || ldy < N)
        return ORACLE_EINVAL;
    if (y_dtype != ORACLE_F32 && y_dtype != ORACLE_BF16)
        return ORACLE_EUNSUPPORTED;
    if (!(alpha > 0.0f) || isinf(alpha))
        return ORACLE_EINVAL;
#pragma omp parallel for schedule(static) num_threads(threads > 0 ? threads : 1)
    for (int64_t r = 0; r < M; ++r) {
        for (int64_t o = 0; o < N; ++o) {
            float t = (float)A[r * N + o];
            t = t * s_x[r];
            if (s_w)
                t = t * s_w[o];
            if (alpha != 1.0f)
                t = t / alpha;
            if (bias)
                t = t + bias[o];
            if (y_dtype == ORACLE_F32)
                ((float *)Y)[r * ldy + o] = t;
            else
                ((uint16_t *)Y)[r * ldy + o] = f32_to_bf16_rne(t);
        }
    }
    return ORACLE_OK;
}

/* ----------------------------------------------------------- whole linear */

/* --------------------------------------------------------- gated residual */

/*
 * Z[r, o] = cast(fl(fl(fl(Y[r, o] * scale) * gate[o]) + widen(R[r, o])))
 * (page "ggml operator extensions", section "sd.cpp integration", the INT8
 * gated-residual fusion; the scale multiply only when scale != 1).  Y is the
 * binary32 reconstruction [M][N] (row stride N), R the residual [M][ldr] in
 * r_dtype, Z [M][ldz] in z_dtype (bf16 by round to nearest even).
 */
int oracle_gated_residual(const float *Y, int64_t M, int64_t N, float scale, const float *gate,
                          const void *R, int r_dtype, int64_t ldr, int z_dtype, void *Z,
                          int64_t ldz, int threads)
{
    if (!Y || !gate || !R || !Z || M < 0 || N < 0 || ldr < N || ldz < N)
        return ORACLE_EINVAL;
    if ((r_dtype != ORACLE_F32 && r_dtype != ORACLE_BF16) ||
        (z_dtype != ORACLE_F32 && z_dtype != ORACLE_BF16))
        return ORACLE_EUNSUPPORTED;
#pragma omp parallel for schedule(static) num_threads(threads > 0 ? threads : 1)
    for (int64_t r = 0; r < M; ++r) {
        for (int64_t o = 0; o < N; ++o) {
            float t = Y[r * N + o];
            if (scale != 1.0f)
                t = t * scale;
            t = t * gate[o];
            t = t + load_widened(R, r_dtype, r * ldr + o);
            if (z_dtype == ORACLE_F32)
                ((float *)Z)[r * ldz + o] = t;
            else
                ((uint16_t *)Z)[r * ldz + o] = f32_to_bf16_rne(t);
        }
    }
    return ORACLE_OK;
}

/*
 * The complete layer for one linear: quantize (packed), contract, reconstruct.
 * Scratch is malloc'ed here; this is the oracle, not the product.
 */
int oracle_linear(const void *X, int x_dtype, int64_t M, int64_t K, int64_t ldx, int G, float alpha,
                  const int8_t *Qw, const float *s_w, const float *bias, int64_t N, void *Y,
                  int y_dtype, int64_t ldy, int threads)
{
    if (!Qw)
        return ORACLE_EINVAL;
    int64_t m_pad = (M + 3) / 4 * 4;
    uint8_t *packed = (uint8_t *)malloc((size_t)oracle_packed_bytes(M, K));
    int32_t *A = (int32_t *)malloc((size_t)(M * N > 0 ? M * N : 1) * sizeof(int32_t));
    float *s_x = (float *)malloc((size_t)(m_pad > 0 ? m_pad : 1) * sizeof(float));
    int rc = ORACLE_EINVAL;
    if (packed && A && s_x) {
        rc = oracle_quantize_rows(X, x_dtype, M, K, ldx, G, alpha, packed, threads);
        if (rc == ORACLE_OK) {
            memcpy(s_x, packed + m_pad * K, (size_t)m_pad * sizeof(float));
            rc = oracle_gemm_i32((const int8_t *)packed, Qw, M, K, N, A, threads);
        }
        if (rc == ORACLE_OK)
            rc = oracle_epilogue(A, M, N, s_x, s_w, bias, alpha, y_dtype, Y, ldy, threads);
    }
    free(packed);
    free(A);
    free(s_x);
    return rc;
}
