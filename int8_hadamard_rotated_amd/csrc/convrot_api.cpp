// C ABI of the INT8 convrot linear library: host-side validation, workspace
// carving and kernel dispatch.  Semantics and conventions are documented in
// include/convrot.h.  Nothing here allocates device memory or synchronizes.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "../../include/convrot.h"
#include "kernels.h"

using namespace convrot_detail;

namespace {

constexpr int64_t kMaxContractionK = 133120;   // largest multiple of 64 with K * 127^2 < 2^31
constexpr int64_t kMaxContractionK4 = 132096;  // largest multiple of 64 with 16 * K * 127 * 8 < 2^31

int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }

// Every row count, column count and row stride is at most 2^30, so that all
// byte extents below fit in int64 (2^30 rows x 2^30 strides x 4 bytes).
constexpr int64_t kMaxDim = (int64_t)1 << 30;

bool dim_ok(int64_t v) { return v >= 0 && v <= kMaxDim; }

// The GEMM numbers its 128 x 128 tiles (the smallest it uses) with an int.
int64_t tiles_of(int64_t M, int64_t cols) { return ((M + 127) / 128) * ((cols + 127) / 128); }

bool tiles_ok(int64_t M, int64_t cols) { return tiles_of(M, cols) <= INT32_MAX; }

// Linears of one grouped launch share the tile numbering.
bool group_tiles_ok(int64_t M, int n, const convrot_linear_desc *descs)
{
    int64_t t = 0;
    for (int i = 0; i < n; ++i)
        t += tiles_of(M, 2 * descs[i].N);
    return t <= INT32_MAX;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Span {
    uintptr_t lo = 0, hi = 0;   // [lo, hi)
    bool empty() const { return hi <= lo; }
};

Span span_of(const void *p, int64_t bytes)
{
    Span s;
    if (p && bytes > 0) {
        s.lo = reinterpret_cast<uintptr_t>(p);
        s.hi = s.lo + (uintptr_t)bytes;
    }
    return s;
}

// Bytes touched by `rows` rows of `cols` elements at row stride `ld` elements.
Span rows_span(const void *p, int64_t rows, int64_t cols, int64_t ld, int64_t elem)
{
    if (rows <= 0 || cols <= 0)
        return Span{};
    return span_of(p, ((rows - 1) * ld + cols) * elem);
}

bool overlap(Span a, Span b) { return !a.empty() && !b.empty() && a.lo < b.hi && b.lo < a.hi; }

int64_t elem_bytes(int dtype) { return dtype == CONVROT_BF16 ? 2 : 4; }

bool dtype_ok(int dtype) { return dtype == CONVROT_F32 || dtype == CONVROT_BF16; }

bool scale_ok(float a) { return std::isfinite(a) && a > 0.0f; }

int hip_status(hipError_t e) { return e == hipSuccess ? CONVROT_OK : CONVROT_EHIP; }

// Group size rule of the convrot checkpoint format (a power of four dividing
// K), restricted to the groups this library implements (1 = no rotation up to
// 256), plus the MFMA K granularity of 64.
int check_quantizer_shape(int64_t K, int G)
{
    if (!(G == 1 || G == 4 || G == 16 || G == 64 || G == 256))
        return CONVROT_EUNSUPPORTED;
    if (K % 64 != 0 || K % G != 0)
        return CONVROT_EUNSUPPORTED;
    if (K > quantize_max_k(K))
        return CONVROT_EUNSUPPORTED;
    return CONVROT_OK;
}

int check_quantize_args(const void *X, int x_dtype, int64_t M, int64_t K, int64_t ldx, int G,
                        float alpha)
{
    if (M < 0 || K < 1 || ldx < K || !dim_ok(M) || !dim_ok(ldx))
        return CONVROT_EINVAL;
    if (!dtype_ok(x_dtype))
        return CONVROT_EUNSUPPORTED;
    const int rc = check_quantizer_shape(K, G);
    if (rc != CONVROT_OK)
        return rc;
    if (!scale_ok(alpha))
        return CONVROT_EINVAL;
    if (M > 0 && (!X || !aligned(X, 16) || (ldx * elem_bytes(x_dtype)) % 16 != 0))
        return CONVROT_EINVAL;
    return CONVROT_OK;
}

struct LinearCheck {
    Span y, reads;   // reads: the weight-side inputs (Qw, s_w, bias)
    Span qw, sw, b;
};

int check_linear(const int8_t *Qw, const float *s_w, const float *bias, int64_t M, int64_t K,
                 int64_t N, float alpha, const void *Y, int y_dtype, int64_t ldy, bool need_scales,
                 LinearCheck *out, int w_bits = 8)
{
    if (N < 0 || ldy < N || !dim_ok(M) || !dim_ok(ldy) || !tiles_ok(M, 2 * N))
        return CONVROT_EINVAL;
    if (need_scales && !dtype_ok(y_dtype))
        return CONVROT_EUNSUPPORTED;
    if (!scale_ok(alpha))
        return CONVROT_EINVAL;
    if (M > 0 && N > 0) {
        if (!Qw || !Y || !aligned(Qw, 16))
            return CONVROT_EINVAL;
        if ((s_w && !aligned(s_w, 4)) || (bias && !aligned(bias, 4)))
            return CONVROT_EINVAL;
        const int64_t ye = need_scales ? elem_bytes(y_dtype) : 4;
        if (!aligned(Y, (uintptr_t)ye))
            return CONVROT_EINVAL;
        out->y = rows_span(Y, M, N, ldy, ye);
        out->qw = span_of(Qw, w_bits == 4 ? N * (K / 2) : N * K);
        out->sw = need_scales ? span_of(s_w, 4 * N) : Span{};
        out->b = need_scales ? span_of(bias, 4 * N) : Span{};
    }
    return CONVROT_OK;
}

bool y_hits_weights(const LinearCheck &c, const LinearCheck &w)
{
    return overlap(c.y, w.qw) || overlap(c.y, w.sw) || overlap(c.y, w.b);
}

int check_contraction_k(int64_t K, int w_bits = 8)
{
    if (K < 1)
        return CONVROT_EINVAL;
    if (K % 64 != 0)
        return CONVROT_EUNSUPPORTED;
    if (K > (w_bits == 4 ? kMaxContractionK4 : kMaxContractionK))
        return CONVROT_EOVERFLOW;
    return CONVROT_OK;
}

GemmLinear make_linear(const int8_t *Qw, const float *s_w, const float *bias, int64_t N,
                       float alpha, void *Y, int kind, int64_t ldy)
{
    GemmLinear l;
    std::memset(&l, 0, sizeof l);
    l.Qw = Qw;
    l.s_w = s_w;
    l.bias = bias;
    l.Y = Y;
    l.N = N;
    l.ldy = ldy;
    l.alpha = alpha;
    l.out_kind = kind;
    const uintptr_t vec_bytes = kind == kOutBF16 ? 8 : 16;
    l.vec_store = (aligned(Y, vec_bytes) && ldy % 4 == 0) ? 1 : 0;
    return l;
}

int out_kind_of(int y_dtype) { return y_dtype == CONVROT_BF16 ? kOutBF16 : kOutF32; }

// Validates a producer descriptor (nullable) and returns the spans it reads.
// The producer's device vectors, for overlap checks.
struct PreSpans {
    Span scale, shift, weight, up;
    bool hits(const Span &s) const
    {
        return overlap(scale, s) || overlap(shift, s) || overlap(weight, s) || overlap(up, s);
    }
};

// The gated activation: a second input of X's dtype and shape.
int check_gated_act(const convrot_pre *pre, int64_t M, int64_t K, int x_dtype, PreOp *op,
                    PreSpans *spans)
{
    if (pre->act != CONVROT_ACT_SILU && pre->act != CONVROT_ACT_SIGMOID)
        return CONVROT_EUNSUPPORTED;
    const int64_t esz = elem_bytes(x_dtype);
    if (!pre->up || !aligned(pre->up, 16) || pre->ld_up < K || !dim_ok(pre->ld_up) ||
        (pre->ld_up * esz) % 16 != 0)
        return CONVROT_EINVAL;
    if (K > quantize_max_k(K, true))
        return CONVROT_EUNSUPPORTED;
    op->kind = kPreGatedAct;
    op->up = pre->up;
    op->ld_up = pre->ld_up;
    op->act = pre->act == CONVROT_ACT_SILU ? kActSilu : kActSigmoid;
    spans->up = M > 0 ? rows_span(pre->up, M, K, pre->ld_up, esz) : Span{};
    return CONVROT_OK;
}

// Norm -> Mul(weight): the weight is the only vector, eps as for RMSNorm.
int check_norm_mul(const convrot_pre *pre, int64_t K, PreOp *op, PreSpans *spans)
{
    if (pre->scale || pre->shift)
        return CONVROT_EINVAL;
    if ((pre->norm_weight && !aligned(pre->norm_weight, 16)) || !std::isfinite(pre->eps) ||
        pre->eps < 0.0f)
        return CONVROT_EINVAL;
    if (K > quantize_max_k(K, true))
        return CONVROT_EUNSUPPORTED;
    op->kind = kPreNormMul;
    op->norm_weight = pre->norm_weight;
    op->eps = pre->eps;
    spans->weight = span_of(pre->norm_weight, 4 * K);
    return CONVROT_OK;
}

int check_pre(const convrot_pre *pre, int64_t M, int64_t K, int x_dtype, PreOp *op, PreSpans *spans)
{
    *op = PreOp{};
    *spans = PreSpans{};
    if (!pre || pre->kind == CONVROT_PRE_NONE)
        return CONVROT_OK;
    if (pre->kind == CONVROT_PRE_GATED_ACT)
        return check_gated_act(pre, M, K, x_dtype, op, spans);
    if (pre->kind == CONVROT_PRE_NORM_MUL)
        return check_norm_mul(pre, K, op, spans);
    if (pre->kind != CONVROT_PRE_MODULATE && pre->kind != CONVROT_PRE_RMSNORM_MODULATE)
        return CONVROT_EUNSUPPORTED;
    const bool rms = pre->kind == CONVROT_PRE_RMSNORM_MODULATE;
    if ((!rms && !pre->scale) || (pre->shift && !pre->scale))
        return CONVROT_EINVAL;
    if ((pre->scale && !aligned(pre->scale, 16)) || (pre->shift && !aligned(pre->shift, 16)))
        return CONVROT_EINVAL;
    if (rms && ((pre->norm_weight && !aligned(pre->norm_weight, 16)) || !std::isfinite(pre->eps) ||
                pre->eps < 0.0f))
        return CONVROT_EINVAL;
    if (rms && K > quantize_max_k(K, true))
        return CONVROT_EUNSUPPORTED;
    op->kind = rms ? kPreRmsNormModulate : kPreModulate;
    op->scale = pre->scale;
    op->shift = pre->shift;
    op->norm_weight = rms ? pre->norm_weight : nullptr;
    op->eps = rms ? pre->eps : 0.0f;
    spans->scale = span_of(pre->scale, 4 * K);
    spans->shift = span_of(pre->shift, 4 * K);
    spans->weight = span_of(op->norm_weight, 4 * K);
    return CONVROT_OK;
}

}  // namespace

extern "C" {

size_t convrot_packed_bytes(int64_t M, int64_t K)
{
    if (M < 0 || K < 1 || !dim_ok(M) || !dim_ok(K))
        return 0;
    const int64_t m_pad = round_up(M, 4);
    return (size_t)(m_pad * K + 4 * m_pad);
}

size_t convrot_workspace_bytes(int64_t M, int64_t K, int n_packed)
{
    if (n_packed < 0)
        return 0;
    size_t bytes = 0;
    if (__builtin_mul_overflow((size_t)n_packed, (size_t)round_up((int64_t)convrot_packed_bytes(M, K), 256),
                               &bytes))
        return 0;
    return bytes;
}

int convrot_quantize_rows_pre(const void *X, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                              const convrot_pre *pre, int group_size, float input_scale,
                              void *packed, void *stream)
{
    int rc = check_quantize_args(X, x_dtype, M, K, ldx, group_size, input_scale);
    if (rc != CONVROT_OK)
        return rc;
    PreOp op;
    PreSpans ps;
    rc = check_pre(pre, M, K, x_dtype, &op, &ps);
    if (rc != CONVROT_OK)
        return rc;
    if (M == 0)
        return CONVROT_OK;
    if (!packed || !aligned(packed, 16))
        return CONVROT_EINVAL;
    const Span out = span_of(packed, (int64_t)convrot_packed_bytes(M, K));
    if (overlap(rows_span(X, M, K, ldx, elem_bytes(x_dtype)), out) || ps.hits(out))
        return CONVROT_EOVERLAP;
    (void)hipGetLastError();
    return hip_status(launch_quantize(X, x_dtype, M, K, ldx, group_size, input_scale, op, packed,
                                      static_cast<hipStream_t>(stream)));
}

int convrot_expf(const float *x, float *y, int64_t n, void *stream)
{
    if (n < 0)
        return CONVROT_EINVAL;
    if (n == 0)
        return CONVROT_OK;
    if (!x || !y || !aligned(x, 4) || !aligned(y, 4) || n > ((int64_t)1 << 38))
        return CONVROT_EINVAL;
    if (x != y && overlap(span_of(x, 4 * n), span_of(y, 4 * n)))
        return CONVROT_EOVERLAP;
    (void)hipGetLastError();
    return hip_status(launch_expf(x, y, n, static_cast<hipStream_t>(stream)));
}

int convrot_quantize_rows(const void *X, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                          int group_size, float input_scale, void *packed, void *stream)
{
    return convrot_quantize_rows_pre(X, x_dtype, M, K, ldx, nullptr, group_size, input_scale,
                                     packed, stream);
}

int convrot_quantize_rows_scales(const void *X, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                                 int group_size, int n, const float *input_scales,
                                 void *const *packed, void *stream)
{
    if (n < 1 || n > kMaxLinears || !input_scales || !packed)
        return CONVROT_EINVAL;
    for (int i = 0; i < n; ++i) {
        const int rc = check_quantize_args(X, x_dtype, M, K, ldx, group_size, input_scales[i]);
        if (rc != CONVROT_OK)
            return rc;
    }
    if (M == 0)
        return CONVROT_OK;
    const int64_t pb = (int64_t)convrot_packed_bytes(M, K);
    const Span xs = rows_span(X, M, K, ldx, elem_bytes(x_dtype));
    for (int i = 0; i < n; ++i) {
        if (!packed[i] || !aligned(packed[i], 16))
            return CONVROT_EINVAL;
        const Span out = span_of(packed[i], pb);
        if (overlap(xs, out))
            return CONVROT_EOVERLAP;
        for (int k = 0; k < i; ++k) {
            if (overlap(out, span_of(packed[k], pb)))
                return CONVROT_EOVERLAP;
        }
    }
    (void)hipGetLastError();
    return hip_status(launch_quantize_scales(X, x_dtype, M, K, ldx, group_size, n, input_scales,
                                             packed, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// Validates an epilogue descriptor (nullable) for an [M][N] output Y.
int check_post(const convrot_post *post, int64_t M, int64_t N, const void *Y, int y_dtype,
               int64_t ldy, const Span &y, GemmLinear *l)
{
    if (!post || post->kind == CONVROT_POST_NONE)
        return CONVROT_OK;
    if (post->kind != CONVROT_POST_GATED_RESIDUAL)
        return CONVROT_EUNSUPPORTED;
    if (!std::isfinite(post->scale))
        return CONVROT_EINVAL;
    if (M == 0 || N == 0)
        return CONVROT_OK;
    const int64_t e = elem_bytes(y_dtype);
    if (!post->gate || !aligned(post->gate, 4) || !post->residual ||
        !aligned(post->residual, (uintptr_t)e) || post->ld_residual < N || !dim_ok(post->ld_residual))
        return CONVROT_EINVAL;
    const Span rs = rows_span(post->residual, M, N, post->ld_residual, e);
    const bool in_place = post->residual == Y && post->ld_residual == ldy;
    if ((!in_place && overlap(rs, y)) || overlap(span_of(post->gate, 4 * N), y))
        return CONVROT_EOVERLAP;
    l->post = 1;
    l->post_scale = post->scale;
    l->gate = post->gate;
    l->residual = post->residual;
    l->ld_res = post->ld_residual;
    l->res_vec = (aligned(post->residual, y_dtype == CONVROT_BF16 ? 8 : 16) &&
                  post->ld_residual % 4 == 0) ? 1 : 0;
    return CONVROT_OK;
}

int linear_impl(const int8_t *Qx, const float *s_x, int64_t M, int64_t K, const int8_t *Qw,
                const float *s_w, const float *bias, int64_t N, float input_scale, void *Y,
                int y_dtype, int64_t ldy, void *stream, int w_bits, const convrot_post *post = nullptr)
{
    if (M < 0)
        return CONVROT_EINVAL;
    int rc = check_contraction_k(K, w_bits);
    if (rc != CONVROT_OK)
        return rc;
    LinearCheck c;
    rc = check_linear(Qw, s_w, bias, M, K, N, input_scale, Y, y_dtype, ldy, true, &c, w_bits);
    if (rc != CONVROT_OK)
        return rc;
    GemmLinear post_fields;
    std::memset(&post_fields, 0, sizeof post_fields);
    rc = check_post(post, M, N, Y, y_dtype, ldy, c.y, &post_fields);
    if (rc != CONVROT_OK)
        return rc;
    if (M == 0 || N == 0)
        return CONVROT_OK;
    if (!Qx || !s_x || !aligned(Qx, 16) || !aligned(s_x, 4))
        return CONVROT_EINVAL;
    if (overlap(c.y, span_of(Qx, M * K)) || overlap(c.y, span_of(s_x, 4 * M)) ||
        y_hits_weights(c, c))
        return CONVROT_EOVERLAP;
    GemmProblem p;
    std::memset(&p, 0, sizeof p);
    p.Qx = Qx;
    p.s_x = s_x;
    p.M = M;
    p.K = K;
    p.w_bits = w_bits;
    p.n_lin = 1;
    p.lin[0] = make_linear(Qw, s_w, bias, N, input_scale, Y, out_kind_of(y_dtype), ldy);
    p.lin[0].post = post_fields.post;
    p.lin[0].post_scale = post_fields.post_scale;
    p.lin[0].gate = post_fields.gate;
    p.lin[0].residual = post_fields.residual;
    p.lin[0].ld_res = post_fields.ld_res;
    p.lin[0].res_vec = post_fields.res_vec;
    (void)hipGetLastError();
    return hip_status(launch_gemm(p, static_cast<hipStream_t>(stream)));
}

int gemm_i32_impl(const int8_t *Qx, const int8_t *Qw, int64_t M, int64_t K, int64_t N,
                  int32_t *A, void *stream, int w_bits)
{
    if (M < 0)
        return CONVROT_EINVAL;
    int rc = check_contraction_k(K, w_bits);
    if (rc != CONVROT_OK)
        return rc;
    LinearCheck c;
    rc = check_linear(Qw, nullptr, nullptr, M, K, N, 1.0f, A, CONVROT_F32, N, false, &c, w_bits);
    if (rc != CONVROT_OK)
        return rc;
    if (M == 0 || N == 0)
        return CONVROT_OK;
    if (!Qx || !aligned(Qx, 16))
        return CONVROT_EINVAL;
    if (overlap(c.y, span_of(Qx, M * K)) || overlap(c.y, c.qw))
        return CONVROT_EOVERLAP;
    GemmProblem p;
    std::memset(&p, 0, sizeof p);
    p.Qx = Qx;
    p.s_x = nullptr;
    p.M = M;
    p.K = K;
    p.w_bits = w_bits;
    p.n_lin = 1;
    p.lin[0] = make_linear(Qw, nullptr, nullptr, N, 1.0f, A, kOutI32, N);
    (void)hipGetLastError();
    return hip_status(launch_gemm(p, static_cast<hipStream_t>(stream)));
}

// Input scales 2^k with |k| <= 16 give the bits of the alpha = 1 pass: the
// pre-scale by 2^k and the division by 2^k are both exact, and so is every
// rounding in between (binary32 rounding commutes with scaling by a power of
// two in the normal range, and the quantizer's input contract keeps every
// rotation value that could round there).  Such linears read the alpha = 1
// packed tensor and skip the division.
constexpr int kFoldedScaleExp = 16;

float quantize_scale_of(float input_scale)
{
    int e = 0;
    if (input_scale > 0.0f && std::frexp(input_scale, &e) == 0.5f && e - 1 >= -kFoldedScaleExp &&
        e - 1 <= kFoldedScaleExp)
        return 1.0f;
    return input_scale;
}

}  // namespace

extern "C" {

int int8_linear(const int8_t *Qx, const float *s_x, int64_t M, int64_t K, const int8_t *Qw,
                const float *s_w, const float *bias, int64_t N, float input_scale, void *Y,
                int y_dtype, int64_t ldy, void *stream)
{
    return linear_impl(Qx, s_x, M, K, Qw, s_w, bias, N, input_scale, Y, y_dtype, ldy, stream, 8);
}

int int8_linear_grouped(const int8_t *Qx, const float *s_x, int64_t M, int64_t K, int n,
                        const convrot_linear_desc *descs, void *stream)
{
    if (M < 0 || n < 1 || n > kMaxLinears || !descs)
        return CONVROT_EINVAL;
    int rc = check_contraction_k(K, 8);
    if (rc != CONVROT_OK)
        return rc;
    LinearCheck chk[kMaxLinears];
    for (int i = 0; i < n; ++i) {
        const convrot_linear_desc &d = descs[i];
        rc = check_linear(d.Qw, d.s_w, d.bias, M, K, d.N, d.input_scale, d.Y, d.y_dtype, d.ldy,
                          true, &chk[i]);
        if (rc != CONVROT_OK)
            return rc;
    }
    if (!group_tiles_ok(M, n, descs))
        return CONVROT_EINVAL;
    // each linear's input: its own (Qx, s_x) or the call's
    const int8_t *qx_of[kMaxLinears];
    const float *sx_of[kMaxLinears];
    bool shared_used = false;
    for (int i = 0; i < n; ++i) {
        if ((descs[i].Qx == nullptr) != (descs[i].s_x == nullptr))
            return CONVROT_EINVAL;
        qx_of[i] = descs[i].Qx ? descs[i].Qx : Qx;
        sx_of[i] = descs[i].Qx ? descs[i].s_x : s_x;
        shared_used = shared_used || (descs[i].Qx == nullptr && descs[i].N > 0);
    }
    if (M == 0)
        return CONVROT_OK;
    if (shared_used && (!Qx || !s_x))
        return CONVROT_EINVAL;
    for (int i = 0; i < n; ++i) {
        if (descs[i].N == 0)
            continue;
        if (!aligned(qx_of[i], 16) || !aligned(sx_of[i], 4))
            return CONVROT_EINVAL;
    }
    for (int i = 0; i < n; ++i) {
        if (descs[i].N == 0)
            continue;
        for (int k = 0; k < n; ++k) {
            if (descs[k].N == 0)
                continue;
            if (overlap(chk[i].y, span_of(qx_of[k], M * K)) ||
                overlap(chk[i].y, span_of(sx_of[k], 4 * M)))
                return CONVROT_EOVERLAP;
            if (y_hits_weights(chk[i], chk[k]))
                return CONVROT_EOVERLAP;
            if (k != i && overlap(chk[i].y, chk[k].y))
                return CONVROT_EOVERLAP;
        }
    }
    GemmProblem p;
    std::memset(&p, 0, sizeof p);
    p.M = M;
    p.K = K;
    p.w_bits = 8;
    for (int i = 0; i < n; ++i) {
        const convrot_linear_desc &d = descs[i];
        if (d.N == 0)
            continue;
        GemmLinear l = make_linear(d.Qw, d.s_w, d.bias, d.N, d.input_scale, d.Y,
                                   out_kind_of(d.y_dtype), d.ldy);
        l.Qx = qx_of[i];
        l.s_x = sx_of[i];
        p.lin[p.n_lin++] = l;
    }
    if (p.n_lin == 0)
        return CONVROT_OK;
    (void)hipGetLastError();
    return hip_status(launch_gemm(p, static_cast<hipStream_t>(stream)));
}

int int8_swiglu_linear(const int8_t *Qx, const float *s_x, int64_t M, int64_t K,
                       const int8_t *Qw_gate, const float *s_w_gate, const int8_t *Qw_up,
                       const float *s_w_up, int64_t N, float input_scale, void *Y, int y_dtype,
                       int64_t ldy, void *stream)
{
    if (M < 0)
        return CONVROT_EINVAL;
    int rc = check_contraction_k(K, 8);
    if (rc != CONVROT_OK)
        return rc;
    LinearCheck cg, cu;
    rc = check_linear(Qw_gate, s_w_gate, nullptr, M, K, N, input_scale, Y, y_dtype, ldy, true, &cg, 8);
    if (rc != CONVROT_OK)
        return rc;
    rc = check_linear(Qw_up, s_w_up, nullptr, M, K, N, input_scale, Y, y_dtype, ldy, true, &cu, 8);
    if (rc != CONVROT_OK)
        return rc;
    if (M == 0 || N == 0)
        return CONVROT_OK;
    if (!Qx || !s_x || !aligned(Qx, 16) || !aligned(s_x, 4))
        return CONVROT_EINVAL;
    if (overlap(cg.y, span_of(Qx, M * K)) || overlap(cg.y, span_of(s_x, 4 * M)) ||
        y_hits_weights(cg, cg) || y_hits_weights(cg, cu))
        return CONVROT_EOVERLAP;
    GemmProblem p;
    std::memset(&p, 0, sizeof p);
    p.Qx = Qx;
    p.s_x = s_x;
    p.M = M;
    p.K = K;
    p.w_bits = 8;
    p.n_lin = 1;
    p.lin[0] = make_linear(Qw_gate, s_w_gate, nullptr, N, input_scale, Y, out_kind_of(y_dtype), ldy);
    p.lin[0].glu = 1;
    p.lin[0].Qw_up = Qw_up;
    p.lin[0].s_w_up = s_w_up;
    (void)hipGetLastError();
    return hip_status(launch_gemm(p, static_cast<hipStream_t>(stream)));
}

int int8_linear_post(const int8_t *Qx, const float *s_x, int64_t M, int64_t K, const int8_t *Qw,
                     const float *s_w, const float *bias, int64_t N, float input_scale,
                     const convrot_post *post, void *Y, int y_dtype, int64_t ldy, void *stream)
{
    return linear_impl(Qx, s_x, M, K, Qw, s_w, bias, N, input_scale, Y, y_dtype, ldy, stream, 8,
                       post);
}

int int4_linear(const int8_t *Qx, const float *s_x, int64_t M, int64_t K, const uint8_t *W4,
                const float *s_w, const float *bias, int64_t N, float input_scale, void *Y,
                int y_dtype, int64_t ldy, void *stream)
{
    return linear_impl(Qx, s_x, M, K, reinterpret_cast<const int8_t *>(W4), s_w, bias, N,
                       input_scale, Y, y_dtype, ldy, stream, 4);
}

int convrot_int4_gemm_i32(const int8_t *Qx, const uint8_t *W4, int64_t M, int64_t K, int64_t N,
                          int32_t *A, void *stream)
{
    return gemm_i32_impl(Qx, reinterpret_cast<const int8_t *>(W4), M, K, N, A, stream, 4);
}

int convrot_int8_gemm_i32(const int8_t *Qx, const int8_t *Qw, int64_t M, int64_t K, int64_t N,
                          int32_t *A, void *stream)
{
    return gemm_i32_impl(Qx, Qw, M, K, N, A, stream, 8);
}

}  // extern "C"

namespace {

// The fused entries: validation, one quantization pass per distinct input
// scale into the workspace, then one grouped GEMM launch over all linears.
// With use_static the workspace is the library's static buffer instead of
// the caller's (taken only after every other argument has been validated).
int shared_impl(const void *X, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                const convrot_pre *pre, int group_size, int n, const convrot_linear_desc *descs,
                void *workspace, size_t workspace_bytes, bool use_static, void *stream)
{
    if (n < 1 || n > kMaxLinears || !descs)
        return CONVROT_EINVAL;
    int rc = check_quantize_args(X, x_dtype, M, K, ldx, group_size, 1.0f);
    if (rc != CONVROT_OK)
        return rc;
    PreOp op;
    PreSpans ps;
    rc = check_pre(pre, M, K, x_dtype, &op, &ps);
    if (rc != CONVROT_OK)
        return rc;
    rc = check_contraction_k(K);
    if (rc != CONVROT_OK)
        return rc;

    LinearCheck chk[kMaxLinears];
    float scales[kMaxLinears];
    int slot_of[kMaxLinears];
    int n_slots = 0;
    for (int i = 0; i < n; ++i) {
        const convrot_linear_desc &d = descs[i];
        if (d.Qx || d.s_x)
            return CONVROT_EINVAL;      // the fused entries quantize X themselves
        rc = check_linear(d.Qw, d.s_w, d.bias, M, K, d.N, d.input_scale, d.Y, d.y_dtype, d.ldy,
                          true, &chk[i]);
        if (rc != CONVROT_OK)
            return rc;
        const float a = quantize_scale_of(d.input_scale);
        int s = 0;
        while (s < n_slots && scales[s] != a)
            ++s;
        if (s == n_slots)
            scales[n_slots++] = a;
        slot_of[i] = s;
    }
    if (!group_tiles_ok(M, n, descs))
        return CONVROT_EINVAL;
    if (M == 0)
        return CONVROT_OK;

    for (int i = 0; i < n; ++i) {
        for (int k = 0; k < n; ++k) {
            if (y_hits_weights(chk[i], chk[k]))
                return CONVROT_EOVERLAP;
            if (k != i && overlap(chk[i].y, chk[k].y))
                return CONVROT_EOVERLAP;
        }
    }

    const int64_t pb = (int64_t)convrot_packed_bytes(M, K);
    const int64_t slot_bytes = round_up(pb, 256);
    if (use_static) {
        if (convrot_workspace_bytes(M, K, n_slots) > kStaticWorkspaceBytes)
            return CONVROT_EWORKSPACE;
        (void)hipGetLastError();
        if (static_workspace(&workspace) != hipSuccess)
            return CONVROT_EHIP;
        workspace_bytes = kStaticWorkspaceBytes;
    }
    if (!workspace || workspace_bytes < convrot_workspace_bytes(M, K, n_slots))
        return CONVROT_EWORKSPACE;
    if (!aligned(workspace, 16))
        return CONVROT_EINVAL;
    const Span ws = span_of(workspace, slot_bytes * n_slots);
    const Span xs = rows_span(X, M, K, ldx, elem_bytes(x_dtype));
    if (overlap(ws, xs) || ps.hits(ws))
        return CONVROT_EOVERLAP;
    for (int i = 0; i < n; ++i) {
        if (overlap(chk[i].y, ws) || overlap(chk[i].qw, ws) || overlap(chk[i].sw, ws) ||
            overlap(chk[i].b, ws))
            return CONVROT_EOVERLAP;
    }

    hipStream_t st = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    int8_t *base = static_cast<int8_t *>(workspace);
    if (op.kind == kPreNone) {
        // plain rows: the passes of every scale together (binary32 rows are
        // then read once per few scales)
        void *outs[kMaxLinears];
        for (int s = 0; s < n_slots; ++s)
            outs[s] = base + s * slot_bytes;
        rc = hip_status(launch_quantize_scales(X, x_dtype, M, K, ldx, group_size, n_slots, scales,
                                               outs, st));
        if (rc != CONVROT_OK)
            return rc;
    } else {
        for (int s = 0; s < n_slots; ++s) {
            rc = hip_status(launch_quantize(X, x_dtype, M, K, ldx, group_size, scales[s], op,
                                            base + s * slot_bytes, st));
            if (rc != CONVROT_OK)
                return rc;
        }
    }
    // one grouped launch: every linear reads the packed tensor of its scale
    const int64_t m_pad = round_up(M, 4);
    GemmProblem p;
    std::memset(&p, 0, sizeof p);
    p.M = M;
    p.K = K;
    p.w_bits = 8;
    for (int i = 0; i < n; ++i) {
        const convrot_linear_desc &d = descs[i];
        if (d.N == 0)
            continue;
        const int s = slot_of[i];
        // the divisor is the scale of the pass this linear reads
        GemmLinear l = make_linear(d.Qw, d.s_w, d.bias, d.N, scales[s], d.Y,
                                   out_kind_of(d.y_dtype), d.ldy);
        l.Qx = base + s * slot_bytes;
        l.s_x = reinterpret_cast<const float *>(base + s * slot_bytes + m_pad * K);
        p.lin[p.n_lin++] = l;
    }
    if (p.n_lin == 0)
        return CONVROT_OK;
    return hip_status(launch_gemm(p, st));
}

convrot_linear_desc one_linear(const int8_t *Qw, const float *s_w, const float *bias, int64_t N,
                               float input_scale, void *Y, int y_dtype, int64_t ldy)
{
    convrot_linear_desc d;
    d.Qw = Qw;
    d.s_w = s_w;
    d.bias = bias;
    d.N = N;
    d.input_scale = input_scale;
    d.Y = Y;
    d.y_dtype = y_dtype;
    d.ldy = ldy;
    d.Qx = nullptr;
    d.s_x = nullptr;
    return d;
}

}  // namespace

extern "C" {

int convrot_int8_linear_shared_pre(const void *X, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                                   const convrot_pre *pre, int group_size, int n,
                                   const convrot_linear_desc *descs, void *workspace,
                                   size_t workspace_bytes, void *stream)
{
    return shared_impl(X, x_dtype, M, K, ldx, pre, group_size, n, descs, workspace,
                       workspace_bytes, false, stream);
}

int convrot_int8_linear_shared(const void *X, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                               int group_size, int n, const convrot_linear_desc *descs,
                               void *workspace, size_t workspace_bytes, void *stream)
{
    return convrot_int8_linear_shared_pre(X, x_dtype, M, K, ldx, nullptr, group_size, n, descs,
                                          workspace, workspace_bytes, stream);
}

int convrot_int8_linear(const void *X, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                        int group_size, float input_scale, const int8_t *Qw, const float *s_w,
                        const float *bias, int64_t N, void *Y, int y_dtype, int64_t ldy,
                        void *workspace, size_t workspace_bytes, void *stream)
{
    const convrot_linear_desc d = one_linear(Qw, s_w, bias, N, input_scale, Y, y_dtype, ldy);
    return convrot_int8_linear_shared(X, x_dtype, M, K, ldx, group_size, 1, &d, workspace,
                                      workspace_bytes, stream);
}

int convrot_int8_linear_noalloc(const void *X, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                                int group_size, float input_scale, const int8_t *Qw,
                                const float *s_w, const float *bias, int64_t N, void *Y,
                                int y_dtype, int64_t ldy, void *stream)
{
    const convrot_linear_desc d = one_linear(Qw, s_w, bias, N, input_scale, Y, y_dtype, ldy);
    return shared_impl(X, x_dtype, M, K, ldx, nullptr, group_size, 1, &d, nullptr, 0, true,
                       stream);
}

const char *convrot_status_string(int status)
{
    switch (status) {
    case CONVROT_OK: return "ok";
    case CONVROT_EINVAL: return "invalid argument (null pointer, shape, stride, alignment or input scale)";
    case CONVROT_EUNSUPPORTED: return "unsupported group size, K granularity or dtype";
    case CONVROT_EOVERFLOW: return "K too large for an exact int32 accumulator";
    case CONVROT_EOVERLAP: return "an output overlaps a buffer that the same kernel reads";
    case CONVROT_EWORKSPACE: return "workspace missing or too small";
    case CONVROT_EHIP: return "HIP runtime error at launch";
    default: return "unknown status";
    }
}

}  // extern "C"
