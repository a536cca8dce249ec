/*
 * convrot.h -- C ABI of the MI355X (gfx950) INT8 convrot linear library.
 *
 * The layer (page "INT8 Convrot Safetensors", sd.cpp docs/int8_convrot.md,
 * section "How INT8 convrot works"):
 *
 *   X_rot = X R            R = block-diagonal H4^(x)n over contiguous groups
 *                          of G = 4^n input features, H4 = [[1,1,1,-1],
 *                          [1,1,-1,1],[1,-1,1,1],[-1,1,1,1]] / 2
 *   s_x[r] = max_i |X_rot[r,i]| / 127           (whole row; subsection
 *   Q_x[r,i] = clamp(round(X_rot[r,i] / s_x[r]), -127, 127)   "Runtime
 *                                                activation quantization")
 *   A[r,o] = sum_i Q_x[r,i] * Q_w[o,i]          (int32)
 *   Y[r,o] = A[r,o] * s_x[r] * s_w[o] + b[o]
 *
 * with Q_w, s_w the offline rotated and per-output-row quantized weights
 * (subsection "Weight quantization"; the same quantizer applied to W's rows,
 * so convrot_quantize_rows on W produces them).  For an input scale alpha != 1
 * the activation is multiplied by alpha before the rotation and the output is
 * divided by alpha before the bias; linears that share an input, the group size
 * and alpha = 1 reuse one packed activation tensor (same section, last
 * paragraph).  The operator-extensions page (sd.cpp docs/ggml_extensions.md,
 * section "sd.cpp integration") fixes the reconstruction order
 * float(A) * s_x * s_w + bias, the nullable weight scale and bias, and the
 * packed layout (I8 rows padded to a multiple of four, then F32 row scales).
 *
 * Arithmetic contract (identical bits to the CPU oracle):
 *   - the rotation is one H4 application per base-4 digit of the in-group
 *     index, digit 0 (stride 1) first; each computes s = (x0 + x1) + (x2 + x3),
 *     h = s * 0.5, y_j = h - x_{3-j}, every operation rounded to nearest even
 *     binary32 (no contraction);
 *   - s_x = fl(m / 127) with m = max |y| over the row; codes are
 *     round-half-to-even(fl(y * fl(127 / m))) clamped to [-127, 127]
 *     (the page's "/ s_x" is taken as a product with the row's correctly
 *     rounded reciprocal); a row with m = 0 gets s_x = 0 and all-zero codes;
 *   - Y = fl(fl(fl(fl(float(A)) * s_x) * s_w) / alpha) + b, each step rounded
 *     separately (the division only when alpha != 1); bf16 output is rounded
 *     to nearest even from that binary32 value.
 *   - inputs must be finite, and every nonzero |x * alpha| must lie in
 *     [2^-100, 2^100]; outside that range results are unspecified.
 *
 * Conventions for every entry point:
 *   - Device pointers unless stated otherwise; the caller owns all memory.
 *     The library never allocates, frees or retains memory (the one
 *     exception is the static buffer of convrot_int8_linear_noalloc, part
 *     of its code object), and never synchronizes: all work is enqueued on `stream` (a hipStream_t; NULL is
 *     the default stream) in call order.  Calls enqueue kernel launches only
 *     (no memory fills or copies), so they may be captured into a HIP graph;
 *     a replay reads the buffers' contents at replay time.
 *   - Row-major, last index contiguous.  X is [M][ldx] (elements), W-side
 *     codes Q_w are [N][K], Y is [M][ldy] (elements).
 *   - Arguments are validated on the host before anything is enqueued; on any
 *     error nothing is enqueued and a negative convrot_status is returned.
 *     Errors are never retried and there is no fallback to another device.
 *   - M = 0 or N = 0 is valid and enqueues nothing.
 *   - GPU support: G in {1, 4, 16, 64, 256}; K a multiple of 64 and of G; the
 *     quantizer needs K <= 65536, the contraction K <= 133120 (so that
 *     K * 127^2 < 2^31: codes are taken to lie in [-127, 127], as the
 *     quantizer produces).  Pointers to X, packed buffers, Q_x, Q_w and the
 *     workspace must be 16-byte aligned, ldx * sizeof(X element) a multiple
 *     of 16; scale and bias pointers 4-byte aligned; Y aligned to its element.
 *   - Concurrent calls that write the same buffers race; calls on one stream
 *     are ordered.
 */
#ifndef CONVROT_H
#define CONVROT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CONVROT_OK = 0,
    CONVROT_EINVAL = -1,        /* null pointer, bad shape/stride/alignment, bad input scale */
    CONVROT_EUNSUPPORTED = -2,  /* group size, K granularity or dtype not supported */
    CONVROT_EOVERFLOW = -3,     /* K too large for an exact int32 accumulator */
    CONVROT_EOVERLAP = -4,      /* an output overlaps a buffer the same kernel reads */
    CONVROT_EWORKSPACE = -5,    /* workspace missing or smaller than required */
    CONVROT_EHIP = -6           /* the HIP runtime reported an error at launch */
} convrot_status;

typedef enum { CONVROT_F32 = 0, CONVROT_BF16 = 1 } convrot_dtype;

/* Bytes of the packed activation tensor for M rows of K features (page
 * "ggml operator extensions", section "sd.cpp integration": I8 rows padded
 * to a multiple of four, followed by the F32 row scales):
 * int8 codes [M_pad][K] followed by float scales [M_pad], M_pad = 4*ceil(M/4).
 * Pad rows hold zero codes and a zero scale.  Returns 0 if M < 0, K < 1, or
 * M or K is above 2^30 (every dimension and row stride of this interface is
 * at most 2^30; larger ones are CONVROT_EINVAL). */
size_t convrot_packed_bytes(int64_t M, int64_t K);

/* Rotate, quantize and pack M rows of X (page "INT8 Convrot Safetensors",
 * section "How INT8 convrot works": the group-wise rotation and, in
 * "Runtime activation quantization", the per-row scale and codes; packed as
 * convrot_packed_bytes describes).
 *   X           [M][ldx] f32 or bf16 (x_dtype), first K columns used
 *   group_size  G, rotation group (power of four dividing K: 1, 4, 16, 64 or
 *               256; G = 1 is the identity, per-row quantization alone)
 *   input_scale alpha > 0, finite; X is multiplied by it before the rotation
 *   packed      convrot_packed_bytes(M, K) bytes, written entirely (pad rows
 *               and pad scales included); must not overlap X
 * Returns CONVROT_OK or a negative status (nothing enqueued on error). */
int convrot_quantize_rows(const void *X, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                          int group_size, float input_scale, void *packed, void *stream);

/* convrot_quantize_rows for several input scales of the same X (page "INT8
 * Convrot Safetensors", section "How INT8 convrot works": each input scale
 * other than 1 gets its own quantization of X, pre-scaled by it): packed[i]
 * receives exactly the bytes of convrot_quantize_rows(..., input_scales[i],
 * packed[i], ...).  Binary32 rows whose workgroups stay within 256 threads
 * (K up to 16 384 with G = 256) are read from HBM once per two scales;
 * other rows are read once per scale.  input_scales and packed are host
 * arrays of n entries, 1 <= n <= 16; each packed[i] is a device buffer of
 * convrot_packed_bytes(M, K), 16-byte aligned, overlapping neither X nor
 * another packed[k] (CONVROT_EOVERLAP). */
int convrot_quantize_rows_scales(const void *X, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                                 int group_size, int n, const float *input_scales,
                                 void *const *packed, void *stream);

/* INT8 linear on already-quantized activations, the GEMM + reconstruction
 * (page "INT8 Convrot Safetensors", section "How INT8 convrot works": the
 * int32 accumulation and Y = A s_x s_w + b; page "ggml operator extensions",
 * section "sd.cpp integration": the order float(A) * s_x * s_w + bias with
 * nullable weight scale and bias):
 *   Y = fl(fl(fl(fl(float(Q_x Q_w^T)) * s_x) * s_w) / input_scale) + bias
 *   Qx     [M][K] int8 codes (row stride K); for a packed tensor pass its base
 *   s_x    [M] float row scales; for a packed tensor pass base + M_pad * K
 *   Qw     [N][K] int8 weight codes
 *   s_w    [N] float weight scales, or NULL (taken as 1, no multiply)
 *   bias   [N] float, or NULL (no add)
 *   input_scale  the divisor alpha (1 = no division)
 *   Y      [M][ldy] f32 or bf16 (y_dtype); must not overlap any input
 */
int int8_linear(const int8_t *Qx, const float *s_x, int64_t M, int64_t K, const int8_t *Qw,
                const float *s_w, const float *bias, int64_t N, float input_scale, void *Y,
                int y_dtype, int64_t ldy, void *stream);

/* Workspace bytes needed by the fused entries for `n_packed` packed tensors of
 * M rows x K features (each rounded up to 256 bytes); 0 when that does not fit
 * a size_t.  The workspace is the framework's, never the library's (page
 * "ggml operator extensions", section "Backend services"). */
size_t convrot_workspace_bytes(int64_t M, int64_t K, int n_packed);

/* The fused layer for one linear (page "INT8 Convrot Safetensors", section
 * "How INT8 convrot works", the whole layer including the input scale):
 * convrot_quantize_rows into the workspace,
 * then int8_linear on it (a power-of-two input scale is folded as in
 * convrot_int8_linear_shared).  workspace >= convrot_workspace_bytes(M, K, 1);
 * contents are not preserved between calls.  Y may alias X (X is fully
 * consumed before Y is written) but not Qw, s_w, bias or the workspace. */
int convrot_int8_linear(const void *X, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                        int group_size, float input_scale, const int8_t *Qw, const float *s_w,
                        const float *bias, int64_t N, void *Y, int y_dtype, int64_t ldy,
                        void *workspace, size_t workspace_bytes, void *stream);

/* convrot_int8_linear without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops,
 * harnesses that forbid hipMalloc).  The packed activation tensor goes to a
 * buffer the library owns: a 64 MiB device array in its code object, one copy
 * per GPU it runs on, held until the process ends; the call itself allocates
 * nothing.  Same arguments, semantics and rules as convrot_int8_linear;
 * CONVROT_EWORKSPACE if convrot_workspace_bytes(M, K, 1) exceeds 64 MiB
 * (M * K up to about 67 million, e.g. 4096 x 16384).  Every call on one GPU
 * uses that GPU's one buffer (contents are not preserved; nothing in it needs
 * to start at zero): calls that can overlap in time on the same GPU, on
 * different streams or from different threads, race, and must be ordered by
 * the caller. */
int convrot_int8_linear_noalloc(const void *X, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                                int group_size, float input_scale, const int8_t *Qw,
                                const float *s_w, const float *bias, int64_t N, void *Y,
                                int y_dtype, int64_t ldy, void *stream);

/* One linear reading a shared input (host-side descriptor). */
typedef struct {
    const int8_t *Qw;     /* [N][K] int8 weight codes (device) */
    const float *s_w;     /* [N] or NULL (device) */
    const float *bias;    /* [N] or NULL (device) */
    int64_t N;            /* output features */
    float input_scale;    /* alpha of this linear */
    void *Y;              /* [M][ldy] output (device) */
    int y_dtype;          /* CONVROT_F32 or CONVROT_BF16 */
    int64_t ldy;          /* output row stride in elements (>= N) */
    const int8_t *Qx;     /* int8_linear_grouped only: this linear's own quantized
                             input [M][K] (device), or NULL for the call's Qx;
                             NULL for the fused entries, which quantize X */
    const float *s_x;     /* with Qx: its [M] row scales (device); else NULL */
} convrot_linear_desc;

/* Several INT8 linears on already-quantized inputs, in one GEMM launch (the
 * contraction and reconstruction of int8_linear for each; page "INT8
 * Convrot Safetensors", section "How INT8 convrot works": one packed
 * activation tensor reused by the linears that share it).  Qx, s_x as for
 * int8_linear: the input of every linear whose descriptor leaves Qx NULL; a
 * linear may name its own (Qx, s_x) instead, e.g. the packed tensor of its
 * own input scale, of the same M and K.  descs is host memory, 1 <= n <= 16,
 * and each linear's input_scale is its divisor (as int8_linear's).  Outputs
 * must not overlap each other, any input codes or scales, or any weight-side
 * input. */
int int8_linear_grouped(const int8_t *Qx, const float *s_x, int64_t M, int64_t K, int n,
                        const convrot_linear_desc *descs, void *stream);

/* Several linears on the same X and group size (page "INT8 Convrot
 * Safetensors", section "How INT8 convrot works", last paragraph: one
 * quantized activation reused by the linears that share it; page "ggml
 * operator extensions", section "sd.cpp integration": F32 or packed input).
 * Every distinct input scale
 * gets one quantization pass (all alpha = 1 linears share one packed tensor,
 * as the page prescribes; linears with equal alpha != 1 also share, which
 * gives the same bits as separate passes); then one grouped GEMM launch
 * covers every linear, each reading the packed tensor of its scale.  The
 * descriptors' Qx and s_x must be NULL.
 *
 * A power-of-two input scale 2^k with |k| <= 16 counts as alpha = 1: such a
 * linear reads the alpha = 1 packed tensor and its reconstruction skips the
 * division.  Multiplying by 2^k before the rotation and dividing by it after
 * are both exact, and binary32 rounding commutes with the scaling, so the
 * output bits are those of its own pass whenever the inputs meet the
 * quantizer's contract (each |x| zero or in [2^-100, 2^100]) and the
 * reconstruction's products stay in the normal range (an extension beyond
 * the pages, which give every alpha != 1 its own pass).
 *
 * descs is host memory, 1 <= n <= 16; workspace >= convrot_workspace_bytes(M,
 * K, number of distinct scales after that folding).  Outputs must not overlap
 * each other, any weight-side input or the workspace. */
int convrot_int8_linear_shared(const void *X, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                               int group_size, int n, const convrot_linear_desc *descs,
                               void *workspace, size_t workspace_bytes, void *stream);

/* A producer fused into the quantization pass: applied to each widened input
 * element before the input scale and the rotation, so that the producer's
 * output never goes to memory.
 *
 * CONVROT_PRE_MODULATE (page "ggml operator extensions", section "sd.cpp
 * integration": the Modulate operator and its fusion with ConvRot, which takes
 * contiguous per-channel parameters):
 *     x' = (x + x * scale[i]) + shift[i]       i = input feature (column)
 * three separately rounded binary32 operations; shift may be NULL (scale-only
 * modulation, no add).  scale and shift are device vectors of K floats shared
 * by every row, 16-byte aligned.
 *
 * CONVROT_PRE_RMSNORM_MODULATE (same page and section: the RMSNorm ->
 * Mul(weight) -> Mul(modulation) -> Add -> Add(shift) -> ConvRot fusion) puts
 * RMSNorm -> Mul(weight) ahead of the Modulate above.  The page does not
 * spell out RMSNorm's arithmetic; per row, with x the widened input:
 *     S = sum of fl(x * x): pairwise within each block of 64 consecutive
 *         features (adjacent pairs, then pairs of those sums, ...), then the
 *         K/64 block sums added left to right
 *     r = fl(1 / fl(sqrt(fl(fl(S / K) + eps))))     (correctly rounded)
 *     x' = fl(x * r), then fl(x' * norm_weight[i]) when norm_weight is given
 * and then Modulate with scale and shift, which are both optional here (no
 * scale: no modulation; shift requires scale).  eps is finite and >= 0;
 * inputs whose squares or sums overflow binary32 are outside the contract.
 * Rows are limited to half the quantizer's K (32768 when K % 256 == 0), else
 * CONVROT_EUNSUPPORTED.
 *
 * CONVROT_PRE_NORM_MUL (same page and section: the Norm -> Mul -> ConvRot
 * fusion; the page names the chain only): Norm divides the deviations from
 * the row mean by the root of the row variance plus eps, with no affine part,
 * and Mul multiplies by the per-channel norm_weight when given.  Per row,
 * with x the widened input and sums taken in RMSNorm's order above:
 *     mean = fl(S1 / K),  S1 = sum of x
 *     d    = fl(x - mean)
 *     r    = fl(1 / fl(sqrt(fl(fl(S2 / K) + eps)))),  S2 = sum of fl(d * d)
 *     x'   = fl(d * r), then fl(x' * norm_weight[i]) when norm_weight is given
 * scale and shift must be NULL (no Modulate in this chain); eps and the row
 * limit as for RMSNORM_MODULATE.  A row whose values are all equal has d = 0
 * and gives zeros for eps > 0 (NaN for eps = 0, outside the contract).
 *
 * CONVROT_PRE_GATED_ACT (same page and section: SiLU/Sigmoid -> Mul ->
 * ConvRot, and SwiGLU -> ConvRot with packed, swapped or separate gate/up
 * inputs): with g the quantizer's input X and u = up[r][i], a second tensor
 * of X's dtype and row stride ld_up (elements; ld_up * element size a
 * multiple of 16, up 16-byte aligned):
 *     sigmoid(g) = fl(1 / fl(1 + e)),  e = exp(-g) correctly rounded
 *     act = CONVROT_ACT_SIGMOID: a = sigmoid(g)
 *     act = CONVROT_ACT_SILU:    a = fl(g * sigmoid(g))
 *     x' = fl(a * u)
 * A packed [gate | up] row of 2K features is X = base, up = base + K with
 * ldx = ld_up = 2K (swapped: the other way round).  up may overlap X; packed
 * must not overlap it.  Same row limit as RMSNORM_MODULATE. */
typedef enum {
    CONVROT_PRE_NONE = 0,
    CONVROT_PRE_MODULATE = 1,
    CONVROT_PRE_RMSNORM_MODULATE = 2,
    CONVROT_PRE_GATED_ACT = 3,
    CONVROT_PRE_NORM_MUL = 4
} convrot_pre_kind;

typedef enum { CONVROT_ACT_SILU = 1, CONVROT_ACT_SIGMOID = 2 } convrot_act;

typedef struct {
    int kind;                  /* convrot_pre_kind */
    const float *scale;        /* MODULATE: [K] (device), required; RMSNORM_MODULATE: [K] or NULL */
    const float *shift;        /* [K] (device) or NULL */
    const float *norm_weight;  /* RMSNORM_MODULATE, NORM_MUL: [K] (device) or NULL */
    float eps;                 /* RMSNORM_MODULATE: added to the mean square; NORM_MUL: to the variance */
    const void *up;            /* GATED_ACT: [M][ld_up] (device), X's dtype */
    int64_t ld_up;             /* GATED_ACT: elements, >= K */
    int act;                   /* GATED_ACT: convrot_act */
} convrot_pre;

/* convrot_quantize_rows with a producer.  pre may be NULL or of kind
 * CONVROT_PRE_NONE (then identical to convrot_quantize_rows).  CONVROT_EINVAL
 * for a MODULATE descriptor without scale, a shift without scale, a
 * NORM_MUL descriptor with scale or shift, a negative or non-finite eps, or
 * misaligned vectors (16 bytes); CONVROT_EUNSUPPORTED
 * for an unknown kind; CONVROT_EOVERLAP if packed overlaps X or a vector. */
int convrot_quantize_rows_pre(const void *X, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                              const convrot_pre *pre, int group_size, float input_scale,
                              void *packed, void *stream);

/* convrot_int8_linear_shared with a producer applied in every quantization
 * pass (same rules for pre as above).  The workspace must not overlap the
 * producer's vectors; an output may alias them (they are consumed before any
 * output is written), like X. */
int convrot_int8_linear_shared_pre(const void *X, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                                   const convrot_pre *pre, int group_size, int n,
                                   const convrot_linear_desc *descs, void *workspace,
                                   size_t workspace_bytes, void *stream);

/* The raw int32 accumulator A = Q_x Q_w^T of page "INT8 Convrot
 * Safetensors", section "Runtime activation quantization" (same contraction
 * kernel as
 * int8_linear, with the reconstruction replaced by an int32 store); for
 * checking the contraction bit for bit.  A is [M][N] int32. */
int convrot_int8_gemm_i32(const int8_t *Qx, const int8_t *Qw, int64_t M, int64_t K, int64_t N,
                          int32_t *A, void *stream);

/* An epilogue applied after the reconstruction, before the output cast.
 *
 * CONVROT_POST_GATED_RESIDUAL (page "ggml operator extensions", section
 * "sd.cpp integration": INT8 GEMM -> [Scale] -> Mul(gate) -> Add(residual),
 * separate FP32 rounding of the gate multiplication and the residual
 * addition):
 *     y' = fl(fl(fl(y * scale) * gate[o]) + residual[r][o])
 * where the scale multiply happens only when scale != 1, gate is a device
 * vector of N floats shared by every row (4-byte aligned) and residual is a
 * device [M][ld_residual] tensor in the output dtype (bf16 widened exactly).
 * The residual may be Y itself (same base and row stride: an exact in-place
 * residual); any other overlap with Y, or a gate overlapping Y, is
 * CONVROT_EOVERLAP.  The chain's optional [Concat] needs no kernel of its
 * own: Y and ldy place the rows in their slice of the concatenated tensor
 * (Y at the slice's first element, ldy the full row length), and nothing
 * outside the M x N slice is written. */
typedef enum { CONVROT_POST_NONE = 0, CONVROT_POST_GATED_RESIDUAL = 1 } convrot_post_kind;

typedef struct {
    int kind;               /* convrot_post_kind */
    float scale;            /* GATED_RESIDUAL: scalar multiply first (1 = none) */
    const float *gate;      /* GATED_RESIDUAL: [N] (device) */
    const void *residual;   /* GATED_RESIDUAL: [M][ld_residual] (device), output dtype */
    int64_t ld_residual;    /* elements, >= N */
} convrot_post;

/* int8_linear followed by an epilogue (post may be NULL or of kind
 * CONVROT_POST_NONE: then identical to int8_linear).  CONVROT_EINVAL for a
 * GATED_RESIDUAL descriptor with a missing or misaligned gate or residual, a
 * row stride below N or a non-finite scale; CONVROT_EUNSUPPORTED for an
 * unknown kind. */
int int8_linear_post(const int8_t *Qx, const float *s_x, int64_t M, int64_t K, const int8_t *Qw,
                     const float *s_w, const float *bias, int64_t N, float input_scale,
                     const convrot_post *post, void *Y, int y_dtype, int64_t ldy, void *stream);

/* Dual GEMM with a SwiGLU epilogue on one packed input (page "ggml operator
 * extensions", section "sd.cpp integration": GEMM -> SwiGLU [-> ConvRot],
 * gate and up weights in separate allocations, with their own weight scales,
 * no bias):
 *     g = fl(fl(fl(float(Q_x Qw_gate^T)) * s_x) * s_w_gate) [/ input_scale]
 *     u = fl(fl(fl(float(Q_x Qw_up^T)) * s_x) * s_w_up) [/ input_scale]
 *     Y = fl(silu(g) * u),  silu(g) = fl(g * fl(1 / fl(1 + exp(-g))))
 * with exp correctly rounded (the one of CONVROT_PRE_GATED_ACT), then one
 * cast to y_dtype.  Both weight tensors are [N][K] int8 (16-byte aligned);
 * the scales are nullable (1).  Y is [M][ldy]; the same rules as int8_linear
 * for everything else.  Quantize Y with convrot_quantize_rows for the
 * optional ConvRot of the result. */
int int8_swiglu_linear(const int8_t *Qx, const float *s_x, int64_t M, int64_t K,
                       const int8_t *Qw_gate, const float *s_w_gate, const int8_t *Qw_up,
                       const float *s_w_up, int64_t N, float input_scale, void *Y, int y_dtype,
                       int64_t ldy, void *stream);

/* 4-bit weights, format convrot_w4a4 (page "INT8 Convrot Safetensors",
 * section "Packed INT4 convrot"): W4 is [N][K/2] bytes, feature k of output o
 * in byte o*K/2 + k/2, low nibble for even k, high nibble for odd k, each a
 * two's-complement value in -8..7; s_w is the F32 per-output weight scale.
 * Activations are the INT8 convrot packed tensor as for int8_linear (the same
 * packed tensor may feed INT8 and 4-bit linears).  Same reconstruction and
 * conventions as int8_linear; W4 16-byte aligned; K % 64 == 0 and
 * K <= 132096 (the contraction runs on 16 times the weights, exactly, in
 * int32), else CONVROT_EUNSUPPORTED / CONVROT_EOVERFLOW. */
int int4_linear(const int8_t *Qx, const float *s_x, int64_t M, int64_t K, const uint8_t *W4,
                const float *s_w, const float *bias, int64_t N, float input_scale, void *Y,
                int y_dtype, int64_t ldy, void *stream);

/* The raw int32 accumulator A = Q_x W^T for 4-bit weights W (same contraction
 * kernel as int4_linear); A is [M][N] int32. */
int convrot_int4_gemm_i32(const int8_t *Qx, const uint8_t *W4, int64_t M, int64_t K, int64_t N,
                          int32_t *A, void *stream);

/* The correctly rounded binary32 exp of CONVROT_PRE_GATED_ACT, elementwise:
 * y[i] = exp(x[i]) for n device floats (0 below -104, +inf above 89; inputs
 * finite).  y may be x itself (in place); any other overlap is
 * CONVROT_EOVERLAP.  Exposed so that the device build of the exp can be
 * checked against a reference directly. */
int convrot_expf(const float *x, float *y, int64_t n, void *stream);

/* Static, human-readable text for a status code (errors are reported, never
 * retried or hidden behind a fallback: page "ggml operator extensions",
 * section "Kernel selection"). */
const char *convrot_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* CONVROT_H */
