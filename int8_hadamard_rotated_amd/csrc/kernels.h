// Internal launch interface between the C ABI (convrot_api.cpp) and the
// gfx950 kernels (quantize.hip, gemm_i8.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace convrot_detail {

// Orders a wave's earlier LDS writes before its later LDS reads, where lanes
// read what other lanes of the same wave wrote (wave-private staging regions).
// The hardware completes one wave's LDS operations in order; the fences keep
// the compiler from moving a read above the writes it depends on.
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------- quantize
// Largest row (in elements) the quantizer handles for a given K: one
// workgroup per group of rows, at most 256 quads of 4 lanes per row (128 with
// the RMSNorm producer); a quad covers 256, 128 or 64 elements.
inline int64_t quantize_max_k(int64_t K, bool rmsnorm = false)
{
    const int64_t quads = rmsnorm ? 128 : 256;
    if (K % 256 == 0)
        return quads * 256;
    if (K % 128 == 0)
        return quads * 128;
    return quads * 64;
}

// Producer applied to each widened input element before the rotation.
enum PreKind : int { kPreNone = 0, kPreModulate = 1, kPreRmsNormModulate = 2, kPreGatedAct = 3, kPreNormMul = 4 };
enum ActKind : int { kActSilu = 1, kActSigmoid = 2 };

struct PreOp {
    int kind = kPreNone;
    const float *scale = nullptr;         // per-channel [K] or null (no modulation), 16-byte aligned
    const float *shift = nullptr;         // per-channel [K] or null (needs scale)
    const float *norm_weight = nullptr;   // kPreRmsNormModulate, kPreNormMul: per-channel [K] or null
    float eps = 0.0f;                     // kPreRmsNormModulate, kPreNormMul
    const void *up = nullptr;             // kPreGatedAct: [M][ld_up], X's dtype
    int64_t ld_up = 0;
    int act = 0;                          // kPreGatedAct: ActKind
};

// y[i] = correctly rounded exp(x[i]) (the gated activation's exp).
hipError_t launch_expf(const float *x, float *y, int64_t n, hipStream_t stream);

// Launch the (producer +) rotate + row-max + quantize + pack kernel.
// Arguments are already validated (see convrot_quantize_rows_pre).
hipError_t launch_quantize(const void *X, int x_dtype, int64_t M, int64_t K, int64_t ldx, int G,
                           float alpha, const PreOp &pre, void *packed, hipStream_t stream);

// Several input scales of one X without a producer: packed[i] receives the
// bytes of launch_quantize with alpha[i].  Binary32 rows that the staged
// kernel takes are read once per kMaxPassScales scales; other rows get one
// pass per scale.
constexpr int kMaxPassScales = 2;
struct ScaleOuts {
    int n;
    float alpha[kMaxPassScales];
    int8_t *Q[kMaxPassScales];
    float *S[kMaxPassScales];
};
hipError_t launch_quantize_scales(const void *X, int x_dtype, int64_t M, int64_t K, int64_t ldx, int G,
                                  int n, const float *alpha, void *const *packed, hipStream_t stream);

// ------------------------------------------------------------------- GEMM
constexpr int kMaxLinears = 16;

enum OutKind : int { kOutF32 = 0, kOutBF16 = 1, kOutI32 = 2 };

struct GemmLinear {
    const int8_t *Qx;    // [M][K] codes this linear reads (row stride K); null: GemmProblem's
    const float *s_x;    // [M] their row scales (with Qx)
    const int8_t *Qw;    // [N][K]
    const float *s_w;    // [N] or null
    const float *bias;   // [N] or null
    void *Y;             // [M][ldy]
    int64_t N;
    int64_t ldy;
    float alpha;         // divisor; 1 = none
    int out_kind;        // OutKind
    int vec_store;       // Y row starts allow 4-element vector stores
    int post;            // 1: gated residual after the reconstruction
    float post_scale;    // post: scalar multiply first (1 = none)
    const float *gate;   // post: per-channel gate [N]
    const void *residual;// post: [M][ld_res] in the output dtype (may equal Y exactly)
    int64_t ld_res;
    int res_vec;         // post: residual row starts allow 4-element vector loads
    int glu;             // 1: SwiGLU pair, Y = silu(gate reconstruction) * up reconstruction
    const int8_t *Qw_up; // glu: up weights [N][K] (Qw holds the gate weights)
    const float *s_w_up; // glu: [N] or null
    int tiles_n;         // filled by the launcher
    int tile_begin;      // filled by the launcher: first linear tile index
};

struct GemmProblem {
    const int8_t *Qx;    // [M][K], row stride K: the input of every linear whose own Qx is null
    const float *s_x;    // [M]
    int64_t M;
    int64_t K;
    int w_bits;          // 8: Qw int8 [N][K]; 4: Qw packed 4-bit [N][K/2] (low nibble first)
    int n_lin;
    GemmLinear lin[kMaxLinears];
};

// Launch one grouped contraction + reconstruction over all linears of `p`.
hipError_t launch_gemm(GemmProblem p, hipStream_t stream);

// ------------------------------------------------------- static workspace
// A library-owned device buffer of this many bytes (one per GPU, held until
// the process ends) for callers that cannot allocate a workspace.
constexpr size_t kStaticWorkspaceBytes = (size_t)64 << 20;

// The current device's copy of that buffer.  Its address is looked up once
// per device (the first call with that device current); no allocation.
hipError_t static_workspace(void **ptr);

}  // namespace convrot_detail
