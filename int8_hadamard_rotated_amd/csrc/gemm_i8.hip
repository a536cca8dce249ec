// INT8 x INT8 -> INT32 contraction on CDNA4 MFMA with the reconstruction
// fused into the epilogue (gfx950).
//
//   A[r, o] = sum_i Q_x[r, i] * Q_w[o, i]                     (exact int32)
//   Y[r, o] = fl(fl(fl(fl(float(A)) * s_x[r]) * s_w[o]) / alpha) + b[o]
//
// page "INT8 Convrot Safetensors", section "How INT8 convrot works" (the
// accumulation and the reconstruction) and page "ggml operator extensions",
// section "sd.cpp integration" (the order float(dot) * X_scale * W_scale +
// bias; weight scale and bias may be absent).  The unscale by the input scale
// before the bias follows the convrot page's last paragraph of that section.
//
// Both operands are K-contiguous.  A workgroup of 4 waves computes a BM x BN
// tile; waves form a 2 x 2 grid, each owning (BM/2) x (BN/2) as 16 x 16 MFMA
// blocks (v_mfma_i32_16x16x64_i8, 64 K-bytes per instruction).  K advances in
// BK-byte steps through two LDS buffers: the next step's global loads are in
// flight while the current step's MFMAs run.  LDS rows are padded by 16 bytes
// so that the 16-byte fragment reads of 8 consecutive rows hit distinct banks.
//
// The integer sum is exact whatever the order of K, so the lane-to-K mapping
// inside an MFMA only has to agree between the two operands, which are read
// with the same pattern.  Several linears sharing one Q_x run in one launch:
// the tile index space is the concatenation of every linear's tile grid.
// Workgroups are renumbered so that each XCD (round-robin dispatch over 8)
// receives a contiguous range of tiles, walked in groups of 4 tile rows, so
// that tiles running together on one XCD share operand panels in its L2.
#pragma clang fp contract(off)

#include "kernels.h"

namespace convrot_detail {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kXcds = 8;
constexpr int kGroupM = 4;

template <int BM, int BN, int BK>
struct Tile {
    static constexpr int kWaveM = BM / 2;
    static constexpr int kWaveN = BN / 2;
    static constexpr int kTM = kWaveM / 16;
    static constexpr int kTN = kWaveN / 16;
    static constexpr int kStride = BK + 16;               // LDS bytes per row
    static constexpr int kChunksPerRow = BK / 16;
    static constexpr int kAChunks = BM * kChunksPerRow / kThreads;
    static constexpr int kBChunks = BN * kChunksPerRow / kThreads;
    static constexpr int kStageBytes = (BM + BN) * kStride;
    static_assert(BM * kChunksPerRow % kThreads == 0 && BN * kChunksPerRow % kThreads == 0, "");
    static_assert(BK % 64 == 0, "");
};

__device__ __forceinline__ uint16_t bf16_rne(float t)
{
    unsigned u = __builtin_bit_cast(unsigned, t);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

template <int BM, int BN, int BK>
__global__ __launch_bounds__(kThreads, 1) void gemm_i8_kernel(GemmProblem p, int tiles_m,
                                                              int total_tiles)
{
    using T = Tile<BM, BN, BK>;
    __shared__ __attribute__((aligned(16))) int8_t lds[2 * T::kStageBytes];

    // ---- tile assignment: contiguous tile range per XCD, then group-M order
    const int bid = blockIdx.x;
    const int per_xcd = total_tiles / kXcds, extra = total_tiles % kXcds;
    const int xcd = bid % kXcds, slot = bid / kXcds;
    const int lin = xcd * per_xcd + (xcd < extra ? xcd : extra) + slot;
    int d = 0;
    while (d + 1 < p.n_lin && lin >= p.lin[d + 1].tile_begin)
        ++d;
    const GemmLinear &L = p.lin[d];
    const int local = lin - L.tile_begin;
    const int group = local / (kGroupM * L.tiles_n);
    const int first_m = group * kGroupM;
    const int gsize = (tiles_m - first_m) < kGroupM ? (tiles_m - first_m) : kGroupM;
    const int in_group = local - group * kGroupM * L.tiles_n;
    const int tm = first_m + in_group % gsize;
    const int tn = in_group / gsize;

    const int64_t M = p.M, K = p.K, N = L.N;
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    // ---- global -> LDS chunk assignment (16 bytes per chunk)
    const int8_t *a_src[T::kAChunks];
    int a_dst[T::kAChunks];
#pragma unroll
    for (int i = 0; i < T::kAChunks; ++i) {
        const int c = tid + kThreads * i;
        const int r = c / T::kChunksPerRow, kc = c % T::kChunksPerRow;
        const int64_t gr = (m0 + r < M) ? m0 + r : M - 1;   // clamped; rows >= M are not stored
        a_src[i] = p.Qx + gr * K + 16 * kc;
        a_dst[i] = r * T::kStride + 16 * kc;
    }
    const int8_t *b_src[T::kBChunks];
    int b_dst[T::kBChunks];
#pragma unroll
    for (int i = 0; i < T::kBChunks; ++i) {
        const int c = tid + kThreads * i;
        const int r = c / T::kChunksPerRow, kc = c % T::kChunksPerRow;
        const int64_t gr = (n0 + r < N) ? n0 + r : N - 1;
        b_src[i] = L.Qw + gr * K + 16 * kc;
        b_dst[i] = BM * T::kStride + r * T::kStride + 16 * kc;
    }

    v4i ra[T::kAChunks], rb[T::kBChunks];
    auto gload = [&](int64_t k0) {
#pragma unroll
        for (int i = 0; i < T::kAChunks; ++i)
            ra[i] = *reinterpret_cast<const v4i *>(a_src[i] + k0);
#pragma unroll
        for (int i = 0; i < T::kBChunks; ++i)
            rb[i] = *reinterpret_cast<const v4i *>(b_src[i] + k0);
    };
    auto swrite = [&](int buf) {
        int8_t *base = lds + buf * T::kStageBytes;
#pragma unroll
        for (int i = 0; i < T::kAChunks; ++i)
            *reinterpret_cast<v4i *>(base + a_dst[i]) = ra[i];
#pragma unroll
        for (int i = 0; i < T::kBChunks; ++i)
            *reinterpret_cast<v4i *>(base + b_dst[i]) = rb[i];
    };

    v4i acc[T::kTM][T::kTN];
#pragma unroll
    for (int i = 0; i < T::kTM; ++i)
#pragma unroll
        for (int j = 0; j < T::kTN; ++j)
            acc[i][j] = v4i{0, 0, 0, 0};

    // fragment read offsets: lane -> (row within 16, 16-byte K slice)
    const int frag_row = lane & 15, frag_k = 16 * (lane >> 4);
    const int a_frag = (wm * T::kWaveM + frag_row) * T::kStride + frag_k;
    const int b_frag = BM * T::kStride + (wn * T::kWaveN + frag_row) * T::kStride + frag_k;

    const int64_t ksteps = K / BK;
    gload(0);
    swrite(0);
    __syncthreads();
    for (int64_t ks = 0; ks < ksteps; ++ks) {
        const int buf = (int)(ks & 1);
        if (ks + 1 < ksteps)
            gload((ks + 1) * BK);
        const int8_t *base = lds + buf * T::kStageBytes;
#pragma unroll
        for (int kk = 0; kk < BK; kk += 64) {
            v4i fa[T::kTM], fb[T::kTN];
#pragma unroll
            for (int i = 0; i < T::kTM; ++i)
                fa[i] = *reinterpret_cast<const v4i *>(base + a_frag + i * 16 * T::kStride + kk);
#pragma unroll
            for (int j = 0; j < T::kTN; ++j)
                fb[j] = *reinterpret_cast<const v4i *>(base + b_frag + j * 16 * T::kStride + kk);
#pragma unroll
            for (int i = 0; i < T::kTM; ++i)
#pragma unroll
                for (int j = 0; j < T::kTN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
        if (ks + 1 < ksteps)
            swrite(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue.  The MFMA 16x16 result block gives lane l column l%16
    // and rows 4*(l/16) + v.  Each wave stages one 16-row slice of its
    // accumulators in LDS (the operand buffers are free by now), then reads it
    // back four consecutive columns per lane, so that the reconstruction and
    // the stores work on 4-wide rows (one 16- or 8-byte store per lane).
    constexpr int kStageStride = T::kWaveN + 4;                 // int32 per staged row
    constexpr int kColQuads = T::kWaveN / 4;
    constexpr int kSlots = 16 * kColQuads / 64;
    static_assert(4 * 16 * kStageStride * 4 <= 2 * T::kStageBytes, "staging fits in LDS");
    int32_t *stage = reinterpret_cast<int32_t *>(lds) + wave * 16 * kStageStride;
    const int kind = L.out_kind;
    const float alpha = L.alpha;
    const float *s_w = L.s_w;
    const float *bias = L.bias;
    void *Yv = L.Y;
    const int64_t ldy = L.ldy;
    const bool vec = L.vec_store != 0;
    const int row_in = 4 * (lane >> 4), col_in = lane & 15;
#pragma unroll
    for (int i = 0; i < T::kTM; ++i) {
        __syncthreads();
#pragma unroll
        for (int j = 0; j < T::kTN; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                stage[(row_in + v) * kStageStride + j * 16 + col_in] = acc[i][j][v];
        __syncthreads();
        for (int sl = 0; sl < kSlots; ++sl) {
            const int slot = lane + 64 * sl;
            const int rr = slot / kColQuads, cq = slot % kColQuads;
            const v4i a = *reinterpret_cast<const v4i *>(stage + rr * kStageStride + 4 * cq);
            const int64_t r = m0 + wm * T::kWaveM + i * 16 + rr;
            const int64_t o = n0 + wn * T::kWaveN + 4 * cq;
            if (r >= M || o >= N)
                continue;
            const bool full = vec && (o + 4 <= N);
            if (kind == kOutI32) {
                int32_t *y = static_cast<int32_t *>(Yv) + r * ldy + o;
                if (full) {
                    *reinterpret_cast<v4i *>(y) = a;
                } else {
                    for (int e = 0; e < 4 && o + e < N; ++e)
                        y[e] = a[e];
                }
                continue;
            }
            const float sx = p.s_x[r];
            float t[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t oe = (o + e < N) ? o + e : N - 1;
                float x = (float)a[e];
                x = x * sx;
                if (s_w)
                    x = x * s_w[oe];
                if (alpha != 1.0f)
                    x = __fdiv_rn(x, alpha);
                if (bias)
                    x = x + bias[oe];
                t[e] = x;
            }
            if (kind == kOutF32) {
                float *y = static_cast<float *>(Yv) + r * ldy + o;
                if (full) {
                    *reinterpret_cast<v4f *>(y) = v4f{t[0], t[1], t[2], t[3]};
                } else {
                    for (int e = 0; e < 4 && o + e < N; ++e)
                        y[e] = t[e];
                }
            } else {
                uint16_t *y = static_cast<uint16_t *>(Yv) + r * ldy + o;
                const uint16_t h0 = bf16_rne(t[0]), h1 = bf16_rne(t[1]);
                const uint16_t h2 = bf16_rne(t[2]), h3 = bf16_rne(t[3]);
                if (full) {
                    v2u w;
                    w.x = (unsigned)h0 | ((unsigned)h1 << 16);
                    w.y = (unsigned)h2 | ((unsigned)h3 << 16);
                    *reinterpret_cast<v2u *>(y) = w;
                } else {
                    const uint16_t hs[4] = {h0, h1, h2, h3};
                    for (int e = 0; e < 4 && o + e < N; ++e)
                        y[e] = hs[e];
                }
            }
        }
    }
}

template <int BM, int BN, int BK>
hipError_t launch_tiled(GemmProblem p, hipStream_t stream)
{
    const int tiles_m = (int)((p.M + BM - 1) / BM);
    int total = 0;
    for (int d = 0; d < p.n_lin; ++d) {
        p.lin[d].tiles_n = (int)((p.lin[d].N + BN - 1) / BN);
        p.lin[d].tile_begin = total;
        total += tiles_m * p.lin[d].tiles_n;
    }
    if (total == 0)
        return hipSuccess;
    hipLaunchKernelGGL((gemm_i8_kernel<BM, BN, BK>), dim3(total), dim3(kThreads), 0, stream, p,
                       tiles_m, total);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(GemmProblem p, hipStream_t stream)
{
    // Large grids use 256 x 256 tiles; grids too small to cover the 256 CUs
    // with them fall back to 128 x 128.
    int64_t big = 0;
    for (int d = 0; d < p.n_lin; ++d)
        big += ((p.M + 255) / 256) * ((p.lin[d].N + 255) / 256);
    if (big >= 256)
        return launch_tiled<256, 256, 64>(p, stream);
    return launch_tiled<128, 128, 64>(p, stream);
}

}  // namespace convrot_detail
