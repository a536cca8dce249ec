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
// Structure.  Both operands are K-contiguous.  A workgroup of WM x WN waves
// computes a BM x BN tile; wave (wm, wn) owns (BM/WM) x (BN/WN) as 16 x 16
// blocks of v_mfma_i32_16x16x64_i8 (64 K-bytes per instruction).  K advances
// in 64-byte steps through a 4-stage LDS ring filled by direct buffer-to-LDS
// loads issued three steps ahead; fragments are read from LDS one step ahead
// into registers.  The integer sum is exact whatever the order of K, so the
// lane-to-K mapping inside an MFMA only has to agree between the two
// operands, which are read with the same pattern.
//
// Several linears run in one launch, each reading the shared Q_x or a packed
// tensor of its own (one per input scale): the tile index space is
// the concatenation of every linear's tile grid.  Workgroups are renumbered
// so that each XCD (round-robin dispatch over 8) receives a contiguous range
// of tiles, walked in groups of 4 tile rows, so that tiles running together
// on one XCD share operand panels in its L2.
#pragma clang fp contract(off)

#include "expf_cr.h"
#include "kernels.h"

#include <type_traits>

namespace convrot_detail {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

constexpr int kXcds = 8;
constexpr int kGroupM = 4;
constexpr int kBufferFlags = 0x00020000;   // raw buffer, 32-bit data format
constexpr int kBK = 64;                    // K bytes per step (one MFMA K)

template <int BM, int BN, int WM, int WN, int STAGES, int WB>
struct Tile {
    static constexpr int kWaves = WM * WN;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kWaveM = BM / WM;
    static constexpr int kWaveN = BN / WN;
    static constexpr int kTM = kWaveM / 16;                // A blocks per wave
    static constexpr int kTN = kWaveN / 16;                // B blocks per wave
    static constexpr int kStride = kBK;                    // LDS bytes per A row (swizzled)
    static constexpr int kStrideB = WB == 4 ? kBK / 2 : kBK;   // LDS bytes per B row (packed when 4-bit)
    static constexpr int kABytes = BM * kStride;
    static constexpr int kStageBytes = kABytes + BN * kStrideB;
    static constexpr int kStages = STAGES;                 // LDS ring depth
    static constexpr int kRowsPerDmaB = 1024 / kStrideB;   // B rows per 1 KB DMA instruction
    static constexpr int kDmaA = BM / 16, kDmaB = BN / kRowsPerDmaB;
    static constexpr int kDma = kDmaA + kDmaB;             // DMA instructions per step
    static constexpr int kLoads = (kDma + kWaves - 1) / kWaves;   // at most, per wave per step
    // 4-bit weights: two slots of expanded B rows (64 bytes each, the int8
    // layout) after the ring; each step's packed rows are expanded once
    static constexpr int kExpOff = kStages * kStageBytes;
    static constexpr int kExpSlot = WB == 4 ? BN * kBK : 0;
    static constexpr int kScaleOff = kExpOff + 2 * kExpSlot;  // s_x [BM], s_w, bias, gate [BN]
    static constexpr int kLdsBytes = kScaleOff + 4 * (BM + 3 * BN);
    // steps whose DMA must have landed beyond the next one at an iteration's
    // top: 4-bit weights expand the step after next there
    static constexpr int kAhead = WB == 4 ? 1 : 0;
    static_assert(WB == 8 || WB == 4, "weight bits");
    static_assert(BN % kRowsPerDmaB == 0, "whole B DMA blocks");
    static_assert(BM % 16 == 0 && kWaveM % 16 == 0 && kWaveN % 16 == 0, "");
    static_assert(kLoads <= kTM, "at most one DMA load per MFMA group");
    static_assert(STAGES >= 4 + kAhead, "ring depth");
    static_assert(WB == 8 || BN == 16 * kWaves, "one packed 8-byte chunk per lane and step");
    static_assert((BM + 3 * BN) % 64 == 0, "64-float scale segments");
    static_assert(kLdsBytes <= 160 * 1024, "gfx950 LDS");
};

// Raw buffer descriptor (stride 0, 32-bit data format) over [base, base + bytes).
__device__ __forceinline__ v4u buffer_rsrc(const void *base, uint32_t bytes)
{
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    return v4u{(uint32_t)a, (uint32_t)(a >> 32) & 0xFFFFu, bytes, (uint32_t)kBufferFlags};
}

// 16 bytes per lane from buffer offset voff + soff into LDS at lds + 16 * lane
// (buffer_load_dwordx4 ... lds).  Issued as inline assembly so that the
// compiler does not hold its LDS reads behind these loads; the matching waits
// are explicit (wait_vmcnt).  Offsets outside the descriptor read as zero.
__device__ __forceinline__ void dma_x4(v4u rsrc, int voff, int soff, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "s"(soff), "s"(lds)
                 : "memory", "m0");
}

// 4 bytes per lane from buffer offset voff + soff into LDS at lds + 4 * lane.
__device__ __forceinline__ void dma_x1(v4u rsrc, int voff, int soff, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dword %0, %1, %2 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "s"(soff), "s"(lds)
                 : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "");
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// XOR swizzle of the four 16-byte K chunks of an LDS row.  The fragment read
// of one MFMA block has lane l read row l%16, chunk l/16; with chunk slot
// c ^ ((r >> 1) & 3) that read pattern measures free of LDS bank conflicts on
// gfx950 (SQ_LDS_BANK_CONFLICT = 0), unlike unswizzled, row-padded or
// low-bit-XOR layouts, which cost two LDS passes per read.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 3; }

// Wait until at most n of this wave's DMA loads are outstanding (0 <= n,
// values above MAXN wait for MAXN).
template <int MAXN>
__device__ __forceinline__ void wait_vmcnt_le(int n)
{
    if constexpr (MAXN <= 0) {
        wait_vmcnt<0>();
    } else {
        if (n >= MAXN)
            wait_vmcnt<MAXN>();
        else
            wait_vmcnt_le<MAXN - 1>(n);
    }
}

// Packed 4-bit weights: 8 bytes (16 two's-complement nibbles, the even
// feature in the low nibble) -> 16 int8 lanes of an MFMA operand, each holding
// 16 times its weight (the nibble moved to the top of its byte, which is the
// same two's-complement value scaled by 16).  The contraction then yields
// exactly 16 A; the epilogue shifts it back.
__device__ __forceinline__ v4i expand_w4(v2u p)
{
    const unsigned lo0 = (p.x << 4) & 0xF0F0F0F0u, hi0 = p.x & 0xF0F0F0F0u;
    const unsigned lo1 = (p.y << 4) & 0xF0F0F0F0u, hi1 = p.y & 0xF0F0F0F0u;
    // byte i of the result: element i; from {hi, lo} pick lo.b0 hi.b0 lo.b1 hi.b1 / lo.b2 hi.b2 lo.b3 hi.b3
    return v4i{(int)__builtin_amdgcn_perm(hi0, lo0, 0x05010400u), (int)__builtin_amdgcn_perm(hi0, lo0, 0x07030602u),
               (int)__builtin_amdgcn_perm(hi1, lo1, 0x05010400u), (int)__builtin_amdgcn_perm(hi1, lo1, 0x07030602u)};
}

// Epilogue kinds: the plain reconstruction, with the gated residual after it,
// or SwiGLU (silu of one reconstruction times another).
enum EpiKind : int { kEpiPlain = 0, kEpiPost = 1, kEpiGlu = 2 };

template <int BM, int BN, int WM, int WN, int STAGES, bool DIV, int WB, int EPI>
__global__ __launch_bounds__(64 * WM * WN, 1) void gemm_i8_kernel(
    GemmProblem p, int tiles_m, int total_tiles)
{
    using T = Tile<BM, BN, WM, WN, STAGES, WB>;
    __shared__ __attribute__((aligned(16))) int8_t lds[T::kLdsBytes];

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

    constexpr bool POST = EPI == kEpiPost;
    constexpr bool GLU = EPI == kEpiGlu;
    static_assert(!GLU || WB == 8, "SwiGLU pairs take int8 weights");
    const int64_t M = p.M, K = p.K, N = L.N;
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    // SwiGLU: the tile's BN columns are BN/2 outputs.  In every wave's column
    // block the first half are gate rows and the second half up rows of the
    // same outputs, so a lane holds the gate and up accumulators of one
    // output column (blocks j and j + kTN/2).
    const int64_t n0o = GLU ? (int64_t)tn * (BN / 2) : n0;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // (lets the compiler resolve which operand a wave's DMA instruction
    // moves, where the instruction count is a multiple of the wave count)
    __builtin_assume(wave >= 0 && wave < T::kWaves);
    const int wm = wave / WN, wn = wave % WN;

    // ---- global -> LDS by direct buffer loads.  A stage holds the BM rows
    // of the A tile (64 bytes each) followed by the BN rows of the B tile
    // (64 bytes each, or 32 for packed 4-bit weights).  A DMA instruction moves
    // 1 KB: A instruction g moves rows 16 g .. 16 g + 15 (lane L writes row
    // 16 g + L/4, slot L%4, which receives logical K chunk (L%4) ^ swz(row));
    // a 4-bit B instruction moves 32 packed rows of 32 bytes (lane L writes
    // row L/2, half L%2).  The swizzle only depends on row bits below the
    // block size, so one per-lane offset serves every instruction.  Wave w issues instructions
    // g = kWaves * q + w (g < kDma), one per MFMA group.
    //
    // Each operand tile is addressed through a buffer descriptor that starts
    // at the tile's first row and ends after its last valid row; rows past M
    // (or N) fall outside it and are never stored.
    const int64_t kb = WB == 4 ? K / 2 : K;                   // weight bytes per row
    const int64_t a_rows = (M - m0) < BM ? (M - m0) : BM;
    const int64_t b_span = GLU ? BN / 2 : BN;
    const int64_t b_rows = (N - n0o) < b_span ? (N - n0o) : b_span;
    const v4u a_rsrc = buffer_rsrc(L.Qx + m0 * K, (uint32_t)(a_rows * K));
    const v4u b_rsrc = buffer_rsrc(L.Qw + n0o * kb, (uint32_t)(b_rows * kb));
    const v4u u_rsrc = buffer_rsrc(GLU ? L.Qw_up + n0o * kb : nullptr, GLU ? (uint32_t)(b_rows * kb) : 0u);
    const int ld_row = lane >> 2;
    const int ld_voff = ld_row * (int)K + 16 * ((lane & 3) ^ swz(ld_row));
    const int ld_voff_b = WB == 4 ? (lane >> 1) * (int)kb + 16 * (lane & 1) : ld_voff;
    const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) int8_t *)lds;
    // DMA instructions this wave issues per step
    const int my_loads = (T::kDma - wave + T::kWaves - 1) / T::kWaves;

    auto issue_one = [&](int step, int q) {
        const uint32_t st = lds_base + (uint32_t)(step % T::kStages) * T::kStageBytes;
        const int g = T::kWaves * q + wave;
        if (g < T::kDmaA) {
            dma_x4(a_rsrc, ld_voff, 16 * g * (int)K + step * kBK, st + 1024 * g);
        } else if (g < T::kDma) {
            const int gb = g - T::kDmaA;
            if constexpr (GLU) {
                // 16 tile rows, all gate or all up (a half-block has >= 16 rows)
                const int v0 = T::kRowsPerDmaB * gb;
                const int within = v0 % T::kWaveN;
                const int src = (v0 / T::kWaveN) * (T::kWaveN / 2) + within % (T::kWaveN / 2);
                dma_x4(within < T::kWaveN / 2 ? b_rsrc : u_rsrc, ld_voff_b,
                       src * (int)kb + step * T::kStrideB, st + T::kABytes + 1024 * gb);
            } else {
                dma_x4(b_rsrc, ld_voff_b, T::kRowsPerDmaB * gb * (int)kb + step * T::kStrideB,
                       st + T::kABytes + 1024 * gb);
            }
        }
    };

    // The epilogue's row scales, weight scales and bias go to LDS first, by
    // the same DMA path (64 floats per instruction), so that their latency is
    // hidden behind the whole main loop.  They are older than every operand
    // load, so the first operand wait also covers them.
    const bool want_sx = L.out_kind != kOutI32;
    // (SwiGLU reads its two weight-scale vectors in the epilogue instead)
    const bool has_sw = !GLU && L.s_w != nullptr, has_bias = !GLU && L.bias != nullptr;
    const bool has_post = POST && L.post != 0;
    {
        constexpr int kSeg = (BM + 3 * BN) / 64;
        const v4u sx_rsrc = buffer_rsrc(want_sx ? L.s_x + m0 : nullptr,
                                        want_sx ? (uint32_t)(a_rows * 4) : 0u);
        const v4u sw_rsrc = buffer_rsrc(has_sw ? L.s_w + n0 : nullptr,
                                        has_sw ? (uint32_t)(b_rows * 4) : 0u);
        const v4u bi_rsrc = buffer_rsrc(has_bias ? L.bias + n0 : nullptr,
                                        has_bias ? (uint32_t)(b_rows * 4) : 0u);
        const v4u gt_rsrc = buffer_rsrc(has_post ? L.gate + n0 : nullptr,
                                        has_post ? (uint32_t)(b_rows * 4) : 0u);
#pragma unroll
        for (int q = 0; q < kSeg; ++q) {
            if (q % T::kWaves != wave)
                continue;
            const uint32_t dst = lds_base + T::kScaleOff + 256 * q;
            if (q < BM / 64) {
                if (want_sx)
                    dma_x1(sx_rsrc, 4 * lane, 256 * q, dst);
            } else if (q < (BM + BN) / 64) {
                if (has_sw)
                    dma_x1(sw_rsrc, 4 * lane, 256 * (q - BM / 64), dst);
            } else if (q < (BM + 2 * BN) / 64) {
                if (has_bias)
                    dma_x1(bi_rsrc, 4 * lane, 256 * (q - (BM + BN) / 64), dst);
            } else if (has_post) {
                dma_x1(gt_rsrc, 4 * lane, 256 * (q - (BM + 2 * BN) / 64), dst);
            }
        }
    }

    v4i acc[T::kTM][T::kTN];
#pragma unroll
    for (int i = 0; i < T::kTM; ++i)
#pragma unroll
        for (int j = 0; j < T::kTN; ++j)
            acc[i][j] = v4i{0, 0, 0, 0};

    // fragment reads: lane -> (row lane%16 of a 16-row block, logical chunk
    // lane/16); the swizzle of rows 16*i + lane%16 does not depend on i.
    const int frag_row = lane & 15, frag_chunk = lane >> 4;
    const int frag_slot = 16 * (frag_chunk ^ swz(frag_row));
    const int a_frag0 = (wm * T::kWaveM + frag_row) * T::kStride + frag_slot;
    // B fragments come from the ring (int8 weights) or from the expanded
    // slots (4-bit weights), both in the int8 row layout
    const int b_frag0 = (wn * T::kWaveN + frag_row) * T::kStride + frag_slot;
    auto read_a = [&](int step, int i) {
        return *reinterpret_cast<const v4i *>(lds + (step % T::kStages) * T::kStageBytes + a_frag0 +
                                              i * 16 * T::kStride);
    };
    auto read_b = [&](int step, int j) {
        const int base = WB == 4 ? T::kExpOff + (step & 1) * T::kExpSlot
                                 : (step % T::kStages) * T::kStageBytes + T::kABytes;
        return *reinterpret_cast<const v4i *>(lds + base + b_frag0 + j * 16 * T::kStride);
    };
    // 4-bit expansion: lane l of wave w takes packed row 16 w + l/4, 8-byte
    // chunk l%4 (logical 16-byte K chunk l%4 of the expanded row)
    const int ex_row = 16 * wave + (lane >> 2), ex_chunk = lane & 3;
    const int ex_src = T::kABytes + ex_row * T::kStrideB + 8 * ex_chunk;
    const int ex_dst = T::kExpOff + ex_row * T::kStride + 16 * (ex_chunk ^ swz(ex_row));
    auto read_packed = [&](int step) {
        return *reinterpret_cast<const v2u *>(lds + (step % T::kStages) * T::kStageBytes + ex_src);
    };
    auto write_expanded = [&](int step, v2u pk) {
        *reinterpret_cast<v4i *>(lds + ex_dst + (step & 1) * T::kExpSlot) = expand_w4(pk);
    };

    // ---- main loop, software-pipelined one K-step ahead on fragments.
    // Iteration k multiplies step k from registers (A block i in fa[i], B
    // block j in fb[j]) in row-major (i, j) order.  At its top the wave waits
    // for its own DMA loads of step k+1 and passes the barrier that
    // certifies everyone's; it then reads step k+1's fragments into the same
    // registers as soon as their last use in step k has been issued: fa[i]
    // after A block i's group and fb[j] right after MFMA (kTM-1, j).  That
    // barrier also shows that every wave has consumed step k-1's fragments
    // (it has issued all of iteration k-1's MFMAs), so the DMA loads of step
    // k + S - 1 (S = ring depth), spread one per MFMA group, may overwrite
    // stage (k-1) % S: loads are issued S - 2 iterations before the barrier
    // that needs them.
    //
    // 4-bit weights (kAhead = 1): the barrier at the top of iteration k also
    // certifies step k+2's DMA; each lane then expands its packed chunk of
    // step k+2 into expanded slot k % 2, whose step-k fragments were read in
    // iteration k-1, and the barrier at the top of iteration k+1 publishes
    // it before step k+2's fragments are read.  Steps 0 and 1 are expanded
    // before the loop.  The ring keeps the same two iterations of DMA
    // lookahead with one more stage.
    constexpr int S = T::kStages;
    constexpr int AH = T::kAhead;
    static_assert((S - 2) * T::kLoads < 64, "vmcnt range");
    v4i fa[T::kTM], fb[T::kTN];
    const int ksteps = (int)(K / kBK);
    //
    // Iterations k <= ksteps - S (steady state) have a next step, issue DMA
    // and leave S - 3 - AH steps in flight at the wait: they run a copy of
    // the body with those facts fixed at compile time (no per-step branches);
    // the last S - 1 iterations run the general body.
    auto iteration = [&](int k, auto steady) {
        constexpr bool STEADY = decltype(steady)::value;
        const bool has_next = STEADY || k + 1 < ksteps;
        const bool expand = WB == 4 && (STEADY || k + 2 < ksteps);
        if (has_next) {
            // steps up to k+1+AH must have landed; k+2+AH .. k+S-2 may stay in flight
            if constexpr (STEADY && T::kDma % T::kWaves == 0) {
                wait_vmcnt<(S - 3 - AH) * T::kLoads>();      // every wave issues kLoads per step
            } else {
                int younger = ksteps - k - 2 - AH;
                younger = younger < S - 3 - AH ? younger : S - 3 - AH;
                younger = younger > 0 ? younger : 0;
                wait_vmcnt_le<(S - 3 - AH) * T::kLoads>(younger * my_loads);
            }
            __syncthreads();
        }
        v2u pk{0u, 0u};
        if constexpr (WB == 4) {
            if (expand)
                pk = read_packed(k + 2);
        }
        const int dma_step = k + S - 1;
        const bool dma = STEADY || dma_step < ksteps;
#pragma unroll
        for (int i = 0; i < T::kTM; ++i) {
            __builtin_amdgcn_sched_barrier(0);
            // The wave's DMA loads are spread evenly over the step's MFMA
            // groups.  Issued back to back in the first groups, every wave's
            // loads reach the vector memory queue at once; spread, mlp_up
            // ran 0.3-1.3% faster for the same bytes.
            constexpr int kEvery = T::kTM / T::kLoads;
            if (dma && i % kEvery == 0 && i / kEvery < T::kLoads)
                issue_one(dma_step, i / kEvery);
            if constexpr (WB == 4) {
                if (i == (T::kTM > 1 ? 1 : 0) && expand)
                    write_expanded(k + 2, pk);
            }
#pragma unroll
            for (int j = 0; j < T::kTN; ++j) {
                acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[i], fb[j], acc[i][j], 0, 0, 0);
                if (i == T::kTM - 1 && has_next)
                    fb[j] = read_b(k + 1, j);
            }
            if (has_next)
                fa[i] = read_a(k + 1, i);
        }
        __builtin_amdgcn_sched_barrier(0);
    };

#pragma unroll
    for (int s0 = 0; s0 < S - 1; ++s0)
        if (s0 < ksteps)
#pragma unroll
            for (int q = 0; q < T::kLoads; ++q)
                issue_one(s0, q);
    {
        // steps 0 .. AH must have landed (and the older scale loads)
        int younger = (ksteps < S - 1 ? ksteps : S - 1) - 1 - AH;
        younger = younger > 0 ? younger : 0;
        wait_vmcnt_le<(S - 2 - AH) * T::kLoads>(younger * my_loads);
    }
    __syncthreads();
    if constexpr (WB == 4) {
        write_expanded(0, read_packed(0));
        if (ksteps > 1)
            write_expanded(1, read_packed(1));
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < T::kTM; ++i)
        fa[i] = read_a(0, i);
#pragma unroll
    for (int j = 0; j < T::kTN; ++j)
        fb[j] = read_b(0, j);
    int k = 0;
    for (; k + S - 1 < ksteps; ++k)
        iteration(k, std::integral_constant<bool, true>{});
    for (; k < ksteps; ++k)
        iteration(k, std::integral_constant<bool, false>{});
    __syncthreads();

    // ---- epilogue.  The MFMA 16x16 result block leaves lane l with column
    // l%16 and rows 4*(l/16) + v.  Each wave stages one 16-row slice of its
    // accumulators in its own LDS region (the operand ring is free by now),
    // then reads it back four consecutive columns per lane: slot s of a slice
    // is (row s / kColQuads, column quad s % kColQuads), and lane l owns slots
    // l + 64 k.  Lanes covering one row then store whole row segments (256
    // contiguous bytes of bf16 for a 128-column wave tile), the pattern the
    // memory system absorbs at full rate; 32-byte row pieces per instruction
    // measured at well under half of it.  The staging region is private to
    // the wave and LDS operations of one wave complete in order, so no
    // workgroup barrier separates writing and reading it, only a wave-scope
    // fence that keeps the compiler's order (wave_lds_sync).
    constexpr int kStageStride = T::kWaveN + 4;                 // int32 per staged row
    constexpr int kColQuads = T::kWaveN / 4;
    constexpr int kSlots = 16 * kColQuads / 64;
    constexpr int kRowStep = 64 / kColQuads;
    static_assert(64 % kColQuads == 0 && kSlots >= 1, "");
    static_assert(T::kWaves * 16 * kStageStride * 4 <= T::kScaleOff, "staging fits in the ring");
    int32_t *stage = reinterpret_cast<int32_t *>(lds) + wave * 16 * kStageStride;
    const float *sx_lds = reinterpret_cast<const float *>(lds + T::kScaleOff);
    const float *sw_lds = sx_lds + BM;
    const float *b_lds = sw_lds + BN;
    const int kind = L.out_kind;
    void *Yv = L.Y;
    const int64_t ldy = L.ldy;
    const float alpha = L.alpha;
    // A divisor 2^k with 2^k and 2^-k both normal (exponent field 1 .. 253)
    // has the exact reciprocal 2^-k, and x * 2^-k and x / 2^k are then the
    // correct roundings of the same real number: such tiles multiply, one
    // operation instead of the division's ten.  (alpha > 0 by contract.)
    const uint32_t alpha_field = (__builtin_bit_cast(uint32_t, alpha) >> 23) & 0xFFu;
    const bool alpha_pow2 = (__builtin_bit_cast(uint32_t, alpha) & 0x7FFFFFu) == 0u && alpha_field >= 1u &&
                            alpha_field <= 253u;
    const float alpha_inv = __builtin_bit_cast(float, (254u - alpha_field) << 23);
    const int row_in = 4 * (lane >> 4), col_in = lane & 15;
    const int cq = lane % kColQuads, rr0 = lane / kColQuads;
    const int cl = wn * T::kWaveN + 4 * cq;                     // column within the tile
    const int64_t o = n0 + cl;
    const bool col_any = o < N;
    const bool full = (L.vec_store != 0) && (o + 4 <= N);
    // A missing weight scale multiplies by 1 and a missing bias adds -0: both
    // leave every binary32 value unchanged, zeros and their signs included,
    // so the operations need no per-element selects.
    const v4f sw = has_sw ? *reinterpret_cast<const v4f *>(sw_lds + cl) : v4f{1.0f, 1.0f, 1.0f, 1.0f};
    const v4f bo = has_bias ? *reinterpret_cast<const v4f *>(b_lds + cl) : v4f{-0.0f, -0.0f, -0.0f, -0.0f};
    // gated residual (after the reconstruction, before the output cast)
    const v4f gt = has_post ? *reinterpret_cast<const v4f *>(b_lds + BN + cl) : v4f{1.0f, 1.0f, 1.0f, 1.0f};
    const float post_scale = L.post_scale;
    const bool res_full = has_post && L.res_vec != 0 && (o + 4 <= N);
    // Addresses: one per-lane element offset of the lane's first row, plus a
    // uniform multiple of the row pitch per slot (scalar arithmetic), so that
    // no slot repeats 64-bit multiplies; rows are checked against the tile's
    // valid row count in 32 bits.
    const int rows_valid = (int)a_rows;
    const int lane_row0 = wm * T::kWaveM + rr0;                 // tile row of slot (0, 0)
    int64_t y_lane = (m0 + lane_row0) * ldy + o;                // element offset in Y
    int64_t r_lane = has_post ? (m0 + lane_row0) * L.ld_res + o : 0;
    // opaque, so that the compiler does not fold the per-slot offsets back
    // into per-slot 64-bit products
    asm volatile("" : "+v"(y_lane));
    asm volatile("" : "+v"(r_lane));

    // Output of four consecutive columns starting at element offset y_off
    // (KIND: kOutF32 or kOutBF16).
    auto store4 = [&](auto kind_tag, int64_t y_off, const float (&t)[4], bool vec, int64_t first_col) {
        if constexpr (decltype(kind_tag)::value == kOutF32) {
            float *y = static_cast<float *>(Yv) + y_off;
            if (vec) {
                __builtin_nontemporal_store(v4f{t[0], t[1], t[2], t[3]}, reinterpret_cast<v4f *>(y));
            } else {
                for (int e = 0; e < 4 && first_col + e < N; ++e)
                    y[e] = t[e];
            }
        } else {
            const unsigned w0 = __builtin_bit_cast(unsigned, __builtin_convertvector(v2f{t[0], t[1]}, v2bf));
            const unsigned w1 = __builtin_bit_cast(unsigned, __builtin_convertvector(v2f{t[2], t[3]}, v2bf));
            uint16_t *y = static_cast<uint16_t *>(Yv) + y_off;
            if (vec) {
                __builtin_nontemporal_store(v2u{w0, w1}, reinterpret_cast<v2u *>(y));
            } else {
                const unsigned ws[4] = {w0 & 0xFFFFu, w0 >> 16, w1 & 0xFFFFu, w1 >> 16};
                for (int e = 0; e < 4 && first_col + e < N; ++e)
                    y[e] = (uint16_t)ws[e];
            }
        }
    };

    if constexpr (GLU) {
        // SwiGLU: lane l owns output column quad l % kOutQuads of its wave
        // (gate columns at 4q.., up columns at kWaveN/2 + 4q.. of the staged
        // rows) and rows l / kOutQuads + kGluRowStep * s of each slice.
        //   g = fl(fl(fl(A_g) * s_x) * s_w_gate) [/ alpha]
        //   u = fl(fl(fl(A_u) * s_x) * s_w_up) [/ alpha]
        //   y = fl(silu(g) * u),  silu(g) = fl(g * fl(1 / fl(1 + exp(-g))))
        // with exp correctly rounded; one output cast.
        constexpr int kOutQuads = T::kWaveN / 8;
        constexpr int kGluSlots = 16 * kOutQuads / 64;
        constexpr int kGluRowStep = 64 / kOutQuads;
        static_assert(64 % kOutQuads == 0 && kGluSlots >= 1, "");
        const int cqo = lane % kOutQuads, rg0 = lane / kOutQuads;
        const int64_t oc = n0o + wn * (T::kWaveN / 2) + 4 * cqo;
        const bool oc_any = oc < N;
        const bool oc_full = (L.vec_store != 0) && (oc + 4 <= N);
        float swg[4] = {1.0f, 1.0f, 1.0f, 1.0f}, swu[4] = {1.0f, 1.0f, 1.0f, 1.0f};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (oc + e < N) {
                if (L.s_w)
                    swg[e] = L.s_w[oc + e];
                if (L.s_w_up)
                    swu[e] = L.s_w_up[oc + e];
            }
        }
        int64_t g_lane = (m0 + wm * T::kWaveM + rg0) * ldy + oc;
        asm volatile("" : "+v"(g_lane));
        auto glu_epilogue = [&](auto kind_tag, auto full_tag) {
            constexpr bool FULL = decltype(full_tag)::value;
#pragma unroll
            for (int i = 0; i < T::kTM; ++i) {
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int j = 0; j < T::kTN; ++j)
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        stage[(row_in + v) * kStageStride + j * 16 + col_in] = acc[i][j][v];
                wave_lds_sync();
#pragma unroll
                for (int sl = 0; sl < kGluSlots; ++sl) {
                    const int rr = rg0 + kGluRowStep * sl;
                    const v4i ag = *reinterpret_cast<const v4i *>(stage + rr * kStageStride + 4 * cqo);
                    const v4i au = *reinterpret_cast<const v4i *>(stage + rr * kStageStride + T::kWaveN / 2 + 4 * cqo);
                    const int rl = wm * T::kWaveM + i * 16 + rr;
                    if (!FULL && (rl >= rows_valid || !oc_any))
                        continue;
                    const float sxr = sx_lds[rl];
                    float t[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        float g = (float)ag[e];
                        g = g * sxr;
                        g = g * swg[e];
                        float u = (float)au[e];
                        u = u * sxr;
                        u = u * swu[e];
                        if constexpr (DIV) {
                            g = __fdiv_rn(g, alpha);
                            u = __fdiv_rn(u, alpha);
                        }
                        const float sg = __fdiv_rn(1.0f, 1.0f + convrot_expf::expf_cr(-g));
                        const float a = g * sg;
                        t[e] = a * u;
                    }
                    store4(kind_tag, g_lane + (int64_t)(i * 16 + kGluRowStep * sl) * ldy, t, FULL || oc_full, oc);
                }
            }
        };
        // tiles wholly inside Y with vector stores allowed skip every bounds check
        const bool tile_full = L.vec_store != 0 && n0o + BN / 2 <= N && m0 + BM <= M;
        if (kind == kOutF32) {
            if (tile_full)
                glu_epilogue(std::integral_constant<int, kOutF32>{}, std::true_type{});
            else
                glu_epilogue(std::integral_constant<int, kOutF32>{}, std::false_type{});
        } else {
            if (tile_full)
                glu_epilogue(std::integral_constant<int, kOutBF16>{}, std::true_type{});
            else
                glu_epilogue(std::integral_constant<int, kOutBF16>{}, std::false_type{});
        }
        return;
    }

    // The plain and gated-residual epilogue, with the output kind and, for
    // tiles wholly inside Y with vector stores allowed, the absence of bounds
    // checks fixed at compile time (no per-slot branches on either).
    auto epilogue = [&](auto kind_tag, auto full_tag, auto div_tag) {
        constexpr int KIND = decltype(kind_tag)::value;
        constexpr bool FULL = decltype(full_tag)::value;
        constexpr bool TDIV = decltype(div_tag)::value;
        // Gated residual on a tile wholly inside Y with vector residual rows:
        // each 16-row block's residual pieces are loaded one block ahead, so
        // that their latency runs under the previous block (4096 x 3072 x
        // 3072 bf16: 49.1 -> 46.4 us in an A/B run).  Kernels with the
        // unscale division keep the direct loads: there the extra registers
        // spilled.  In place (residual = Y) each element is still read before
        // the same lane writes it: block i + 1 is read while block i is
        // written.
        constexpr bool PF = POST && FULL && KIND != kOutI32 && !DIV;
        using ResV = typename std::conditional<KIND == kOutF32, v4f, v2u>::type;
        using ResE = typename std::conditional<KIND == kOutF32, float, uint16_t>::type;
        const bool pf_on = PF && has_post && L.res_vec != 0;
        ResV res_cur[kSlots], res_nxt[kSlots];
        auto res_load = [&](int i, ResV (&dst)[kSlots]) {
#pragma unroll
            for (int sl = 0; sl < kSlots; ++sl) {
                const int dr = i * 16 + kRowStep * sl;
                const ResE *rp = static_cast<const ResE *>(L.residual) + r_lane + (int64_t)dr * L.ld_res;
                dst[sl] = *reinterpret_cast<const ResV *>(rp);
            }
        };
        if constexpr (PF) {
            if (pf_on)
                res_load(0, res_cur);
        }
#pragma unroll
        for (int i = 0; i < T::kTM; ++i) {
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (PF) {
                if (pf_on && i + 1 < T::kTM)
                    res_load(i + 1, res_nxt);
            }
#pragma unroll
            for (int j = 0; j < T::kTN; ++j)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    stage[(row_in + v) * kStageStride + j * 16 + col_in] =
                        WB == 4 ? (acc[i][j][v] >> 4) : acc[i][j][v];   // 4-bit weights: 16 A
            wave_lds_sync();
#pragma unroll
            for (int sl = 0; sl < kSlots; ++sl) {
                const int rr = rr0 + kRowStep * sl;
                const v4i a = *reinterpret_cast<const v4i *>(stage + rr * kStageStride + 4 * cq);
                const int rl = wm * T::kWaveM + i * 16 + rr;        // row within the tile
                if (!FULL && (rl >= rows_valid || !col_any))
                    continue;
                const int dr = i * 16 + kRowStep * sl;              // rows below the lane's first
                const int64_t y_off = y_lane + (int64_t)dr * ldy;
                if constexpr (KIND == kOutI32) {
                    int32_t *y = static_cast<int32_t *>(Yv) + y_off;
                    if (FULL || full) {
                        *reinterpret_cast<v4i *>(y) = a;
                    } else {
                        for (int e = 0; e < 4 && o + e < N; ++e)
                            y[e] = a[e];
                    }
                    continue;
                } else {
                    const float sxr = sx_lds[rl];
                    float t[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        float x = (float)a[e];
                        x = x * sxr;
                        t[e] = x * sw[e];
                    }
                    if constexpr (TDIV) {
                        // uniform per tile: a power-of-two divisor multiplies
                        // by its exact reciprocal (same bits, see alpha_inv)
                        if (alpha_pow2) {
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                t[e] = t[e] * alpha_inv;
                        } else {
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                t[e] = __fdiv_rn(t[e], alpha);
                        }
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        t[e] = t[e] + bo[e];
                    if constexpr (POST) {
                        if (has_post) {
                            // fl(fl(fl(y * scale) * gate) + residual), the residual in
                            // the output dtype (bf16 widened exactly)
                            float rv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
                            if (PF && pf_on) {
                                if constexpr (KIND == kOutF32) {
                                    const v4f q = res_cur[sl];
                                    rv[0] = q.x; rv[1] = q.y; rv[2] = q.z; rv[3] = q.w;
                                } else {
                                    const v2u q = res_cur[sl];
                                    rv[0] = __builtin_bit_cast(float, (q.x & 0xFFFFu) << 16);
                                    rv[1] = __builtin_bit_cast(float, q.x & 0xFFFF0000u);
                                    rv[2] = __builtin_bit_cast(float, (q.y & 0xFFFFu) << 16);
                                    rv[3] = __builtin_bit_cast(float, q.y & 0xFFFF0000u);
                                }
                            } else if constexpr (KIND == kOutF32) {
                                const float *rp = static_cast<const float *>(L.residual) + r_lane + (int64_t)dr * L.ld_res;
                                if (res_full) {
                                    const v4f q = *reinterpret_cast<const v4f *>(rp);
                                    rv[0] = q.x; rv[1] = q.y; rv[2] = q.z; rv[3] = q.w;
                                } else {
                                    for (int e = 0; e < 4 && o + e < N; ++e)
                                        rv[e] = rp[e];
                                }
                            } else {
                                const uint16_t *rp = static_cast<const uint16_t *>(L.residual) + r_lane + (int64_t)dr * L.ld_res;
                                unsigned h[4] = {0u, 0u, 0u, 0u};
                                if (res_full) {
                                    const v2u q = *reinterpret_cast<const v2u *>(rp);
                                    h[0] = q.x & 0xFFFFu; h[1] = q.x >> 16; h[2] = q.y & 0xFFFFu; h[3] = q.y >> 16;
                                } else {
                                    for (int e = 0; e < 4 && o + e < N; ++e)
                                        h[e] = rp[e];
                                }
#pragma unroll
                                for (int e = 0; e < 4; ++e)
                                    rv[e] = __builtin_bit_cast(float, h[e] << 16);
                            }
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                float x = t[e];
                                if (post_scale != 1.0f)
                                    x = x * post_scale;
                                x = x * gt[e];
                                t[e] = x + rv[e];
                            }
                        }
                    }
                    if constexpr (KIND == kOutF32) {
                        float *y = static_cast<float *>(Yv) + y_off;
                        if (FULL || full) {
                            __builtin_nontemporal_store(v4f{t[0], t[1], t[2], t[3]}, reinterpret_cast<v4f *>(y));
                        } else {
                            for (int e = 0; e < 4 && o + e < N; ++e)
                                y[e] = t[e];
                        }
                    } else {
                        // Round to nearest even (the hardware conversion, finite
                        // inputs).  Both halves are taken from the packed words with
                        // integer operations: extracting the high element of a bf16
                        // vector is miscompiled by this toolchain.
                        const unsigned w0 = __builtin_bit_cast(unsigned, __builtin_convertvector(v2f{t[0], t[1]}, v2bf));
                        const unsigned w1 = __builtin_bit_cast(unsigned, __builtin_convertvector(v2f{t[2], t[3]}, v2bf));
                        uint16_t *y = static_cast<uint16_t *>(Yv) + y_off;
                        if (FULL || full) {
                            __builtin_nontemporal_store(v2u{w0, w1}, reinterpret_cast<v2u *>(y));
                        } else {
                            const unsigned ws[4] = {w0 & 0xFFFFu, w0 >> 16, w1 & 0xFFFFu, w1 >> 16};
                            for (int e = 0; e < 4 && o + e < N; ++e)
                                y[e] = (uint16_t)ws[e];
                        }
                    }
                }
            }
            if constexpr (PF) {
                if (i + 1 < T::kTM) {
#pragma unroll
                    for (int sl = 0; sl < kSlots; ++sl)
                        res_cur[sl] = res_nxt[sl];
                }
            }
        }
    };
    // A launch compiled with the division may also hold linears whose
    // divisor is 1 (a grouped launch over several input scales): their tiles
    // skip it, which gives the same bits (x / 1 is exact) without its cost.
    auto run = [&](auto kind_tag, auto full_tag) {
        if constexpr (DIV) {
            if (alpha != 1.0f) {
                epilogue(kind_tag, full_tag, std::true_type{});
                return;
            }
        }
        epilogue(kind_tag, full_tag, std::false_type{});
    };
    const bool tile_full = L.vec_store != 0 && n0 + BN <= N && m0 + BM <= M;
    if (kind == kOutBF16) {
        if (tile_full)
            run(std::integral_constant<int, kOutBF16>{}, std::true_type{});
        else
            run(std::integral_constant<int, kOutBF16>{}, std::false_type{});
    } else if (kind == kOutF32) {
        if (tile_full)
            run(std::integral_constant<int, kOutF32>{}, std::true_type{});
        else
            run(std::integral_constant<int, kOutF32>{}, std::false_type{});
    } else {
        epilogue(std::integral_constant<int, kOutI32>{}, std::false_type{}, std::false_type{});
    }
}

// PLAIN_ONLY: the configuration serves only the plain epilogue (its other
// kernels are not instantiated).
template <int BM, int BN, int WM, int WN, int STAGES, int WB, bool PLAIN_ONLY = false>
hipError_t launch_tiled(GemmProblem p, hipStream_t stream)
{
    using T = Tile<BM, BN, WM, WN, STAGES, WB>;
    const int tiles_m = (int)((p.M + BM - 1) / BM);
    int total = 0;
    for (int d = 0; d < p.n_lin; ++d) {
        if (!p.lin[d].Qx) {
            p.lin[d].Qx = p.Qx;
            p.lin[d].s_x = p.s_x;
        }
        // a SwiGLU pair spends two tile columns per output column
        const int64_t cols = p.lin[d].glu ? 2 * p.lin[d].N : p.lin[d].N;
        p.lin[d].tiles_n = (int)((cols + BN - 1) / BN);
        p.lin[d].tile_begin = total;
        total += tiles_m * p.lin[d].tiles_n;
    }
    if (total == 0)
        return hipSuccess;
    // the unscale division and the epilogue extras are compiled in only when
    // some linear needs them (a SwiGLU problem holds SwiGLU pairs only)
    bool div = false, post = false, glu = false;
    for (int d = 0; d < p.n_lin; ++d) {
        div = div || p.lin[d].alpha != 1.0f;
        post = post || p.lin[d].post != 0;
        glu = glu || p.lin[d].glu != 0;
    }
#define CONVROT_GEMM(D, E)                                                                       \
    hipLaunchKernelGGL((gemm_i8_kernel<BM, BN, WM, WN, STAGES, D, WB, E>), dim3(total),         \
                       dim3(T::kThreads), 0, stream, p, tiles_m, total)
    if constexpr (PLAIN_ONLY) {
        if (glu || post)
            return hipErrorInvalidValue;        // not reached: the caller routes these elsewhere
    } else {
        if constexpr (WB == 8) {
            if (glu) {
                if (div) CONVROT_GEMM(true, kEpiGlu); else CONVROT_GEMM(false, kEpiGlu);
                return hipGetLastError();
            }
        }
        if (post) {
            if (div) CONVROT_GEMM(true, kEpiPost); else CONVROT_GEMM(false, kEpiPost);
            return hipGetLastError();
        }
    }
    if (div) CONVROT_GEMM(true, kEpiPlain); else CONVROT_GEMM(false, kEpiPlain);
#undef CONVROT_GEMM
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(GemmProblem p, hipStream_t stream)
{
    // Large grids use 256 x 256 tiles (16 waves of 64 x 64, four per SIMD, so
    // that one wave's LDS and barrier waits are covered by the MFMAs of the
    // others; or 8 waves of 128 x 64 for the plain epilogue, below); grids of
    // fewer than 160 such tiles (under 62.5% of the
    // 256 CUs for one round) use 128 x 128 tiles with 8 waves (2 x 4; 64 KB of
    // LDS, so two workgroups fit on a CU).  Measured on gfx950 at K = 3072: a
    // round of 256 x 256 tiles costs about the same for any count up to 256
    // (192 tiles: 50 us against 59 us in 128 x 128 tiles; 96 tiles: 44 us
    // against 34 us).  Both use a 4-stage ring (5 with 4-bit weights, which
    // expand a step ahead): deeper rings (6 or 8 stages)
    // were slower for every shape tried once they cost the second resident
    // workgroup, and no faster otherwise.
    int64_t big = 0;
    for (int d = 0; d < p.n_lin; ++d)
        big += ((p.M + 255) / 256) * (((p.lin[d].glu ? 2 : 1) * p.lin[d].N + 255) / 256);
    constexpr int64_t kBigTiles = 160;
    if (p.w_bits == 4) {
        if (big >= kBigTiles)
            return launch_tiled<256, 256, 4, 4, 5, 4>(p, stream);
        return launch_tiled<128, 128, 2, 4, 5, 4>(p, stream);
    }
    if (big >= kBigTiles) {
        // The plain epilogue takes 8 waves of 128 x 64 (2 x 4): a quarter
        // fewer LDS fragment reads per MFMA, 1-2% faster on the plain
        // workloads.  The gated-residual and SwiGLU epilogues keep 16 waves
        // of 64 x 64: with 8 waves their heavier epilogues ran 10-20% slower.
        bool heavy = false;
        for (int d = 0; d < p.n_lin; ++d)
            heavy = heavy || p.lin[d].post != 0 || p.lin[d].glu != 0;
        if (heavy)
            return launch_tiled<256, 256, 4, 4, 4, 8>(p, stream);
        return launch_tiled<256, 256, 2, 4, 4, 8, true>(p, stream);
    }
    return launch_tiled<128, 128, 2, 4, 4, 8>(p, stream);
}

}  // namespace convrot_detail
