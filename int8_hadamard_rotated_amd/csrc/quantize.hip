// Rotate + row-max + quantize + pack, one pass over X (gfx950, wave64).
//
// Computes, per activation row (page "INT8 Convrot Safetensors", section
// "How INT8 convrot works", subsection "Runtime activation quantization"):
//   x  = widen(X[r, :])
//   x  = (x + x * scale) + shift           (optional Modulate producer: page
//                                           "ggml operator extensions", section
//                                           "sd.cpp integration"; per-channel
//                                           vectors, shift optional)
//   x  = fl(act(x) * u)                    (optional gated activation, SiLU or
//                                           Sigmoid of x times a second input
//                                           u, same page and section)
//   x  = fl(x * r) [* w]                   (optional RMSNorm -> Mul(weight)
//                                           ahead of Modulate, same page and
//                                           section; r per row, see below)
//   x  = fl(fl(x - mean) * r) [* w]        (or Norm -> Mul(weight), same page
//                                           and section; mean and r per row,
//                                           see below)
//   x  = x * alpha                         (multiply only when alpha != 1)
//   y  = x R_G per contiguous G-group       (R_G = H4^(x)n, G = 4^n)
//   m  = max |y| over the whole row
//   s  = fl(m / 127)  and  q = rne(fl(y * fl(127 / m)))  (m = 0: s = 0, q = 0)
// and writes the packed tensor: int8 [M_pad][K] then float [M_pad]
// (page "ggml operator extensions", section "sd.cpp integration": rows padded
// to a multiple of four, followed by the F32 row scales).
//
// Every binary32 operation is the oracle's, in the oracle's order: one H4 per
// base-4 digit of the in-group index, digit 0 first, each as
// s = (x0 + x1) + (x2 + x3), h = s * 0.5, y_j = h - x_{3-j}.
//
// Data layout.  A quad (4 adjacent lanes, j = j0 + 2*j1) owns a span of
// 32*NC consecutive elements of one row; each lane holds NC chunks of 8
// consecutive elements (p = 0..7).  Chunk c of lane j starts at span offset
//   8*j0 + 16*(c & 1) + 32*j1 + 64*(c >> 1)
// so the element index is e = p + 8*j0 + 16*c0 + 32*j1 + 64*c1, and its
// base-4 digits sit at
//   digit 0 = p & 3                      in-register
//   digit 1 = (p >> 2) + 2*j0            low bit in-register, high bit lane^1
//   digit 2 = c0 + 2*j1                  low bit in-register, high bit lane^2
//   digit 3 = c1 & 3                     in-register (G = 256, NC = 8)
// A digit split as (in-register low bit, lane high bit) keeps the oracle's
// pairing: each lane forms x_{2H} + x_{2H+1} locally, adds its partner's pair
// sum through one DPP quad_perm, and IEEE addition being commutative, both
// lanes hold the bits of (x0 + x1) + (x2 + x3).  Output y_{2H+l} = h - x_{3-2H-l}
// needs the partner's element with the other low bit: y[l] = h - partner[1-l].
// No lane-dependent selects are needed, and every DPP exchange stays inside a
// quad, which is always fully active.
//
// One workgroup holds R whole rows (R * quads_per_row quads); the row maximum
// is reduced in-lane, across the quad (DPP), then across the row's quads with
// an LDS unsigned max (non-negative binary32 values order like their bits).
//
// Codes: t = fl(y * inv) lies in [-127 - 2^-17, 127 + 2^-17] because
// |y| <= m and inv = fl(127/m), so round-half-even(t) is already within
// [-127, 127] and the clamp of the formula never changes a value.  The
// rounding uses fl(t + 1.5 * 2^23): for |t| < 2^22 that sum is exactly
// 1.5 * 2^23 + rne(t) (ulp 1, and 1.5 * 2^23 is even, so ties go to the even
// code), whose low byte is the two's-complement int8 code.
#pragma clang fp contract(off)

#include <type_traits>

#include "expf_cr.h"
#include "kernels.h"

namespace convrot_detail {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));

constexpr int kQuadPermXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kQuadPermXor2 = 0x4E;  // quad_perm [2,3,0,1]

// The row normalization ahead of the quantizer: none, RMSNorm (root mean
// square), or Norm (mean and variance).
enum NormKind : int { kNormNone = 0, kNormRms = 1, kNormMean = 2 };

template <int CTRL>
__device__ __forceinline__ float quad_swap(float x)
{
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

template <int CTRL>
__device__ __forceinline__ unsigned quad_swap_u(unsigned x)
{
    return (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, true);
}

// H4 on four in-register values.
__device__ __forceinline__ void h4_local(float &x0, float &x1, float &x2, float &x3)
{
    const float s = (x0 + x1) + (x2 + x3);
    const float h = s * 0.5f;
    const float y0 = h - x3, y1 = h - x2, y2 = h - x1, y3 = h - x0;
    x0 = y0;
    x1 = y1;
    x2 = y2;
    x3 = y3;
}

// H4 on a digit whose low bit is in-register (lo0: 0, lo1: 1) and whose high
// bit is the lane bit that CTRL flips.
template <int CTRL>
__device__ __forceinline__ void h4_split(float &lo0, float &lo1)
{
    const float pair = lo0 + lo1;
    const float s = pair + quad_swap<CTRL>(pair);
    const float h = s * 0.5f;
    const float p0 = quad_swap<CTRL>(lo0);
    const float p1 = quad_swap<CTRL>(lo1);
    lo0 = h - p1;
    lo1 = h - p0;
}

__device__ __forceinline__ void load8(const float *src, float (&v)[8])
{
    const v4f a = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(src));
    const v4f b = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(src) + 1);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// bf16 -> binary32 is exact: the bf16 bits are the upper half.
__device__ __forceinline__ void widen8(const v4u &u, float (&v)[8])
{
    const unsigned w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __builtin_bit_cast(float, w[i] << 16);
        v[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xFFFF0000u);
    }
}

__device__ __forceinline__ void load8(const uint16_t *src, float (&v)[8])
{
    widen8(__builtin_nontemporal_load(reinterpret_cast<const v4u *>(src)), v);
}

// Four independent H4s of split digits (each as h4_split) in lockstep: every
// DPP read of a freshly written pair sum then has three other instructions
// before it, the wait states the exchange needs, instead of no-ops.  Same
// operations, so the same bits.
template <int CTRL>
__device__ __forceinline__ void h4_split4(float &a0, float &a1, float &b0, float &b1, float &c0, float &c1,
                                          float &d0, float &d1)
{
    const float pa = a0 + a1, pb = b0 + b1, pc = c0 + c1, pd = d0 + d1;
    const float sa = pa + quad_swap<CTRL>(pa), sb = pb + quad_swap<CTRL>(pb);
    const float sc = pc + quad_swap<CTRL>(pc), sd = pd + quad_swap<CTRL>(pd);
    const float ha = sa * 0.5f, hb = sb * 0.5f, hc = sc * 0.5f, hd = sd * 0.5f;
    const float a0n = ha - quad_swap<CTRL>(a1), b0n = hb - quad_swap<CTRL>(b1);
    const float c0n = hc - quad_swap<CTRL>(c1), d0n = hd - quad_swap<CTRL>(d1);
    a1 = ha - quad_swap<CTRL>(a0);
    b1 = hb - quad_swap<CTRL>(b0);
    c1 = hc - quad_swap<CTRL>(c0);
    d1 = hd - quad_swap<CTRL>(d0);
    a0 = a0n;
    b0 = b0n;
    c0 = c0n;
    d0 = d0n;
}

// Low bytes of four words -> one word (byte i from w[i]).
__device__ __forceinline__ unsigned pack_low_bytes(unsigned w0, unsigned w1, unsigned w2, unsigned w3)
{
    const unsigned lo = __builtin_amdgcn_perm(w1, w0, 0x0c0c0400u);
    const unsigned hi = __builtin_amdgcn_perm(w3, w2, 0x04000c0cu);
    return lo | hi;
}

// Span offset of chunk c of lane (j0, j1) in its quad (see the layout above).
__device__ __forceinline__ int chunk_offset(int j0, int j1, int c)
{
    return 8 * j0 + 16 * (c & 1) + 32 * j1 + 64 * (c >> 1);
}

// The rotation of one quad span held in the quad layout: one H4 per base-4
// digit of the in-group index, digit 0 first.  LS: the split digits' H4s run
// four in lockstep (h4_split4); measured faster for passes of one round of
// waves, slower where more registers cost resident waves (see the launcher).
template <int G, int NC, bool LS = false>
__device__ __forceinline__ void rotate_span(float (&v)[NC][8])
{
    // G = 1 (4^0): no digit, the identity
    // digit 0 (stride 1)
    if constexpr (G >= 4) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            h4_local(v[c][0], v[c][1], v[c][2], v[c][3]);
            h4_local(v[c][4], v[c][5], v[c][6], v[c][7]);
        }
    }
    // digit 1 (stride 4): low bit p>>2, high bit lane bit 0
    if constexpr (G >= 16) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            if constexpr (LS) {
                h4_split4<kQuadPermXor1>(v[c][0], v[c][4], v[c][1], v[c][5], v[c][2], v[c][6], v[c][3],
                                         v[c][7]);
            } else {
#pragma unroll
                for (int p = 0; p < 4; ++p)
                    h4_split<kQuadPermXor1>(v[c][p], v[c][p + 4]);
            }
        }
    }
    // digit 2 (stride 16): low bit c&1, high bit lane bit 1
    if constexpr (G >= 64) {
#pragma unroll
        for (int c = 0; c < NC; c += 2) {
            if constexpr (LS) {
#pragma unroll
                for (int p = 0; p < 8; p += 4)
                    h4_split4<kQuadPermXor2>(v[c][p], v[c + 1][p], v[c][p + 1], v[c + 1][p + 1], v[c][p + 2],
                                             v[c + 1][p + 2], v[c][p + 3], v[c + 1][p + 3]);
            } else {
#pragma unroll
                for (int p = 0; p < 8; ++p)
                    h4_split<kQuadPermXor2>(v[c][p], v[c + 1][p]);
            }
        }
    }
    // digit 3 (stride 64): chunk bits 1..2
    if constexpr (G >= 256) {
#pragma unroll
        for (int c0 = 0; c0 < 2; ++c0)
#pragma unroll
            for (int p = 0; p < 8; ++p)
                h4_local(v[c0][p], v[c0 + 2][p], v[c0 + 4][p], v[c0 + 6][p]);
    }
}

// max |y| over the quad's span, the same in all four lanes.
template <int NC>
__device__ __forceinline__ float quad_abs_max(const float (&v)[NC][8])
{
    float m = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int p = 0; p < 8; ++p)
            m = fmaxf(m, fabsf(v[c][p]));
    m = fmaxf(m, quad_swap<kQuadPermXor1>(m));
    return fmaxf(m, quad_swap<kQuadPermXor2>(m));
}

// Correctly rounded binary32 square root of a finite x >= 0.  Start from the
// hardware's approximation and step to the neighbour while sqrt(x) lies
// outside the candidate's rounding interval; the interval ends have at most
// 25 significant bits, so their squares compare with x exactly in binary64
// (a tie at an end goes to the even candidate).
__device__ __forceinline__ float sqrt_rn(float x)
{
    if (!(x > 0.0f) || x == __builtin_huge_valf())
        return x;
    float s = __builtin_sqrtf(x);
    const double xd = x;
    for (int it = 0; it < 4; ++it) {
        const unsigned b = __builtin_bit_cast(unsigned, s);
        const float below = __builtin_bit_cast(float, b - 1u);
        const float above = __builtin_bit_cast(float, b + 1u);
        const double lo = 0.5 * ((double)s + (double)below);
        const double hi = 0.5 * ((double)s + (double)above);
        const bool odd = (b & 1u) != 0;
        if (lo * lo > xd || (lo * lo == xd && odd))
            s = below;
        else if (hi * hi < xd || (hi * hi == xd && odd))
            s = above;
        else
            break;
    }
    return s;
}

// The normalizations' sums for the quad's 64-feature blocks (block b = chunks
// 2b and 2b+1): the pairwise tree of the 64 values (SQ: of their squares),
// adjacent pairs first.  Its levels are the element index bits: 0..2 in the
// chunk, 3 = lane bit 0, 4 = chunk bit 0, 5 = lane bit 1; IEEE addition being
// commutative, both lanes of a DPP pair hold the same bits.  Every lane of the
// quad ends with every block sum.
template <int NC, bool SQ>
__device__ __forceinline__ void block_sums(const float (&v)[NC][8], float (&bs)[NC / 2])
{
#pragma unroll
    for (int b = 0; b < NC / 2; ++b) {
        float s16[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const float(&x)[8] = v[2 * b + h];
            float q[8];
#pragma unroll
            for (int p = 0; p < 8; ++p)
                q[p] = SQ ? x[p] * x[p] : x[p];
            const float a0 = q[0] + q[1], a1 = q[2] + q[3], a2 = q[4] + q[5], a3 = q[6] + q[7];
            const float s8 = (a0 + a1) + (a2 + a3);
            s16[h] = s8 + quad_swap<kQuadPermXor1>(s8);
        }
        const float s32 = s16[0] + s16[1];
        bs[b] = s32 + quad_swap<kQuadPermXor2>(s32);
    }
}

// x = fl(x * w[col + p]) on one chunk (RMSNorm's weight), read through the
// caches like the Modulate vectors.
__device__ __forceinline__ void weight8(float (&v)[8], const float *__restrict__ w, int64_t col)
{
    const v4f w0 = *reinterpret_cast<const v4f *>(w + col);
    const v4f w1 = *reinterpret_cast<const v4f *>(w + col + 4);
    const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
    for (int p = 0; p < 8; ++p)
        v[p] = v[p] * wv[p];
}

// LDS index of column col of a per-channel vector staged in LDS (the
// Modulate scale and shift, the RMSNorm weight): the 16-byte slots of each
// 256-column block are XOR-ed with 4 (block & 1) + 16 ((block >> 1) & 1)
// floats, so that the quads of a wave, which read the same slot of four
// consecutive blocks, land on distinct banks.  Slots stay whole and inside
// their block.
__device__ __forceinline__ int param_index(int col)
{
    const int b = col >> 8;
    return col ^ (4 * (b & 1) + 16 * ((b >> 1) & 1));
}

__device__ __forceinline__ void lds_params8(const float *vec, int col, float (&out)[8])
{
    const v4f a = *reinterpret_cast<const v4f *>(vec + param_index(col));
    const v4f b = *reinterpret_cast<const v4f *>(vec + param_index(col + 4));
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}

// LDS index of element e of the gated activation's staged rows: 4 floats of
// padding after every 256 (an 8-element piece never straddles a boundary).
__device__ __forceinline__ int act_index(int e) { return e + (e >> 8) * 4; }

// Dynamic LDS bytes of that staging for `elems` elements.
inline size_t act_stage_bytes(int64_t elems) { return (size_t)(elems + (elems >> 8) * 4 + 8) * 4; }

// The gated activation on one value: sigmoid(g) = fl(1 / fl(1 + exp(-g)))
// with exp correctly rounded; SiLU is fl(g * sigmoid(g)).  Division by IEEE
// rule (the toolchain's default single-precision division is correctly
// rounded).
template <int ACT>
__device__ __forceinline__ float gated_act(float g)
{
    const float e = convrot_expf::expf_cr(-g);
    const float d = 1.0f + e;
    const float sg = __fdiv_rn(1.0f, d);
    if constexpr (ACT == kActSilu)
        return g * sg;
    return sg;
}

// Codes of one chunk: rne(fl(y * inv)) in two's complement, 8 bytes.
__device__ __forceinline__ v2u encode8(const float (&v)[8], float inv)
{
    unsigned w[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const float t = v[p] * inv;
        w[p] = __builtin_bit_cast(unsigned, t + 12582912.0f);
    }
    v2u out;
    out.x = pack_low_bytes(w[0], w[1], w[2], w[3]);
    out.y = pack_low_bytes(w[4], w[5], w[6], w[7]);
    return out;
}

// Codes of chunks c and c + 1 of the two lanes of a pair (j0 = 0, 1): they
// cover 32 consecutive bytes, [0, 8) and [16, 24) in lane 0, [8, 16) and
// [24, 32) in lane 1.  One exchange across the pair returns [0, 16) to lane 0
// and [16, 32) to lane 1, so that every lane stores 16 bytes at
// chunk_offset(0, j1, c) + 16 j0 and a quad 64 contiguous ones.  Both lanes of
// the pair must be active.
__device__ __forceinline__ v4u encode_pair16(const float (&a)[8], const float (&b)[8], float inv, int j0)
{
    const v2u e0 = encode8(a, inv), e1 = encode8(b, inv);
    const v2u send = j0 ? e0 : e1;
    const v2u recv{quad_swap_u<kQuadPermXor1>(send.x), quad_swap_u<kQuadPermXor1>(send.y)};
    const v2u lo = j0 ? recv : e0, hi = j0 ? e1 : recv;
    return v4u{lo.x, lo.y, hi.x, hi.y};
}

// Workgroup quad index -> (row within the workgroup, quad within the row).
// Without a producer quads are row-major.  With the Modulate producer they
// are column-major, so that the quads of one wave that read the same columns
// (of different rows) load the same per-channel parameters in one
// instruction, which the memory pipeline serves once.
template <int MOD>
__device__ __forceinline__ void quad_place(int quad, int quads_per_row, int rows_per_wg, int &row,
                                           int &q_in_row)
{
    if constexpr (MOD != 0) {
        row = quad % rows_per_wg;
        q_in_row = quad / rows_per_wg;
    } else {
        row = quad / quads_per_row;
        q_in_row = quad - row * quads_per_row;
    }
}

// The Modulate producer on one chunk of 8 elements whose first column is
// `col`: x = (x + x * scale) + shift, each operation rounded on its own (the
// file is compiled without contraction).  MOD: 1 scale only, 2 with shift.
// The vectors are read through the caches: every row reads the same ones.
template <int MOD>
__device__ __forceinline__ void modulate8(float (&v)[8], const float *__restrict__ scale,
                                          const float *__restrict__ shift, int64_t col)
{
    if constexpr (MOD != 0) {
        const v4f s0 = *reinterpret_cast<const v4f *>(scale + col);
        const v4f s1 = *reinterpret_cast<const v4f *>(scale + col + 4);
        const float sc[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
        for (int p = 0; p < 8; ++p)
            v[p] = v[p] + v[p] * sc[p];
        if constexpr (MOD == 2) {
            const v4f h0 = *reinterpret_cast<const v4f *>(shift + col);
            const v4f h1 = *reinterpret_cast<const v4f *>(shift + col + 4);
            const float sh[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
#pragma unroll
            for (int p = 0; p < 8; ++p)
                v[p] = v[p] + sh[p];
        }
    }
}

// The same two producers with their vectors staged in LDS (same arithmetic).
template <int MOD>
__device__ __forceinline__ void modulate8_lds(float (&v)[8], const float *scale, const float *shift, int col)
{
    if constexpr (MOD != 0) {
        float sc[8];
        lds_params8(scale, col, sc);
#pragma unroll
        for (int p = 0; p < 8; ++p)
            v[p] = v[p] + v[p] * sc[p];
        if constexpr (MOD == 2) {
            float sh[8];
            lds_params8(shift, col, sh);
#pragma unroll
            for (int p = 0; p < 8; ++p)
                v[p] = v[p] + sh[p];
        }
    }
}

__device__ __forceinline__ void weight8_lds(float (&v)[8], const float *w, int col)
{
    float wv[8];
    lds_params8(w, col, wv);
#pragma unroll
    for (int p = 0; p < 8; ++p)
        v[p] = v[p] * wv[p];
}

// Vectors staged (PS = true) when a Modulate is present and the producer's
// per-channel vectors (with the RMSNorm weight, if any) fit in
// kParamLdsBytes: the workgroup copies them to LDS once, in 16-byte pieces,
// instead of every lane loading 8 values per vector and chunk from the caches
// (the same columns for each of the wave's rows).  Measured on the 4096 x 3072
// bf16 pass: 10.8% faster with scale and shift, 4.7% with scale only, 5.4%
// for RMSNorm with weight, scale and shift; RMSNorm with its weight alone ran
// 5% slower staged, so it keeps the cached loads.
constexpr int kParamLdsBytes = 48 * 1024;

//
// RMSNorm (NRM = kNormRms) takes two more workgroup phases before the
// Modulate: each quad stores its 64-feature block sums of squares in LDS; one
// lane per row adds the row's K/64 block sums left to right and forms
// r = fl(1 / fl(sqrt(fl(fl(S / K) + eps)))) with correctly rounded operations;
// every lane then scales its values by its row's r (and the weight).  Norm
// (NRM = kNormMean) first takes the same two phases over the values
// themselves, mean = fl(S1 / K), and centres every value on it, so that the
// squares are the deviations' and S / K is the variance.
//
// With a row normalization or a gated activation the workgroup has at most 512 threads
// (two waves per SIMD), so that the row data, the block sums or the exp's
// binary64 temporaries fit in registers.
//
// A gated activation (ACT != 0) first computes fl(act(x) * u) over the
// workgroup's rows in a plain layout: thread t takes the 8-element pieces
// t, t + T, t + 2T, ... (T threads) of the rows laid end to end, with
// coalesced 16- or 32-byte loads of x and up, in a loop that is not unrolled,
// so that only one piece's exps are in flight per thread and the kernel
// keeps few registers.  The binary32 results go to LDS (act_stage; 4 floats
// of padding after every 256, so that the quads of a wave, whose spans are
// 256 elements apart, read distinct banks), and the quad layout then reads
// its values from there.  Same arithmetic per element as the other producers'
// direct path; it only changes where the values wait.
// RMSNorm with Modulate's scale and shift staged in LDS, at alpha = 1: capped
// for three waves per SIMD (168 registers), so that a pass of three waves per
// SIMD runs in one round (4096 x 3072 bf16: 20.35 -> 19.32 us, A/B on MI355X).
// The other RMSNorm kernels keep two: the cap spills registers there.
template <bool SCALED, int MOD, bool RMS, bool PS>
constexpr int kQuantizeWaves = (RMS && PS && MOD == 2 && !SCALED) ? 3 : 1;

template <typename XT, int G, int NC, bool SCALED, int MOD, int NRM, int ACT, bool PS, bool LS>
__global__ __launch_bounds__((NRM != kNormNone || ACT != 0) ? 512 : 1024,
                             (kQuantizeWaves<SCALED, MOD, NRM != kNormNone, PS>)) void quantize_rows_kernel(
    const XT *__restrict__ X, int64_t M, int64_t M_pad, int64_t K, int64_t ldx, float alpha,
    const float *__restrict__ mod_scale, const float *__restrict__ mod_shift,
    const float *__restrict__ norm_weight, float eps, const XT *__restrict__ up, int64_t ld_up,
    int8_t *__restrict__ Q, float *__restrict__ S, int quads_per_row, int rows_per_wg,
    int wave_store)
{
    static_assert(NC == 2 || NC == 4 || NC == 8, "chunks per lane");
    static_assert(G == 1 || G == 4 || G == 16 || G == 64 || (G == 256 && NC == 8), "group size vs span");
    constexpr bool RMS = NRM != kNormNone;               // a row normalization (either kind)
    static_assert(NRM != kNormMean || MOD == 0, "Norm -> Mul has no Modulate");
    constexpr int kBlocks = NC / 2;                      // 64-feature blocks per quad span
    __shared__ unsigned row_max[256];
    __shared__ float norm_part[RMS ? 256 * kBlocks : 1];
    __shared__ float norm_r[RMS ? 256 : 1];
    extern __shared__ __attribute__((aligned(16))) float act_stage[];

    const int tid = threadIdx.x;
    const int quad = tid >> 2;
    const int j0 = tid & 1, j1 = (tid >> 1) & 1;
    int row_local, q_in_row;
    quad_place<(MOD != 0 || RMS) ? 1 : 0>(quad, quads_per_row, rows_per_wg, row_local, q_in_row);
    static_assert(ACT == 0 || (MOD == 0 && !RMS), "one producer at a time");
    const int64_t row = (int64_t)blockIdx.x * rows_per_wg + row_local;
    const int64_t span0 = (int64_t)q_in_row * (32 * NC);
    // With a gated activation the workgroup may have more threads than the
    // quad layout uses (4 per quad): the extra ones only share the
    // activation pass, then wait at the barriers.
    const bool worker = tid < 4 * quads_per_row * rows_per_wg;
    // A quad never straddles rows, so this branch is uniform per quad and the
    // DPP exchanges below only read lanes that take the same path.
    const bool live = worker && row < M;

    static_assert(!PS || (ACT == 0 && MOD != 0), "staged vectors belong to a Modulate producer");
    float v[NC][8];
    if constexpr (PS) {
        // row data first, so that its loads are in flight during the staging
        if (live) {
            const XT *xr = X + row * ldx + span0;
#pragma unroll
            for (int c = 0; c < NC; ++c)
                load8(xr + 8 * j0 + 16 * (c & 1) + 32 * j1 + 64 * (c >> 1), v[c]);
        }
    }
    // staged vectors, K floats each, in this order: scale, shift, RMSNorm weight
    float *const p_scale = act_stage;
    float *const p_shift = act_stage + (MOD != 0 ? K : 0);
    float *const p_weight = act_stage + ((MOD != 0 ? K : 0) + (MOD == 2 ? K : 0));
    if constexpr (PS) {
        const int n = (int)K;
#pragma unroll 1
        for (int e = 4 * tid; e < n; e += 4 * (int)blockDim.x) {
            const int d = param_index(e);
            if constexpr (MOD != 0)
                *reinterpret_cast<v4f *>(p_scale + d) = *reinterpret_cast<const v4f *>(mod_scale + e);
            if constexpr (MOD == 2)
                *reinterpret_cast<v4f *>(p_shift + d) = *reinterpret_cast<const v4f *>(mod_shift + e);
            if constexpr (RMS) {
                if (norm_weight)
                    *reinterpret_cast<v4f *>(p_weight + d) = *reinterpret_cast<const v4f *>(norm_weight + e);
            }
        }
    }
    if (tid < rows_per_wg)
        row_max[tid] = 0u;
    __syncthreads();

    if constexpr (ACT != 0) {
        const int n_threads = (int)blockDim.x;
        const int row_len = (int)K;
        const int elems = rows_per_wg * row_len;
        if constexpr (sizeof(XT) == 2) {
            // bf16: the next piece's raw 16-byte loads are issued before this
            // piece's activation, so that their latency runs under it
            // (4096 x 12288: 124.8 -> 118.9 us in an A/B run; binary32 rows,
            // twice the raw registers, ran 5% slower this way)
            const int stride = 8 * n_threads;
            // Every lane loads every round; a piece past the rows reads row
            // M - 1 instead (in bounds, not used), so that no loaded register
            // is merged with another value before it is needed.
            auto fetch = [&](int ee, v4u &rg, v4u &ru) -> bool {
                const int rl = ee / row_len;
                const int64_t grow = (int64_t)blockIdx.x * rows_per_wg + rl;
                const bool valid = ee < elems && grow < M;
                const int64_t r = valid ? grow : M - 1;
                const int col = valid ? ee - rl * row_len : 0;
                rg = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(X + r * ldx + col));
                ru = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(up + r * ld_up + col));
                return valid;
            };
            int e = 8 * tid;
            v4u rg, ru;
            bool ok = fetch(e, rg, ru);
#pragma unroll 1
            for (; e < elems; e += stride) {
                v4u ng, nu;
                const bool okn = fetch(e + stride, ng, nu);
                if (ok) {
                    float g[8], u[8];
                    widen8(rg, g);
                    widen8(ru, u);
#pragma unroll
                    for (int p = 0; p < 8; ++p)
                        g[p] = gated_act<ACT>(g[p]) * u[p];
                    float *dst = act_stage + act_index(e);
                    *reinterpret_cast<v4f *>(dst) = v4f{g[0], g[1], g[2], g[3]};
                    *reinterpret_cast<v4f *>(dst + 4) = v4f{g[4], g[5], g[6], g[7]};
                }
                rg = ng;
                ru = nu;
                ok = okn;
            }
        } else {
#pragma unroll 1
            for (int e = 8 * tid; e < elems; e += 8 * n_threads) {   // element of the rows laid end to end
                const int rl = e / row_len;
                const int col = e - rl * row_len;
                const int64_t grow = (int64_t)blockIdx.x * rows_per_wg + rl;
                if (grow < M) {
                    float g[8], u[8];
                    load8(X + grow * ldx + col, g);
                    load8(up + grow * ld_up + col, u);
#pragma unroll
                    for (int p = 0; p < 8; ++p)
                        g[p] = gated_act<ACT>(g[p]) * u[p];
                    float *dst = act_stage + act_index(e);
                    *reinterpret_cast<v4f *>(dst) = v4f{g[0], g[1], g[2], g[3]};
                    *reinterpret_cast<v4f *>(dst + 4) = v4f{g[4], g[5], g[6], g[7]};
                }
            }
        }
        __syncthreads();
        if (live) {
            const int base = row_local * row_len + (int)span0;
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const float *src = act_stage + act_index(base + chunk_offset(j0, j1, c));
                const v4f a = *reinterpret_cast<const v4f *>(src);
                const v4f b = *reinterpret_cast<const v4f *>(src + 4);
                v[c][0] = a.x; v[c][1] = a.y; v[c][2] = a.z; v[c][3] = a.w;
                v[c][4] = b.x; v[c][5] = b.y; v[c][6] = b.z; v[c][7] = b.w;
            }
        }
    } else if constexpr (!PS) {
        if (live) {
            const XT *xr = X + row * ldx + span0;
#pragma unroll
            for (int c = 0; c < NC; ++c)
                load8(xr + 8 * j0 + 16 * (c & 1) + 32 * j1 + 64 * (c >> 1), v[c]);
        }
    }
    if constexpr (RMS) {
        const int row_blocks = quads_per_row * kBlocks;
        if constexpr (NRM == kNormMean) {
            // Norm: the row mean first, summed in the same tree (block sums,
            // then the row's block sums left to right), and every value
            // centred on it; the squares below are then the deviations'.
            // norm_part and norm_r are next written after the barrier that
            // follows every read here.
            if (live) {
                float bs[kBlocks];
                block_sums<NC, false>(v, bs);
                if ((tid & 3) == 0)
#pragma unroll
                    for (int b = 0; b < kBlocks; ++b)
                        norm_part[row_local * row_blocks + q_in_row * kBlocks + b] = bs[b];
            }
            __syncthreads();
            if (tid < rows_per_wg) {
                const float *bp = norm_part + tid * row_blocks;
                float sum = bp[0];
                for (int b = 1; b < row_blocks; ++b)
                    sum = sum + bp[b];
                norm_r[tid] = __fdiv_rn(sum, (float)K);
            }
            __syncthreads();
            if (live) {
                const float mean = norm_r[row_local];
#pragma unroll
                for (int c = 0; c < NC; ++c)
#pragma unroll
                    for (int p = 0; p < 8; ++p)
                        v[c][p] = v[c][p] - mean;
            }
        }
        if (live) {
            float bs[kBlocks];
            block_sums<NC, true>(v, bs);
            if ((tid & 3) == 0)
#pragma unroll
                for (int b = 0; b < kBlocks; ++b)
                    norm_part[row_local * row_blocks + q_in_row * kBlocks + b] = bs[b];
        }
        __syncthreads();
        if (tid < rows_per_wg) {
            const float *bp = norm_part + tid * row_blocks;
            float sum = bp[0];
            for (int b = 1; b < row_blocks; ++b)
                sum = sum + bp[b];
            const float mean = __fdiv_rn(sum, (float)K);
            norm_r[tid] = __fdiv_rn(1.0f, sqrt_rn(mean + eps));
        }
        __syncthreads();
        if (live) {
            const float r = norm_r[row_local];
#pragma unroll
            for (int c = 0; c < NC; ++c)
#pragma unroll
                for (int p = 0; p < 8; ++p)
                    v[c][p] = v[c][p] * r;
            if (norm_weight) {
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    if constexpr (PS)
                        weight8_lds(v[c], p_weight, (int)span0 + chunk_offset(j0, j1, c));
                    else
                        weight8(v[c], norm_weight, span0 + chunk_offset(j0, j1, c));
                }
            }
        }
    }
    if (live) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            if constexpr (PS)
                modulate8_lds<MOD>(v[c], p_scale, p_shift, (int)span0 + chunk_offset(j0, j1, c));
            else
                modulate8<MOD>(v[c], mod_scale, mod_shift, span0 + chunk_offset(j0, j1, c));
        }

        if constexpr (SCALED) {
#pragma unroll
            for (int c = 0; c < NC; ++c)
#pragma unroll
                for (int p = 0; p < 8; ++p)
                    v[c][p] = v[c][p] * alpha;
        }

        rotate_span<G, NC, LS>(v);

        // row max: lane, quad (DPP), then the row's quads (LDS)
        const float m = quad_abs_max<NC>(v);
        if ((tid & 3) == 0)
            atomicMax(&row_max[row_local], __builtin_bit_cast(unsigned, m));
    }
    __syncthreads();
    // Wave stores (wave_store != 0; plain rows, whole waves): each wave's 16
    // quads own 16 consecutive spans of the packed codes.  The codes go
    // through a wave-private LDS region and leave it as 1 KB per store
    // instruction.  Every lane takes part in the stores (it may carry pieces
    // of other quads), so no lane returns early on this path.
    if constexpr (ACT == 0 && MOD == 0 && !RMS) {
      if (wave_store) {
        constexpr int kSpan = 32 * NC;
        const int wave = tid >> 6, lane = tid & 63;
        int8_t *stage = reinterpret_cast<int8_t *>(act_stage) + wave * (16 * kSpan);
        const int quad_w = (tid >> 2) & 15;
        if (row < M_pad) {
            int8_t *sq = stage + quad_w * kSpan;
            if (!live) {
#pragma unroll
                for (int c = 0; c < NC; c += 2)
                    *reinterpret_cast<v4u *>(sq + chunk_offset(0, j1, c) + 16 * j0) = v4u{0u, 0u, 0u, 0u};
                if (q_in_row == 0 && (tid & 3) == 0)
                    S[row] = 0.0f;
            } else {
                const float m = __builtin_bit_cast(float, row_max[row_local]);
                const float inv = m > 0.0f ? __fdiv_rn(127.0f, m) : 0.0f;
                if (q_in_row == 0 && (tid & 3) == 0)
                    S[row] = __fdiv_rn(m, 127.0f);
#pragma unroll
                for (int c = 0; c < NC; c += 2)
                    *reinterpret_cast<v4u *>(sq + chunk_offset(0, j1, c) + 16 * j0) = encode_pair16(v[c], v[c + 1], inv, j0);
            }
        }
        wave_lds_sync();   // lanes store pieces other lanes staged
        const int64_t wave_q0 = (int64_t)blockIdx.x * rows_per_wg * quads_per_row + 16 * wave;
        const int64_t q_total = M_pad * quads_per_row;
        const int wg_quads = quads_per_row * rows_per_wg;
        int8_t *dst = Q + wave_q0 * kSpan;
#pragma unroll
        for (int i = 0; i < NC / 2; ++i) {
            const int o = 16 * lane + 1024 * i;
            const int qw = o / kSpan;
            if (16 * wave + qw < wg_quads && wave_q0 + qw < q_total)
                *reinterpret_cast<v4u *>(dst + o) = *reinterpret_cast<const v4u *>(stage + o);
        }
        return;
      }
    }
    if (!worker || row >= M_pad)
        return;

    int8_t *qr = Q + row * K + span0;
    if (!live) {
        // pad rows of the packed tensor: zero codes, zero scale
#pragma unroll
        for (int c = 0; c < NC; ++c)
            *reinterpret_cast<v2u *>(qr + 8 * j0 + 16 * (c & 1) + 32 * j1 + 64 * (c >> 1)) = v2u{0u, 0u};
        if (q_in_row == 0 && (tid & 3) == 0)
            S[row] = 0.0f;
        return;
    }

    const float m = __builtin_bit_cast(float, row_max[row_local]);
    const float inv = m > 0.0f ? __fdiv_rn(127.0f, m) : 0.0f;
    if (q_in_row == 0 && (tid & 3) == 0)
        S[row] = __fdiv_rn(m, 127.0f);
#pragma unroll
    for (int c = 0; c < NC; c += 2)
        *reinterpret_cast<v4u *>(qr + chunk_offset(0, j1, c) + 16 * j0) = encode_pair16(v[c], v[c + 1], inv, j0);
}

// ---- binary32 inputs: the same arithmetic with the row data staged in LDS.
//
// A wave's 16 quads own 16 consecutive spans (16 KB of binary32).  The quad
// layout above makes every load instruction touch two 32-byte pieces per
// quad; here each load instruction instead reads 64 consecutive 16-byte
// pieces (1 KB), which the memory system serves at a clearly higher rate.
// The pieces go to a wave-private LDS region and each lane reads back its own
// chunks; the codes take the same route in reverse, so stores are also 1 KB
// per instruction.  LDS operations of one wave complete in order, so the
// region needs no workgroup barrier, only a wave-scope fence that keeps the
// compiler's order (wave_lds_sync).  Odd quads store their pieces with the slot index
// XOR-ed by one (codes: by 4 * (quad % 4)) so that the lanes of one read
// instruction spread over distinct LDS banks.
//
// NS = 2: one pass for two input scales (no producer).  The rows are loaded
// and staged once; every lane scales and rotates its chunks for both scales
// in registers, the row maxima of both meet at one barrier, and the codes of
// each scale go out in turn through the staging region.  Each scale's bytes
// are those of its own pass.
template <int G, int NC, bool SCALED, int MOD, int NS = 1>
__global__ __launch_bounds__(256) void quantize_rows_staged(
    const float *__restrict__ X, int64_t M, int64_t M_pad, int64_t K, int64_t ldx, float alpha,
    const float *__restrict__ mod_scale, const float *__restrict__ mod_shift,
    int8_t *__restrict__ Q, float *__restrict__ S, int quads_per_row, int rows_per_wg,
    ScaleOuts outs)
{
    constexpr bool MULTI = NS > 1;
    static_assert(NS == 1 || (NS == 2 && MOD == 0 && !SCALED), "two scales: plain rows, scales in outs");
    static_assert(NC == 2 || NC == 4 || NC == 8, "chunks per lane");
    static_assert(G == 1 || G == 4 || G == 16 || G == 64 || (G == 256 && NC == 8), "group size vs span");
    constexpr int kPC = 2;                                // 16-B pieces per 8-element chunk
    constexpr int kQuadPieces = 4 * NC * kPC;            // 16-B input pieces per quad span
    constexpr int kWavePieces = 16 * kQuadPieces;        // per wave
    constexpr int kLoadsPerLane = kWavePieces / 64;      // = NC * kPC
    constexpr int kOutPieces = 16 * (32 * NC / 16);      // 16-B code pieces per wave
    constexpr int kStoresPerLane = kOutPieces / 64;      // = NC / 2
    extern __shared__ __attribute__((aligned(16))) unsigned char stage_lds[];
    __shared__ unsigned row_max[NS * 256];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int quad = tid >> 2;
    const int j0 = tid & 1, j1 = (tid >> 1) & 1;
    const int n_quads = quads_per_row * rows_per_wg;
    int row_local, q_in_row;
    quad_place<MOD>(quad, quads_per_row, rows_per_wg, row_local, q_in_row);
    const int64_t row0 = (int64_t)blockIdx.x * rows_per_wg;
    const int64_t row = row0 + row_local;
    const bool live = row < M;
    constexpr int kQuadOut = 32 * NC / 16;                      // 16-B code pieces per quad
    unsigned char *wst = stage_lds + wave * (kWavePieces * 16);
    constexpr int kFlip = 1;

    if (tid < rows_per_wg) {
#pragma unroll
        for (int a = 0; a < NS; ++a)
            row_max[256 * a + tid] = 0u;
    }

    // contiguous loads: lane L, instruction i takes wave piece p = 64 i + L
    using Raw = v4u;
    Raw raw[kLoadsPerLane];
#pragma unroll
    for (int i = 0; i < kLoadsPerLane; ++i) {
        const int p = 64 * i + lane;
        const int qw = 16 * wave + p / kQuadPieces;            // quad within the workgroup
        int rl, qi;
        quad_place<MOD>(qw, quads_per_row, rows_per_wg, rl, qi);
        const int64_t r = row0 + rl;
        if (qw < n_quads && r < M) {
            const unsigned char *src = reinterpret_cast<const unsigned char *>(X + r * ldx + (int64_t)qi * (32 * NC)) +
                                       16 * (p % kQuadPieces);
            raw[i] = __builtin_nontemporal_load(reinterpret_cast<const Raw *>(src));
        }
    }
#pragma unroll
    for (int i = 0; i < kLoadsPerLane; ++i) {
        const int p = 64 * i + lane;
        const int ql = p / kQuadPieces, pi = p % kQuadPieces;
        *reinterpret_cast<Raw *>(wst + 16 * (ql * kQuadPieces + (pi ^ (kFlip * (ql & 1))))) = raw[i];
    }
    __syncthreads();   // row_max cleared (the staging region is wave-private)

    const int ql_me = (tid >> 2) & 15;                          // my quad within the wave
    float v[NS][NC][8];
    if (live) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int e = 8 * j0 + 16 * (c & 1) + 32 * j1 + 64 * (c >> 1);   // element offset in the span
#pragma unroll
            for (int h = 0; h < kPC; ++h) {
                const int pi = e / 4 + h;
                const Raw u = *reinterpret_cast<const Raw *>(wst + 16 * (ql_me * kQuadPieces + (pi ^ (kFlip * (ql_me & 1)))));
                // the element is converted to a value before the bit cast:
                // a bit cast of a vector element lvalue reads element 0 with
                // this toolchain
                const unsigned w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    v[0][c][4 * h + t] = __builtin_bit_cast(float, w[t]);
            }
        }
        const int64_t span_me = (int64_t)q_in_row * (32 * NC);
#pragma unroll
        for (int c = 0; c < NC; ++c)
            modulate8<MOD>(v[0][c], mod_scale, mod_shift, span_me + 8 * j0 + 16 * (c & 1) + 32 * j1 + 64 * (c >> 1));
#pragma unroll
        for (int a = NS - 1; a >= 0; --a) {
            const float alpha_a = MULTI ? outs.alpha[a] : alpha;
            if (SCALED || (MULTI && alpha_a != 1.0f)) {
#pragma unroll
                for (int c = 0; c < NC; ++c)
#pragma unroll
                    for (int p = 0; p < 8; ++p)
                        v[a][c][p] = v[0][c][p] * alpha_a;
            } else if (a > 0) {
#pragma unroll
                for (int c = 0; c < NC; ++c)
#pragma unroll
                    for (int p = 0; p < 8; ++p)
                        v[a][c][p] = v[0][c][p];
            }
            rotate_span<G, NC, MOD == 0>(v[a]);
            const float m = quad_abs_max<NC>(v[a]);
            if ((tid & 3) == 0)
                atomicMax(&row_max[256 * a + row_local], __builtin_bit_cast(unsigned, m));
        }
    }
    __syncthreads();

#pragma unroll
    for (int a = 0; a < NS; ++a) {
        int8_t *const Qa = MULTI ? outs.Q[a] : Q;
        float *const Sa = MULTI ? outs.S[a] : S;
        if constexpr (MULTI) {
            if (a > 0)
                wave_lds_sync();   // these codes reuse the region the last stores read
        }
        // codes: 8 bytes per chunk into the wave's staging region (32 NC bytes
        // per quad), then contiguous 16-B stores
        if (row < M_pad) {
            unsigned char *qst = wst + 16 * ql_me * kQuadOut;
            if (!live) {
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    const int o = 8 * j0 + 16 * (c & 1) + 32 * j1 + 64 * (c >> 1);
                    *reinterpret_cast<v2u *>(qst + 16 * ((o >> 4) ^ (4 * (ql_me & 3) % kQuadOut)) + (o & 15)) = v2u{0u, 0u};
                }
                if (q_in_row == 0 && (tid & 3) == 0)
                    Sa[row] = 0.0f;
            } else {
                const float m = __builtin_bit_cast(float, row_max[256 * a + row_local]);
                const float inv = m > 0.0f ? __fdiv_rn(127.0f, m) : 0.0f;
                if (q_in_row == 0 && (tid & 3) == 0)
                    Sa[row] = __fdiv_rn(m, 127.0f);
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    const int o = chunk_offset(j0, j1, c);
                    *reinterpret_cast<v2u *>(qst + 16 * ((o >> 4) ^ (4 * (ql_me & 3) % kQuadOut)) + (o & 15)) = encode8(v[a][c], inv);
                }
            }
        }
        wave_lds_sync();   // lanes store pieces other lanes staged
#pragma unroll
        for (int i = 0; i < kStoresPerLane; ++i) {
            const int p = 64 * i + lane;                            // wave code piece
            const int ql = p / kQuadOut, pi = p % kQuadOut;
            const int qw = 16 * wave + ql;
            int rl, qi;
            quad_place<MOD>(qw, quads_per_row, rows_per_wg, rl, qi);
            const int64_t r = row0 + rl;
            if (qw < n_quads && r < M_pad) {
                const v4u val = *reinterpret_cast<const v4u *>(wst + 16 * (ql * kQuadOut + (pi ^ (4 * (ql & 3) % kQuadOut))));
                *reinterpret_cast<v4u *>(Qa + r * K + (int64_t)qi * (32 * NC) + 16 * pi) = val;
            }
        }
    }
}

// LDS bytes per wave of the staged kernel (16 quads of 32 NC binary32 values).
template <int NC>
constexpr size_t kStagedWaveBytes = 16 * 32 * NC * 4;

template <int G, int NC, int MOD>
hipError_t launch_staged(const float *X, int64_t M, int64_t K, int64_t ldx, float alpha, const PreOp &pre,
                   int8_t *Q, float *S, int64_t m_pad, int qr, int rows, hipStream_t stream)
{
    const int threads = 4 * qr * rows;
    const size_t lds = (size_t)((threads + 63) / 64) * kStagedWaveBytes<NC>;
    const int64_t blocks = (m_pad + rows - 1) / rows;
    if (alpha != 1.0f)
        hipLaunchKernelGGL((quantize_rows_staged<G, NC, true, MOD>), dim3((unsigned)blocks), dim3(threads), lds,
                           stream, X, M, m_pad, K, ldx, alpha, pre.scale, pre.shift, Q, S, qr, rows, ScaleOuts{});
    else
        hipLaunchKernelGGL((quantize_rows_staged<G, NC, false, MOD>), dim3((unsigned)blocks), dim3(threads), lds,
                           stream, X, M, m_pad, K, ldx, alpha, pre.scale, pre.shift, Q, S, qr, rows, ScaleOuts{});
    return hipGetLastError();
}

// Two scales in one staged pass (binary32 rows, no producer).
template <int G, int NC>
hipError_t launch_staged_scales(const float *X, int64_t M, int64_t K, int64_t ldx, const ScaleOuts &outs,
                                int64_t m_pad, int qr, int rows, hipStream_t stream)
{
    const int threads = 4 * qr * rows;
    const size_t lds = (size_t)((threads + 63) / 64) * kStagedWaveBytes<NC>;
    const int64_t blocks = (m_pad + rows - 1) / rows;
    hipLaunchKernelGGL((quantize_rows_staged<G, NC, false, 0, 2>), dim3((unsigned)blocks), dim3(threads), lds,
                       stream, X, M, m_pad, K, ldx, 1.0f, nullptr, nullptr, nullptr, nullptr, qr, rows, outs);
    return hipGetLastError();
}

int gcd_int(int a, int b)
{
    while (b) {
        const int t = a % b;
        a = b;
        b = t;
    }
    return a;
}

// Rows per workgroup for qr quads per row: the smallest row count that fills
// whole waves, then grown towards 256 threads.
int plan_rows(int qr, int max_threads)
{
    int rows = 16 / gcd_int(qr, 16);
    if (4 * qr * rows > max_threads)
        rows = max_threads / (4 * qr) > 0 ? max_threads / (4 * qr) : 1;
    while (4 * qr * rows * 2 <= 256)
        rows *= 2;
    return rows;
}

template <typename XT, int G, int NC, int MOD, int NRM, int ACT>
hipError_t launch_typed(const void *X, int64_t M, int64_t K, int64_t ldx, float alpha, const PreOp &pre,
                  void *packed, hipStream_t stream)
{
    constexpr bool RMS = NRM != kNormNone;
    const int64_t m_pad = (M + 3) / 4 * 4;
    const int qr = (int)(K / (32 * NC));
    constexpr int kMaxThreads = (RMS || ACT != 0) ? 512 : 1024;
    // the producer's per-channel vectors go to LDS when they fit
    const int64_t n_vec = (MOD != 0 ? 1 : 0) + (MOD == 2 ? 1 : 0) + (RMS && pre.norm_weight ? 1 : 0);
    const size_t vec_bytes = (size_t)(4 * K * n_vec);
    const bool stage_vec = ACT == 0 && MOD != 0 && vec_bytes <= (size_t)kParamLdsBytes;
    int rows = plan_rows(qr, kMaxThreads);
    if (sizeof(XT) == 2 && stage_vec && !RMS) {
        // every workgroup copies the vectors once: workgroups of up to 1024
        // threads share the copy among more rows (4096 x 3072 bf16 with
        // scale and shift: 16 rows, 13.56 -> 12.87 us in an A/B run; RMSNorm's
        // 512-thread kernels gained nothing from more rows)
        while (4 * qr * rows * 2 <= kMaxThreads)
            rows *= 2;
    }
    int threads = 4 * qr * rows;
    // the gated activation doubles the threads of its activation pass where
    // the launch bounds allow (the quad layout keeps 4 * qr * rows of them)
    if (ACT != 0 && 2 * threads <= kMaxThreads)
        threads *= 2;
    const int64_t blocks = (m_pad + rows - 1) / rows;
    int8_t *Q = static_cast<int8_t *>(packed);
    float *S = reinterpret_cast<float *>(Q + m_pad * K);
    if constexpr (sizeof(XT) == 4 && !RMS && ACT == 0) {
        // binary32 rows of up to 256 threads per workgroup take the staged kernel
        if (threads <= 256)
            return launch_staged<G, NC, MOD>(static_cast<const float *>(X), M, K, ldx, alpha, pre, Q,
                                             S, m_pad, qr, rows, stream);
    }
    const XT *up = static_cast<const XT *>(pre.up);
    // the gated activation stages the workgroup's rows in LDS (at most 512
    // threads of 64 elements: 130 KB)
    // Plain rows in whole waves store their codes through LDS, 1 KB per store
    // instruction, when the pass runs many rounds of waves (at least 8192
    // waves): on the 16384 x 12288 bf16 pass that took 101.7 -> 95.6 us, while
    // a pass of one round (4096 x 3072 bf16, 3072 waves) ran 4% slower.
    const int64_t total_waves = blocks * ((threads + 63) / 64);
    const int wave_store = ACT == 0 && MOD == 0 && !RMS && threads % 64 == 0 && total_waves >= 8192;
    const size_t lds = ACT != 0 ? act_stage_bytes((int64_t)rows * K)
                       : stage_vec ? vec_bytes
                       : wave_store ? (size_t)(threads / 64) * 16 * 32 * NC : 0;
    // the kernel's static LDS: row maxima, and RMSNorm's block sums and factors
    constexpr size_t kStaticLds = 4 * 256 + (RMS ? 4 * 256 * (NC / 2) + 4 * 256 : 8);
    auto go = [&](auto ps, auto ls) -> hipError_t {
        constexpr bool PS = decltype(ps)::value;
        constexpr bool LS = decltype(ls)::value;
        if (lds + kStaticLds > 64 * 1024) {
            // beyond the default LDS limit of a launch: raise the kernel's
            // dynamic maximum first, and make no launch if that fails
            const void *fn =
                alpha != 1.0f ? reinterpret_cast<const void *>(&quantize_rows_kernel<XT, G, NC, true, MOD, NRM, ACT, PS, LS>)
                              : reinterpret_cast<const void *>(&quantize_rows_kernel<XT, G, NC, false, MOD, NRM, ACT, PS, LS>);
            const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e != hipSuccess)
                return e;
        }
        if (alpha != 1.0f)
            hipLaunchKernelGGL((quantize_rows_kernel<XT, G, NC, true, MOD, NRM, ACT, PS, LS>), dim3((unsigned)blocks),
                               dim3(threads), lds, stream, static_cast<const XT *>(X), M, m_pad, K, ldx,
                               alpha, pre.scale, pre.shift, pre.norm_weight, pre.eps, up, pre.ld_up, Q, S,
                               qr, rows, wave_store);
        else
            hipLaunchKernelGGL((quantize_rows_kernel<XT, G, NC, false, MOD, NRM, ACT, PS, LS>), dim3((unsigned)blocks),
                               dim3(threads), lds, stream, static_cast<const XT *>(X), M, m_pad, K, ldx,
                               alpha, pre.scale, pre.shift, pre.norm_weight, pre.eps, up, pre.ld_up, Q, S,
                               qr, rows, wave_store);
        return hipGetLastError();
    };
    if constexpr (ACT == 0 && MOD != 0) {
        if (stage_vec)
            return go(std::true_type{}, std::false_type{});
    }
    if constexpr (ACT == 0 && MOD == 0 && !RMS) {
        // Plain rows with direct code stores (passes of few wave rounds) run
        // the rotation's split digits four in lockstep: identical bytes, in
        // an A/B run 4096 x 3072 bf16 10.45 -> 10.04 us.  Passes of many rounds
        // (the wave-store path) keep the plain order: there the lockstep form
        // measured 105.5 -> 110.1 us on 16384 x 12288 bf16.
        if (!wave_store)
            return go(std::false_type{}, std::true_type{});
    }
    return go(std::false_type{}, std::false_type{});
}

template <typename XT, int NC, int MOD, int NRM, int ACT>
hipError_t launch_nc(int G, const void *X, int64_t M, int64_t K, int64_t ldx, float alpha,
                     const PreOp &pre, void *packed, hipStream_t stream)
{
    switch (G) {
    case 1: return launch_typed<XT, 1, NC, MOD, NRM, ACT>(X, M, K, ldx, alpha, pre, packed, stream);
    case 4: return launch_typed<XT, 4, NC, MOD, NRM, ACT>(X, M, K, ldx, alpha, pre, packed, stream);
    case 16: return launch_typed<XT, 16, NC, MOD, NRM, ACT>(X, M, K, ldx, alpha, pre, packed, stream);
    case 64: return launch_typed<XT, 64, NC, MOD, NRM, ACT>(X, M, K, ldx, alpha, pre, packed, stream);
    default:
        if constexpr (NC == 8)
            return launch_typed<XT, 256, 8, MOD, NRM, ACT>(X, M, K, ldx, alpha, pre, packed, stream);
        return hipErrorInvalidValue;   // not reached: the API admits G = 256 only with K % 256 == 0
    }
}

template <typename XT, int MOD, int NRM, int ACT>
hipError_t launch_dtype(int G, const void *X, int64_t M, int64_t K, int64_t ldx, float alpha,
                        const PreOp &pre, void *packed, hipStream_t stream)
{
    if (K % 256 == 0)
        return launch_nc<XT, 8, MOD, NRM, ACT>(G, X, M, K, ldx, alpha, pre, packed, stream);
    if (K % 128 == 0)
        return launch_nc<XT, 4, MOD, NRM, ACT>(G, X, M, K, ldx, alpha, pre, packed, stream);
    return launch_nc<XT, 2, MOD, NRM, ACT>(G, X, M, K, ldx, alpha, pre, packed, stream);
}

template <typename XT, int NRM>
hipError_t launch_mod(int G, const void *X, int64_t M, int64_t K, int64_t ldx, float alpha,
                      const PreOp &pre, void *packed, hipStream_t stream)
{
    if (pre.scale && pre.shift)
        return launch_dtype<XT, 2, NRM, 0>(G, X, M, K, ldx, alpha, pre, packed, stream);
    if (pre.scale)
        return launch_dtype<XT, 1, NRM, 0>(G, X, M, K, ldx, alpha, pre, packed, stream);
    return launch_dtype<XT, 0, NRM, 0>(G, X, M, K, ldx, alpha, pre, packed, stream);
}

template <typename XT>
hipError_t launch_pre(int G, const void *X, int64_t M, int64_t K, int64_t ldx, float alpha,
                      const PreOp &pre, void *packed, hipStream_t stream)
{
    if (pre.kind == kPreRmsNormModulate)
        return launch_mod<XT, kNormRms>(G, X, M, K, ldx, alpha, pre, packed, stream);
    if (pre.kind == kPreNormMul)
        return launch_dtype<XT, 0, kNormMean, 0>(G, X, M, K, ldx, alpha, pre, packed, stream);
    if (pre.kind == kPreGatedAct && pre.act == kActSilu)
        return launch_dtype<XT, 0, kNormNone, kActSilu>(G, X, M, K, ldx, alpha, pre, packed, stream);
    if (pre.kind == kPreGatedAct)
        return launch_dtype<XT, 0, kNormNone, kActSigmoid>(G, X, M, K, ldx, alpha, pre, packed, stream);
    return launch_mod<XT, kNormNone>(G, X, M, K, ldx, alpha, pre, packed, stream);
}

// y may be x (each lane reads its element before writing it).
__global__ __launch_bounds__(256) void expf_kernel(const float *x, float *y, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n)
        y[i] = convrot_expf::expf_cr(x[i]);
}

}  // namespace

hipError_t launch_expf(const float *x, float *y, int64_t n, hipStream_t stream)
{
    const int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(expf_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, x, y, n);
    return hipGetLastError();
}

hipError_t launch_quantize(const void *X, int x_dtype, int64_t M, int64_t K, int64_t ldx, int G,
                           float alpha, const PreOp &pre, void *packed, hipStream_t stream)
{
    if (x_dtype == 0)
        return launch_pre<float>(G, X, M, K, ldx, alpha, pre, packed, stream);
    return launch_pre<uint16_t>(G, X, M, K, ldx, alpha, pre, packed, stream);
}

namespace {

template <int NC>
hipError_t launch_scales_nc(int G, const float *X, int64_t M, int64_t K, int64_t ldx, const ScaleOuts &outs,
                            int64_t m_pad, int qr, int rows, hipStream_t stream)
{
    switch (G) {
    case 1: return launch_staged_scales<1, NC>(X, M, K, ldx, outs, m_pad, qr, rows, stream);
    case 4: return launch_staged_scales<4, NC>(X, M, K, ldx, outs, m_pad, qr, rows, stream);
    case 16: return launch_staged_scales<16, NC>(X, M, K, ldx, outs, m_pad, qr, rows, stream);
    case 64: return launch_staged_scales<64, NC>(X, M, K, ldx, outs, m_pad, qr, rows, stream);
    default:
        if constexpr (NC == 8)
            return launch_staged_scales<256, 8>(X, M, K, ldx, outs, m_pad, qr, rows, stream);
        return hipErrorInvalidValue;   // not reached: G = 256 comes with K % 256 == 0
    }
}

}  // namespace

hipError_t launch_quantize_scales(const void *X, int x_dtype, int64_t M, int64_t K, int64_t ldx, int G,
                                  int n, const float *alpha, void *const *packed, hipStream_t stream)
{
    // the staged kernel's rows: binary32 with at most 256 threads per
    // workgroup (the choice launch_typed makes for plain rows)
    const int nc = K % 256 == 0 ? 8 : K % 128 == 0 ? 4 : 2;
    const int qr = (int)(K / (32 * nc));
    const int rows = plan_rows(qr, 1024);
    const bool staged = x_dtype == 0 && 4 * qr * rows <= 256;
    if (!staged || n < 2) {
        for (int i = 0; i < n; ++i) {
            const hipError_t e = launch_quantize(X, x_dtype, M, K, ldx, G, alpha[i], PreOp{}, packed[i], stream);
            if (e != hipSuccess)
                return e;
        }
        return hipSuccess;
    }
    const int64_t m_pad = (M + 3) / 4 * 4;
    for (int i0 = 0; i0 < n; i0 += kMaxPassScales) {
        if (n - i0 == 1)      // an odd scale left over: its own pass
            return launch_quantize(X, x_dtype, M, K, ldx, G, alpha[i0], PreOp{}, packed[i0], stream);
        ScaleOuts outs{};
        outs.n = kMaxPassScales;
        for (int a = 0; a < outs.n; ++a) {
            outs.alpha[a] = alpha[i0 + a];
            outs.Q[a] = static_cast<int8_t *>(packed[i0 + a]);
            outs.S[a] = reinterpret_cast<float *>(outs.Q[a] + m_pad * K);
        }
        const float *Xf = static_cast<const float *>(X);
        const hipError_t e = nc == 8 ? launch_scales_nc<8>(G, Xf, M, K, ldx, outs, m_pad, qr, rows, stream)
                             : nc == 4 ? launch_scales_nc<4>(G, Xf, M, K, ldx, outs, m_pad, qr, rows, stream)
                                       : launch_scales_nc<2>(G, Xf, M, K, ldx, outs, m_pad, qr, rows, stream);
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

}  // namespace convrot_detail
