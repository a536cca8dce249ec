// Measurement kernels for the roofline report, built into their own library
// (libconvrot_probe.so) and not part of the convrot interface.
//
// convrot_probe_mfma: the int8 MFMA rate the chip sustains on given codes
// when nothing but MFMAs run.
// It has the contraction kernel's occupancy and wave shape: workgroups of 8
// waves holding 132 KB of LDS (one per CU, two waves per SIMD), each wave
// repeating the 32 v_mfma_i32_16x16x64_i8 of one 64-byte K step of a
// 128 x 64 wave tile, on 8 A and 4 B fragments loaded once from the codes it
// is given.  With no loads, LDS traffic or barriers in the loop, what limits
// the rate is the matrix units and the clock the board's power limit allows
// for those codes.
//
// convrot_probe_copy: the quantize pass's memory traffic with no arithmetic,
// as a ceiling for it: read a row-major [n] tensor of 2- or 4-byte elements
// and write one byte per element (the element's top byte), with 16-byte
// loads and stores.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 512;
constexpr int kProbeLds = 132 * 1024;

__global__ __launch_bounds__(kProbeThreads, 1) void probe_mfma_kernel(
    const int8_t *__restrict__ qa, int64_t a_bytes, const int8_t *__restrict__ qb, int64_t b_bytes,
    int steps, int32_t *__restrict__ out)
{
    __shared__ int8_t hold[kProbeLds];   // occupancy only: one workgroup per CU
    const int tid = threadIdx.x;
    const int64_t gid = (int64_t)blockIdx.x * kProbeThreads + tid;
    // fragments: 16 consecutive code bytes per lane, from spread-out places
    v4i fa[8], fb[4];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t off = ((gid * 8 + i) * 4099 * 16) % (a_bytes - 16);
        fa[i] = *reinterpret_cast<const v4i *>(qa + (off & ~(int64_t)15));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t off = ((gid * 4 + j) * 4111 * 16) % (b_bytes - 16);
        fb[j] = *reinterpret_cast<const v4i *>(qb + (off & ~(int64_t)15));
    }
    v4i acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = v4i{0, 0, 0, 0};
    for (int s = 0; s < steps; ++s) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    int x = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            x ^= acc[i][j][0] ^ acc[i][j][1] ^ acc[i][j][2] ^ acc[i][j][3];
    hold[tid] = (int8_t)x;
    __syncthreads();
    out[gid] = x + hold[(tid + 1) % kProbeThreads];
}

typedef unsigned v4u __attribute__((ext_vector_type(4)));

// One chunk = 16 output bytes = 16 input elements (ESZ bytes each).
template <int ESZ>
__global__ __launch_bounds__(256) void probe_copy_kernel(const v4u *__restrict__ x, v4u *__restrict__ y,
                                                         int64_t chunks)
{
    constexpr int kIn = ESZ;                       // 16-byte input pieces per chunk
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < chunks; c += stride) {
        v4u in[kIn];
#pragma unroll
        for (int k = 0; k < kIn; ++k)
            in[k] = __builtin_nontemporal_load(x + c * kIn + k);
        unsigned w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            // top bytes of the four elements of output word q
            if constexpr (ESZ == 4) {
                const v4u a = in[q];
                w[q] = __builtin_amdgcn_perm(a.y, a.x, 0x0c0c0703u) | __builtin_amdgcn_perm(a.w, a.z, 0x07030c0cu);
            } else {
                const v4u a = in[q / 2];
                const unsigned lo = (q & 1) ? a.z : a.x, hi = (q & 1) ? a.w : a.y;
                w[q] = __builtin_amdgcn_perm(hi, lo, 0x07050301u);
            }
        }
        __builtin_nontemporal_store(v4u{w[0], w[1], w[2], w[3]}, y + c);
    }
}

}  // namespace

extern "C" {

// y[i] = top byte of x[i] for n elements of esz (2 or 4) bytes; x and y
// 16-byte aligned device pointers, n a multiple of 16.  Returns a hipError_t.
int convrot_probe_copy(const void *x, int esz, int64_t n, void *y, void *stream)
{
    if (!x || !y || n < 16 || n % 16 != 0 || (esz != 2 && esz != 4))
        return (int)hipErrorInvalidValue;
    const int64_t chunks = n / 16;
    const int64_t want = (chunks + 255) / 256;
    const unsigned blocks = (unsigned)(want < 8192 ? want : 8192);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (esz == 2)
        hipLaunchKernelGGL(probe_copy_kernel<2>, dim3(blocks), dim3(256), 0, st,
                           static_cast<const v4u *>(x), static_cast<v4u *>(y), chunks);
    else
        hipLaunchKernelGGL(probe_copy_kernel<4>, dim3(blocks), dim3(256), 0, st,
                           static_cast<const v4u *>(x), static_cast<v4u *>(y), chunks);
    return (int)hipGetLastError();
}


// Runs blocks x 512 threads, each wave issuing steps x 32 MFMAs (2 * 16 * 16
// * 64 int8 operations each).  qa, qb: device codes of a_bytes, b_bytes
// (>= 32 each); out: blocks * 512 int32 (device).  Returns a hipError_t.
int convrot_probe_mfma(const int8_t *qa, int64_t a_bytes, const int8_t *qb, int64_t b_bytes,
                       int steps, int blocks, int32_t *out, void *stream)
{
    if (!qa || !qb || !out || a_bytes < 32 || b_bytes < 32 || steps < 1 || blocks < 1)
        return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(probe_mfma_kernel, dim3(blocks), dim3(kProbeThreads), 0,
                       static_cast<hipStream_t>(stream), qa, a_bytes, qb, b_bytes, steps, out);
    return (int)hipGetLastError();
}

}  // extern "C"
