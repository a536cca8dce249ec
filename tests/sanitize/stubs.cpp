// Host stand-ins for the kernel launchers, so that the C ABI's validation,
// workspace carving and dispatch run under the host sanitizers with no GPU:
// each launcher records what it was asked to launch.  Test infrastructure.
#include "kernels.h"
#include "stubs.h"

namespace convrot_detail {

StubLog g_log;
static int8_t g_static_ws[4096];

hipError_t launch_expf(const float *, float *, int64_t n, hipStream_t)
{
    g_log.expf_calls++;
    g_log.last_n = n;
    return hipSuccess;
}

hipError_t launch_quantize(const void *X, int x_dtype, int64_t M, int64_t K, int64_t ldx, int G,
                           float alpha, const PreOp &pre, void *packed, hipStream_t)
{
    g_log.quantize_calls++;
    g_log.q_X = X;
    g_log.q_dtype = x_dtype;
    g_log.q_M = M;
    g_log.q_K = K;
    g_log.q_ldx = ldx;
    g_log.q_G = G;
    g_log.q_alpha = alpha;
    g_log.q_pre = pre.kind;
    g_log.q_packed = packed;
    return hipSuccess;
}

hipError_t launch_quantize_scales(const void *X, int x_dtype, int64_t M, int64_t K, int64_t ldx, int G,
                                  int n, const float *alpha, void *const *packed, hipStream_t stream)
{
    // recorded as one call, and as the passes it stands for
    g_log.scales_calls++;
    g_log.q_n = n;
    for (int i = 0; i < n; ++i)
        launch_quantize(X, x_dtype, M, K, ldx, G, alpha[i], PreOp{}, packed[i], stream);
    return hipSuccess;
}

hipError_t launch_gemm(GemmProblem p, hipStream_t)
{
    g_log.gemm_calls++;
    g_log.gemm = p;
    return hipSuccess;
}

hipError_t static_workspace(void **ptr)
{
    *ptr = g_static_ws;
    return hipSuccess;
}

}  // namespace convrot_detail
