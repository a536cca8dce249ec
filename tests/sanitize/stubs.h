// What the host stand-ins of the kernel launchers record.  Test infrastructure.
#pragma once
#include "kernels.h"

namespace convrot_detail {

struct StubLog {
    int quantize_calls = 0, gemm_calls = 0, expf_calls = 0, scales_calls = 0, q_n = 0;
    int64_t last_n = 0;
    const void *q_X = nullptr;
    int q_dtype = -1;
    int64_t q_M = 0, q_K = 0, q_ldx = 0;
    int q_G = 0;
    float q_alpha = 0.0f;
    int q_pre = -1;
    void *q_packed = nullptr;
    GemmProblem gemm{};
};

extern StubLog g_log;

}  // namespace convrot_detail
