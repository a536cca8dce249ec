// Drives every entry point of the C ABI through its host-side validation and
// dispatch, built with the host compiler's address and undefined-behaviour
// sanitizers against stand-in launchers (stubs.cpp): valid calls must reach
// the launchers with the expected arguments, invalid ones must return their
// status without reaching them.  Pointers are fake, aligned addresses that
// nothing dereferences.  Prints "abi ok" and exits 0 on success.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <limits>

#include "../../include/convrot.h"
#include "stubs.h"

using convrot_detail::g_log;

static int failures = 0;

#define EXPECT(cond)                                                            \
    do {                                                                        \
        if (!(cond)) {                                                          \
            std::fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #cond); \
            ++failures;                                                         \
        }                                                                       \
    } while (0)

static void *at(uintptr_t mib) { return reinterpret_cast<void *>((uintptr_t)0x7F0000000000ull + (mib << 20)); }
template <typename T> static T *at_t(uintptr_t mib) { return static_cast<T *>(at(mib)); }

static void reset() { g_log = convrot_detail::StubLog{}; }

static void sizes()
{
    EXPECT(convrot_packed_bytes(0, 256) == 0);
    EXPECT(convrot_packed_bytes(1, 256) == 4 * 256 + 16);
    EXPECT(convrot_packed_bytes(5, 64) == 8 * 64 + 32);
    EXPECT(convrot_packed_bytes(-1, 64) == 0);
    EXPECT(convrot_packed_bytes(4, 0) == 0);
    EXPECT(convrot_workspace_bytes(5, 64, 2) == 2 * 768);
    EXPECT(convrot_workspace_bytes(5, 64, -1) == 0);
    // sizes whose byte counts do not fit are reported as 0, not wrapped
    EXPECT(convrot_packed_bytes(std::numeric_limits<int64_t>::max(), 1 << 20) == 0);
    EXPECT(convrot_workspace_bytes(std::numeric_limits<int64_t>::max() / 2, 1 << 20, 4) == 0);
}

static void quantize()
{
    reset();
    EXPECT(convrot_quantize_rows(at(0), CONVROT_BF16, 7, 3072, 3072, 256, 0.5f, at(64), nullptr) == CONVROT_OK);
    EXPECT(g_log.quantize_calls == 1 && g_log.q_M == 7 && g_log.q_K == 3072 && g_log.q_G == 256);
    EXPECT(g_log.q_alpha == 0.5f && g_log.q_packed == at(64) && g_log.q_dtype == CONVROT_BF16);
    reset();
    EXPECT(convrot_quantize_rows(at(0), CONVROT_F32, 7, 3072, 3072, 2, 1.0f, at(64), nullptr) == CONVROT_EUNSUPPORTED);
    EXPECT(convrot_quantize_rows(at(0), CONVROT_F32, 7, 3000, 3000, 4, 1.0f, at(64), nullptr) == CONVROT_EUNSUPPORTED);
    EXPECT(convrot_quantize_rows(at(0), CONVROT_F32, 7, 3072, 3071, 256, 1.0f, at(64), nullptr) == CONVROT_EINVAL);
    EXPECT(convrot_quantize_rows(at(0), CONVROT_F32, 7, 3072, 3072, 256, 0.0f, at(64), nullptr) == CONVROT_EINVAL);
    EXPECT(convrot_quantize_rows(at(0), CONVROT_F32, 7, 3072, 3072, 256, 1.0f, at(0), nullptr) == CONVROT_EOVERLAP);
    EXPECT(convrot_quantize_rows(at(0), 7, 7, 3072, 3072, 256, 1.0f, at(64), nullptr) == CONVROT_EUNSUPPORTED);
    EXPECT(convrot_quantize_rows(at(0), CONVROT_F32, 7, 131072, 131072, 256, 1.0f, at(64), nullptr) == CONVROT_EUNSUPPORTED);
    EXPECT(convrot_quantize_rows(at(0), CONVROT_F32, 0, 256, 256, 16, 1.0f, nullptr, nullptr) == CONVROT_OK);
    // rows whose byte extent does not fit an int64 are rejected, not wrapped
    EXPECT(convrot_quantize_rows(at(0), CONVROT_F32, std::numeric_limits<int64_t>::max() / 4, 65536, 65536, 256,
                                 1.0f, at(64), nullptr) == CONVROT_EINVAL);
    EXPECT(g_log.quantize_calls == 0);

    convrot_pre pre{};
    pre.kind = CONVROT_PRE_MODULATE;
    pre.scale = at_t<const float>(200);
    pre.shift = at_t<const float>(201);
    reset();
    EXPECT(convrot_quantize_rows_pre(at(0), CONVROT_BF16, 9, 3072, 3072, &pre, 256, 1.0f, at(64), nullptr) == CONVROT_OK);
    EXPECT(g_log.quantize_calls == 1 && g_log.q_pre == convrot_detail::kPreModulate);
    pre.scale = nullptr;
    EXPECT(convrot_quantize_rows_pre(at(0), CONVROT_BF16, 9, 3072, 3072, &pre, 256, 1.0f, at(64), nullptr) == CONVROT_EINVAL);
    pre.kind = CONVROT_PRE_RMSNORM_MODULATE;
    pre.eps = 1e-6f;
    pre.shift = nullptr;
    pre.norm_weight = at_t<const float>(202);
    reset();
    EXPECT(convrot_quantize_rows_pre(at(0), CONVROT_F32, 9, 3072, 3072, &pre, 256, 1.0f, at(64), nullptr) == CONVROT_OK);
    EXPECT(g_log.q_pre == convrot_detail::kPreRmsNormModulate);
    pre.eps = -1.0f;
    EXPECT(convrot_quantize_rows_pre(at(0), CONVROT_F32, 9, 3072, 3072, &pre, 256, 1.0f, at(64), nullptr) == CONVROT_EINVAL);
    convrot_pre nm{};
    nm.kind = CONVROT_PRE_NORM_MUL;
    nm.norm_weight = at_t<const float>(202);
    nm.eps = 1e-6f;
    reset();
    EXPECT(convrot_quantize_rows_pre(at(0), CONVROT_BF16, 9, 3072, 3072, &nm, 256, 1.0f, at(64), nullptr) == CONVROT_OK);
    EXPECT(g_log.q_pre == convrot_detail::kPreNormMul);
    nm.scale = at_t<const float>(200);
    EXPECT(convrot_quantize_rows_pre(at(0), CONVROT_BF16, 9, 3072, 3072, &nm, 256, 1.0f, at(64), nullptr) == CONVROT_EINVAL);
    nm.scale = nullptr;
    nm.norm_weight = at_t<const float>(64);          // packed over the weight
    EXPECT(convrot_quantize_rows_pre(at(0), CONVROT_BF16, 9, 3072, 3072, &nm, 256, 1.0f, at(64), nullptr) == CONVROT_EOVERLAP);
    convrot_pre act{};
    act.kind = CONVROT_PRE_GATED_ACT;
    act.up = at(300);
    act.ld_up = 3072;
    act.act = CONVROT_ACT_SILU;
    reset();
    EXPECT(convrot_quantize_rows_pre(at(0), CONVROT_BF16, 9, 3072, 3072, &act, 256, 1.0f, at(64), nullptr) == CONVROT_OK);
    EXPECT(g_log.q_pre == convrot_detail::kPreGatedAct);
    act.act = 9;
    EXPECT(convrot_quantize_rows_pre(at(0), CONVROT_BF16, 9, 3072, 3072, &act, 256, 1.0f, at(64), nullptr) == CONVROT_EUNSUPPORTED);
}

static void linears()
{
    reset();
    EXPECT(int8_linear(at_t<const int8_t>(0), at_t<const float>(16), 100, 3072, at_t<const int8_t>(32),
                       at_t<const float>(80), at_t<const float>(81), 300, 0.3f, at(100), CONVROT_BF16, 300,
                       nullptr) == CONVROT_OK);
    EXPECT(g_log.gemm_calls == 1 && g_log.gemm.n_lin == 1 && g_log.gemm.lin[0].alpha == 0.3f);
    EXPECT(g_log.gemm.lin[0].N == 300 && g_log.gemm.M == 100 && g_log.gemm.K == 3072);
    reset();
    EXPECT(int8_linear(at_t<const int8_t>(0), at_t<const float>(16), 100, 3072, at_t<const int8_t>(32), nullptr,
                       nullptr, 300, 1.0f, at(0), CONVROT_F32, 300, nullptr) == CONVROT_EOVERLAP);
    EXPECT(int8_linear(at_t<const int8_t>(0), at_t<const float>(16), 100, 3000, at_t<const int8_t>(32), nullptr,
                       nullptr, 300, 1.0f, at(100), CONVROT_F32, 300, nullptr) == CONVROT_EUNSUPPORTED);
    EXPECT(int8_linear(at_t<const int8_t>(0), at_t<const float>(16), 100, 133120 + 64, at_t<const int8_t>(32),
                       nullptr, nullptr, 300, 1.0f, at(100), CONVROT_F32, 300, nullptr) == CONVROT_EOVERFLOW);
    EXPECT(int8_linear(at_t<const int8_t>(0), at_t<const float>(16), 100, 3072, at_t<const int8_t>(32), nullptr,
                       nullptr, 300, 1.0f, at(100), CONVROT_F32, 299, nullptr) == CONVROT_EINVAL);
    EXPECT(int8_linear(at_t<const int8_t>(0), at_t<const float>(16), std::numeric_limits<int64_t>::max() / 2,
                       3072, at_t<const int8_t>(32), nullptr, nullptr, 300, 1.0f, at(100), CONVROT_F32, 300,
                       nullptr) == CONVROT_EINVAL);
    EXPECT(g_log.gemm_calls == 0);

    convrot_post post{};
    post.kind = CONVROT_POST_GATED_RESIDUAL;
    post.scale = 1.0f;
    post.gate = at_t<const float>(90);
    post.residual = at(100);
    post.ld_residual = 300;
    reset();
    EXPECT(int8_linear_post(at_t<const int8_t>(0), at_t<const float>(16), 100, 3072, at_t<const int8_t>(32),
                            nullptr, nullptr, 300, 1.0f, &post, at(100), CONVROT_BF16, 300, nullptr) == CONVROT_OK);
    EXPECT(g_log.gemm.lin[0].post == 1);
    post.residual = static_cast<char *>(at(100)) + 64;   // overlaps Y without being Y
    EXPECT(int8_linear_post(at_t<const int8_t>(0), at_t<const float>(16), 100, 3072, at_t<const int8_t>(32),
                            nullptr, nullptr, 300, 1.0f, &post, at(100), CONVROT_F32, 300, nullptr) == CONVROT_EOVERLAP);

    reset();
    EXPECT(int8_swiglu_linear(at_t<const int8_t>(0), at_t<const float>(16), 100, 3072, at_t<const int8_t>(32),
                              nullptr, at_t<const int8_t>(48), nullptr, 300, 1.0f, at(100), CONVROT_BF16, 300,
                              nullptr) == CONVROT_OK);
    EXPECT(g_log.gemm.lin[0].glu == 1);
    reset();
    EXPECT(int4_linear(at_t<const int8_t>(0), at_t<const float>(16), 100, 3072, at_t<const uint8_t>(32), nullptr,
                       nullptr, 300, 1.0f, at(100), CONVROT_F32, 300, nullptr) == CONVROT_OK);
    EXPECT(g_log.gemm.w_bits == 4);
    EXPECT(int4_linear(at_t<const int8_t>(0), at_t<const float>(16), 4, 132096 + 64, at_t<const uint8_t>(32),
                       nullptr, nullptr, 3, 1.0f, at(100), CONVROT_F32, 3, nullptr) == CONVROT_EOVERFLOW);
    reset();
    EXPECT(convrot_int8_gemm_i32(at_t<const int8_t>(0), at_t<const int8_t>(32), 5, 64, 7, at_t<int32_t>(100),
                                 nullptr) == CONVROT_OK);
    EXPECT(g_log.gemm.lin[0].out_kind == convrot_detail::kOutI32);
    reset();
    EXPECT(convrot_expf(at_t<const float>(0), at_t<float>(0), 1000, nullptr) == CONVROT_OK);
    EXPECT(g_log.expf_calls == 1 && g_log.last_n == 1000);
    EXPECT(convrot_expf(at_t<const float>(0), at_t<float>(0) + 1, 1000, nullptr) == CONVROT_EOVERLAP);
}

static convrot_linear_desc desc(uintptr_t w, uintptr_t y, int64_t N, float a)
{
    convrot_linear_desc d{};
    d.Qw = at_t<const int8_t>(w);
    d.N = N;
    d.input_scale = a;
    d.Y = at(y);
    d.y_dtype = CONVROT_F32;
    d.ldy = N;
    return d;
}

static void shared_and_grouped()
{
    // alpha 1, 0.5 (folded into the alpha = 1 pass) and 0.3 (its own pass)
    convrot_linear_desc d[3] = {desc(32, 200, 96, 1.0f), desc(40, 300, 64, 0.5f), desc(48, 400, 17, 0.3f)};
    const size_t ws = convrot_workspace_bytes(257, 768, 2);
    reset();
    EXPECT(convrot_int8_linear_shared(at(0), CONVROT_BF16, 257, 768, 768, 256, 3, d, at(100), ws, nullptr) == CONVROT_OK);
    EXPECT(g_log.quantize_calls == 2 && g_log.gemm_calls == 1);
    EXPECT(g_log.scales_calls == 1 && g_log.q_n == 2);   // both scales in one quantization call
    EXPECT(g_log.q_alpha == 0.3f);                       // the last pass
    // one launch: the first two linears read the alpha = 1 tensor, the third its own
    EXPECT(g_log.gemm.n_lin == 3 && g_log.gemm.lin[1].alpha == 1.0f && g_log.gemm.lin[2].alpha == 0.3f);
    EXPECT(g_log.gemm.lin[0].Qx == at_t<const int8_t>(100) && g_log.gemm.lin[1].Qx == g_log.gemm.lin[0].Qx);
    EXPECT(g_log.gemm.lin[2].Qx == at_t<const int8_t>(100) + convrot_workspace_bytes(257, 768, 1));
    EXPECT(g_log.gemm.lin[2].s_x != nullptr && g_log.gemm.lin[2].s_x != g_log.gemm.lin[0].s_x);
    convrot_linear_desc named[2] = {desc(32, 200, 96, 1.0f), desc(40, 300, 64, 1.0f)};
    named[1].Qx = at_t<const int8_t>(500);
    named[1].s_x = at_t<const float>(520);
    EXPECT(convrot_int8_linear_shared(at(0), CONVROT_BF16, 257, 768, 768, 256, 2, named, at(100), ws, nullptr) ==
           CONVROT_EINVAL);
    EXPECT(convrot_int8_linear_shared(at(0), CONVROT_BF16, 257, 768, 768, 256, 3, d, at(100), ws - 1, nullptr) ==
           CONVROT_EWORKSPACE);
    EXPECT(convrot_int8_linear_shared(at(0), CONVROT_BF16, 257, 768, 768, 256, 0, d, at(100), ws, nullptr) == CONVROT_EINVAL);
    EXPECT(convrot_int8_linear_shared(at(0), CONVROT_BF16, 257, 768, 768, 256, 17, d, at(100), ws, nullptr) == CONVROT_EINVAL);

    reset();
    EXPECT(int8_linear_grouped(at_t<const int8_t>(0), at_t<const float>(16), 257, 768, 3, d, nullptr) == CONVROT_OK);
    EXPECT(g_log.gemm_calls == 1 && g_log.gemm.n_lin == 3);
    EXPECT(g_log.gemm.lin[1].alpha == 0.5f && g_log.gemm.lin[2].alpha == 0.3f);
    convrot_linear_desc clash[2] = {desc(32, 200, 96, 1.0f), desc(40, 200, 64, 1.0f)};
    EXPECT(int8_linear_grouped(at_t<const int8_t>(0), at_t<const float>(16), 257, 768, 2, clash, nullptr) == CONVROT_EOVERLAP);
    // a linear with its own quantized input
    reset();
    EXPECT(int8_linear_grouped(at_t<const int8_t>(0), at_t<const float>(16), 257, 768, 2, named, nullptr) == CONVROT_OK);
    EXPECT(g_log.gemm_calls == 1 && g_log.gemm.n_lin == 2);
    EXPECT(g_log.gemm.lin[0].Qx == at_t<const int8_t>(0) && g_log.gemm.lin[0].s_x == at_t<const float>(16));
    EXPECT(g_log.gemm.lin[1].Qx == at_t<const int8_t>(500) && g_log.gemm.lin[1].s_x == at_t<const float>(520));
    named[1].s_x = nullptr;
    EXPECT(int8_linear_grouped(at_t<const int8_t>(0), at_t<const float>(16), 257, 768, 2, named, nullptr) == CONVROT_EINVAL);
    named[1].s_x = at_t<const float>(520);
    named[0].Y = at(500);                               // an output on the other linear's codes
    EXPECT(int8_linear_grouped(at_t<const int8_t>(0), at_t<const float>(16), 257, 768, 2, named, nullptr) == CONVROT_EOVERLAP);

    // several input scales of one X
    reset();
    const float sc[3] = {1.0f, 0.5f, 0.3f};
    const size_t pb = convrot_packed_bytes(257, 768);
    void *outs[3] = {at(100), static_cast<char *>(at(100)) + pb, at(120)};
    EXPECT(convrot_quantize_rows_scales(at(0), CONVROT_F32, 257, 768, 768, 256, 3, sc, outs, nullptr) == CONVROT_OK);
    EXPECT(g_log.scales_calls == 1 && g_log.q_n == 3 && g_log.quantize_calls == 3 && g_log.q_packed == at(120));
    EXPECT(convrot_quantize_rows_scales(at(0), CONVROT_F32, 257, 768, 768, 256, 0, sc, outs, nullptr) == CONVROT_EINVAL);
    EXPECT(convrot_quantize_rows_scales(at(0), CONVROT_F32, 257, 768, 768, 256, 3, nullptr, outs, nullptr) == CONVROT_EINVAL);
    void *overlapping[2] = {at(100), static_cast<char *>(at(100)) + pb - 16};
    EXPECT(convrot_quantize_rows_scales(at(0), CONVROT_F32, 257, 768, 768, 256, 2, sc, overlapping, nullptr) == CONVROT_EOVERLAP);
    void *on_x[1] = {at(0)};
    EXPECT(convrot_quantize_rows_scales(at(0), CONVROT_F32, 257, 768, 768, 256, 1, sc, on_x, nullptr) == CONVROT_EOVERLAP);
    const float bad[2] = {1.0f, 0.0f};
    EXPECT(convrot_quantize_rows_scales(at(0), CONVROT_F32, 257, 768, 768, 256, 2, bad, outs, nullptr) == CONVROT_EINVAL);

    reset();
    EXPECT(convrot_int8_linear_noalloc(at(0), CONVROT_BF16, 4096, 3072, 3072, 256, 1.0f, at_t<const int8_t>(32),
                                       nullptr, nullptr, 3072, at(200), CONVROT_BF16, 3072, nullptr) == CONVROT_OK);
    EXPECT(g_log.quantize_calls == 1 && g_log.gemm_calls == 1 && g_log.q_packed != nullptr);
    EXPECT(convrot_int8_linear_noalloc(at(0), CONVROT_BF16, 8192, 8192, 8192, 256, 1.0f, at_t<const int8_t>(32),
                                       nullptr, nullptr, 3072, at(300), CONVROT_BF16, 3072, nullptr) ==
           CONVROT_EWORKSPACE);
}

int main()
{
    sizes();
    quantize();
    linears();
    shared_and_grouped();
    for (int s = -7; s <= 1; ++s)
        EXPECT(convrot_status_string(s) != nullptr);
    if (failures) {
        std::fprintf(stderr, "%d expectation(s) failed\n", failures);
        return 1;
    }
    std::printf("abi ok\n");
    return 0;
}
