"""The dual GEMM with its SwiGLU epilogue on one packed input (page "ggml
operator extensions", section "sd.cpp integration": GEMM -> SwiGLU
[-> ConvRot], gate and up weights in separate allocations, no bias), against
the oracle's two contractions, two reconstructions and its gated activation,
bit for bit (after the error gates of the linear tests)."""
import numpy as np
import pytest

import int8_hadamard_rotated_amd as cr
import oracle
import workloads
from gpu_util import THREADS, assert_bits_equal, dev, dev_x, host, say
from test_gpu_linear import check_y

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def want_swiglu(orc, A_g, A_u, s_x, sw_g, sw_u, alpha, y_dtype):
    g = orc.epilogue(A_g, s_x, sw_g, None, alpha, oracle.F32, threads=THREADS)
    u = orc.epilogue(A_u, s_x, sw_u, None, alpha, oracle.F32, threads=THREADS)
    z = orc.gated_act_rows(g, u, oracle.ACT_SILU, threads=THREADS)
    return z if y_dtype == oracle.F32 else workloads.f32_to_bf16_bits(z)


# 128 x 128 tiles (64 gate + 64 up columns) and 256 x 256 tiles, ragged M and N
SHAPES = [(1, 64, 1), (3, 128, 17), (129, 192, 250), (257, 3072, 300), (1024 + 3, 256, 2048 + 5),
          (4096 + 13, 128, 2048 + 7)]


@pytest.mark.parametrize("y_dtype", [oracle.F32, oracle.BF16])
@pytest.mark.parametrize("M,K,N", SHAPES)
def test_swiglu_bit_exact(orc, y_dtype, M, K, N):
    rng = np.random.default_rng(M + 7 * K + N)
    X = workloads.gaussian_activations(rng, M, K, 0.01, 30.0, workloads.F32)
    Wg, _ = workloads.gaussian_weights(rng, N, K)
    Wu, _ = workloads.gaussian_weights(rng, N, K)
    G = 64
    Qg, sg = orc.weight_prep(Wg, G, threads=THREADS)
    Qu, su = orc.weight_prep(Wu, G, threads=THREADS)
    for alpha in (1.0, 0.3):
        p = orc.quantize_rows(X, G, alpha, threads=THREADS)
        A_g = orc.gemm_i32(p.q, Qg, threads=THREADS)
        A_u = orc.gemm_i32(p.q, Qu, threads=THREADS)
        d = [dev(v) for v in (p.q, p.s, Qg, sg, Qu, su)]
        for use_sw in (True, False):
            say("swiglu", M, K, N, y_dtype, alpha, use_sw)
            want = want_swiglu(orc, A_g, A_u, p.s, sg if use_sw else None, su if use_sw else None,
                               alpha, y_dtype)
            Y = cr.int8_swiglu_linear(d[0], d[1], d[2], d[3] if use_sw else None, d[4],
                                      d[5] if use_sw else None, alpha, y_dtype=y_dtype)
            check_y(host(Y), want, y_dtype, f"swiglu {M}x{K}x{N} a={alpha} sw={use_sw}")


@pytest.mark.parametrize("y_dtype", [oracle.F32, oracle.BF16])
def test_swiglu_big_grid_unscale(orc, y_dtype):
    """2051 rows into 2 x 2567 columns is 9 x 21 = 189 tiles of 256 x 256 (the
    SwiGLU 256 x 256 kernel), with an input scale that is not a power of two
    (its unscale division) and K = 512 (8 steps: the steady-state loop runs)."""
    rng = np.random.default_rng(93 + y_dtype)
    M, K, N = 2051, 512, 2567
    alpha = 0.3
    X = workloads.gaussian_activations(rng, M, K, 0.005, 30.0, workloads.BF16)
    Wg, _ = workloads.gaussian_weights(rng, N, K)
    Wu, _ = workloads.gaussian_weights(rng, N, K)
    Qg, sg = orc.weight_prep(Wg, 256, threads=THREADS)
    Qu, su = orc.weight_prep(Wu, 256, threads=THREADS)
    p = orc.quantize_rows(X, 256, alpha, threads=THREADS)
    want = want_swiglu(orc, orc.gemm_i32(p.q, Qg, threads=THREADS), orc.gemm_i32(p.q, Qu, threads=THREADS),
                       p.s, sg, su, alpha, y_dtype)
    say("swiglu big grid", M, K, N, y_dtype, alpha)
    Y = cr.int8_swiglu_linear(dev(p.q), dev(p.s), dev(Qg), dev(sg), dev(Qu), dev(su), alpha,
                              y_dtype=y_dtype)
    check_y(host(Y), want, y_dtype, f"swiglu big grid alpha={alpha}")


def test_swiglu_strided_output(orc):
    """ldy > N, and an output whose rows do not allow vector stores."""
    import torch
    rng = np.random.default_rng(91)
    M, K, N = 70, 256, 61
    Qx = workloads.random_codes(rng, (M, K))
    Qg = workloads.random_codes(rng, (N, K))
    Qu = workloads.random_codes(rng, (N, K))
    sx = workloads.random_scales(rng, M)
    sg, su = workloads.random_scales(rng, N), workloads.random_scales(rng, N)
    want = want_swiglu(orc, orc.gemm_i32(Qx, Qg), orc.gemm_i32(Qx, Qu), sx, sg, su, 1.0, oracle.F32)
    for ld in (N, 64, 67):
        big = torch.full((M, ld), -7.0, dtype=torch.float32, device="cuda:0")
        say("swiglu strided", ld)
        cr.int8_swiglu_linear(dev(Qx), dev(sx), dev(Qg), dev(sg), dev(Qu), dev(su), Y=big[:, :N])
        got = host(big)
        assert_bits_equal(np.ascontiguousarray(got[:, :N]), want, f"swiglu ldy={ld}")
        assert np.all(got[:, N:] == -7.0), "wrote past N"


def test_swiglu_workload_then_convrot(orc):
    """mlp_up_swiglu at full size from a GPU-quantized packed tensor, every
    output compared, then the optional ConvRot of its output (the next
    linear's input)."""
    w = workloads.WORKLOADS["mlp_up_swiglu"]
    inp = workloads.make_inputs(w)
    (Qg, sg), (Qu, su) = [orc.weight_prep(W, w.G, threads=THREADS) for W in inp.W]
    say("mlp_up_swiglu")
    packed = cr.convrot_quantize_rows(dev_x(inp.X), w.G)
    qx, sx = cr.packed_parts(packed, w.M, w.K)
    Y = cr.int8_swiglu_linear(qx, sx, dev(Qg), dev(sg), dev(Qu), dev(su), y_dtype=oracle.BF16, M=w.M)
    p = orc.quantize_rows(inp.X, w.G, threads=THREADS)
    want = want_swiglu(orc, orc.gemm_i32(p.q, Qg, threads=THREADS), orc.gemm_i32(p.q, Qu, threads=THREADS),
                       p.s, sg, su, 1.0, oracle.BF16)
    check_y(host(Y), want, oracle.BF16, "mlp_up_swiglu Y")
    say("mlp_up_swiglu convrot of the output")
    got = host(cr.convrot_quantize_rows(Y, w.G))
    assert_bits_equal(got, orc.quantize_rows(want, w.G, threads=THREADS).raw, "convrot of the SwiGLU output")
