"""convrot_w4a4 linears (packed 4-bit weights, page "INT8 Convrot Safetensors",
section "Packed INT4 convrot") against the oracle's decoding followed by its
contraction and reconstruction: the int32 accumulator and the outputs bit for
bit (after the error gates of the INT8 linear tests)."""
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


SHAPES = [(1, 64, 1), (3, 128, 17), (129, 192, 250), (257, 3072, 300), (64, 12288, 96),
          (4096 + 13, 128, 4096 + 7), (1024, 3072, 3072)]


@pytest.mark.parametrize("M,K,N", SHAPES)
def test_int4_gemm_i32_bit_exact(orc, M, K, N):
    rng = np.random.default_rng(M + 3 * K + N)
    Qx = workloads.random_codes(rng, (M, K))
    W4 = workloads.random_int4_packed(rng, N, K)
    say("int4 gemm_i32", M, K, N)
    A = host(cr.convrot_int4_gemm_i32(dev(Qx), dev(W4)))
    assert_bits_equal(A, orc.gemm_i32(Qx, orc.unpack_int4(W4, K), threads=THREADS),
                      f"A {M}x{K}x{N}")


def test_int4_gemm_i32_extreme_k(orc):
    """The largest K allowed for 4-bit weights, at the extreme codes and weights."""
    K = 132096
    Qx = np.full((4, K), 127, np.int8)
    Qx[1] = -127
    W4 = np.full((40, K // 2), 0x88, np.uint8)        # every weight -8
    W4[3::2] = 0x77                                    # every weight 7
    say("int4 gemm_i32 max K")
    A = host(cr.convrot_int4_gemm_i32(dev(Qx), dev(W4)))
    want = orc.gemm_i32(Qx, orc.unpack_int4(W4, K), threads=THREADS)
    assert abs(int(want[0, 0])) == K * 127 * 8
    assert_bits_equal(A, want, "A at max K")


@pytest.mark.parametrize("y_dtype", [oracle.F32, oracle.BF16])
def test_int4_linear_bit_exact(orc, y_dtype):
    rng = np.random.default_rng(61)
    for (M, K, N) in ((129, 192, 250), (1024 + 3, 256, 4096 + 5)):
        X = workloads.gaussian_activations(rng, M, K, 0.01, 30.0, workloads.F32)
        W4 = workloads.random_int4_packed(rng, N, K)
        sw = workloads.random_scales(rng, N, 1e-3, 1e-2)
        b = (rng.standard_normal(N) * 0.1).astype(np.float32)
        Qw = orc.unpack_int4(W4, K)
        for alpha in (1.0, 0.3):
            p = orc.quantize_rows(X, 64, alpha, threads=THREADS)
            A = orc.gemm_i32(p.q, Qw, threads=THREADS)
            for use_sw, use_b in ((True, True), (False, False)):
                say("int4_linear", M, K, N, y_dtype, alpha, use_sw, use_b)
                want = orc.epilogue(A, p.s, sw if use_sw else None, b if use_b else None, alpha,
                                    y_dtype, threads=THREADS)
                Y = cr.int4_linear(dev(p.q), dev(p.s), dev(W4), dev(sw) if use_sw else None,
                                   dev(b) if use_b else None, alpha, y_dtype=y_dtype)
                check_y(host(Y), want, y_dtype, f"Y {M}x{K}x{N} a={alpha} sw={use_sw} b={use_b}")


@pytest.mark.parametrize("y_dtype", [oracle.F32, oracle.BF16])
def test_int4_linear_big_grid_unscale(orc, y_dtype):
    """189 tiles of 256 x 256 (the 4-bit 256 x 256 kernel) with an input scale
    that is not a power of two (its unscale division); K = 512 is 8 steps, so
    the 5-stage ring's steady-state loop runs."""
    rng = np.random.default_rng(63 + y_dtype)
    M, K, N = 2051, 512, 5125
    alpha = 0.3
    X = workloads.gaussian_activations(rng, M, K, 0.005, 30.0, workloads.BF16)
    W4 = workloads.random_int4_packed(rng, N, K)
    sw = workloads.random_scales(rng, N, 1e-3, 1e-2)
    b = (rng.standard_normal(N) * 0.1).astype(np.float32)
    p = orc.quantize_rows(X, 256, alpha, threads=THREADS)
    A = orc.gemm_i32(p.q, orc.unpack_int4(W4, K), threads=THREADS)
    want = orc.epilogue(A, p.s, sw, b, alpha, y_dtype, threads=THREADS)
    say("int4_linear big grid", M, K, N, y_dtype, alpha)
    Y = cr.int4_linear(dev(p.q), dev(p.s), dev(W4), dev(sw), dev(b), alpha, y_dtype=y_dtype)
    check_y(host(Y), want, y_dtype, f"int4 big grid alpha={alpha}")


def test_int4_workload_shares_packed_input(orc):
    """mlp_up with 4-bit weights at full size, from a packed tensor quantized on
    the GPU (the same packed tensor an INT8 linear would read), every output
    compared."""
    w = workloads.WORKLOADS["mlp_up_w4"]
    inp = workloads.make_inputs(w)
    say("mlp_up_w4")
    packed = cr.convrot_quantize_rows(dev_x(inp.X), w.G)
    qx, sx = cr.packed_parts(packed, w.M, w.K)
    Y = host(cr.int4_linear(qx, sx, dev(inp.W[0]), dev(inp.s_w[0]), dev(inp.b[0]),
                            y_dtype=oracle.BF16, M=w.M))
    want = orc.linear(inp.X, w.G, orc.unpack_int4(inp.W[0], w.K), inp.s_w[0], inp.b[0], 1.0,
                      oracle.BF16, threads=THREADS)
    check_y(Y, want, oracle.BF16, "mlp_up_w4 Y")
