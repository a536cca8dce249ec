"""The gated-residual epilogue (page "ggml operator extensions", section
"sd.cpp integration": INT8 GEMM -> [Scale] -> Mul(gate) -> Add(residual))
against the oracle's reconstruction followed by its gated residual, bit for
bit (after the error gates of the linear tests)."""
import numpy as np
import pytest

import int8_hadamard_rotated_amd as cr
import oracle
import workloads
from gpu_util import THREADS, dev, dev_x, host, say
from test_gpu_linear import check_y

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def case(rng, orc, M, K, N, G=64):
    X = workloads.gaussian_activations(rng, M, K, 0.01, 30.0, workloads.F32)
    W, b = workloads.gaussian_weights(rng, N, K)
    Qw, sw = orc.weight_prep(W, G, threads=THREADS)
    p = orc.quantize_rows(X, G, threads=THREADS)
    A = orc.gemm_i32(p.q, Qw, threads=THREADS)
    gate = (rng.standard_normal(N) * 0.3).astype(np.float32)
    return p, Qw, sw, b, A, gate


@pytest.mark.parametrize("y_dtype", [oracle.F32, oracle.BF16])
def test_gated_residual_bit_exact(orc, y_dtype):
    import torch
    rng = np.random.default_rng(71)
    tdt = torch.float32 if y_dtype == oracle.F32 else torch.bfloat16
    for (M, K, N) in ((129, 192, 250), (1024 + 3, 256, 4096 + 5)):
        p, Qw, sw, b, A, gate = case(rng, orc, M, K, N)
        R = workloads.gaussian_activations(rng, M, N, 0.0, 1.0,
                                           workloads.F32 if y_dtype == oracle.F32 else workloads.BF16)
        Yf = orc.epilogue(A, p.s, sw, b, 1.0, oracle.F32, threads=THREADS)
        for scale in (1.0, 0.37):
            want = orc.gated_residual(Yf, gate, R, scale, y_dtype, threads=THREADS)
            say("gated residual", M, K, N, y_dtype, scale)
            Rd = dev_x(R) if y_dtype == oracle.BF16 else dev(R)
            Y = cr.int8_linear_post(dev(p.q), dev(p.s), dev(Qw), dev(sw), dev(b), 1.0,
                                    cr.GatedResidual(dev(gate), Rd, scale), y_dtype=y_dtype)
            check_y(host(Y), want, y_dtype, f"gated {M}x{K}x{N} scale={scale}")
            # in place: the residual is the output tensor
            say("gated residual in place", M, K, N, y_dtype, scale)
            Yi = Rd.clone()
            cr.int8_linear_post(dev(p.q), dev(p.s), dev(Qw), dev(sw), dev(b), 1.0,
                                cr.GatedResidual(dev(gate), Yi, scale), Y=Yi)
            check_y(host(Yi), want, y_dtype, f"gated in place {M}x{K}x{N} scale={scale}")


@pytest.mark.parametrize("y_dtype", [oracle.F32, oracle.BF16])
def test_gated_residual_big_grid_unscale(orc, y_dtype):
    """189 tiles of 256 x 256 (the gated-residual 256 x 256 kernel) with an
    input scale that is not a power of two (its unscale division), K = 512 so
    that the steady-state loop runs; in place on the residual."""
    rng = np.random.default_rng(73 + y_dtype)
    M, K, N = 2051, 512, 5125
    alpha = 0.3
    X = workloads.gaussian_activations(rng, M, K, 0.005, 30.0, workloads.BF16)
    W, b = workloads.gaussian_weights(rng, N, K)
    Qw, sw = orc.weight_prep(W, 256, threads=THREADS)
    p = orc.quantize_rows(X, 256, alpha, threads=THREADS)
    A = orc.gemm_i32(p.q, Qw, threads=THREADS)
    gate = (rng.standard_normal(N) * 0.3).astype(np.float32)
    R = workloads.gaussian_activations(rng, M, N, 0.0, 1.0,
                                       workloads.F32 if y_dtype == oracle.F32 else workloads.BF16)
    Yf = orc.epilogue(A, p.s, sw, b, alpha, oracle.F32, threads=THREADS)
    want = orc.gated_residual(Yf, gate, R, 0.37, y_dtype, threads=THREADS)
    Yi = dev_x(R) if y_dtype == oracle.BF16 else dev(R)
    say("gated residual big grid", M, K, N, y_dtype, alpha)
    cr.int8_linear_post(dev(p.q), dev(p.s), dev(Qw), dev(sw), dev(b), alpha,
                        cr.GatedResidual(dev(gate), Yi, 0.37), Y=Yi)
    check_y(host(Yi), want, y_dtype, f"gated big grid alpha={alpha}")


def test_gated_residual_strided(orc):
    """A residual with a row stride above N and an output with another one."""
    import torch
    rng = np.random.default_rng(72)
    M, K, N = 70, 256, 61
    p, Qw, sw, b, A, gate = case(rng, orc, M, K, N)
    Rw = rng.standard_normal((M, N + 3)).astype(np.float32)
    want = orc.gated_residual(orc.epilogue(A, p.s, sw, b), gate, np.ascontiguousarray(Rw[:, :N]))
    big = torch.full((M, 67), -7.0, dtype=torch.float32, device="cuda:0")
    say("gated strided")
    cr.int8_linear_post(dev(p.q), dev(p.s), dev(Qw), dev(sw), dev(b), 1.0,
                        cr.GatedResidual(dev(gate), dev(Rw)[:, :N]), Y=big[:, :N])
    got = host(big)
    check_y(np.ascontiguousarray(got[:, :N]), want, oracle.F32, "gated strided")
    assert np.all(got[:, N:] == -7.0), "wrote past N"


@pytest.mark.parametrize("col0,extra", [(256, 256), (64, 3)])
def test_gated_residual_concat(orc, col0, extra):
    """The chain's optional [Concat] (page "ggml operator extensions", section
    "sd.cpp integration": INT8 GEMM -> [Scale] -> Mul(gate) -> Add(residual)
    -> [Concat]): the result written straight into its slice of the
    concatenated tensor through Y and ldy, along the features (a column
    block of a wider row) and along the tokens (a row block), every other
    element left as it was.  col0 = 256 keeps 16-byte rows (vector stores),
    col0 = 64 with an odd width does not; 171 tiles of 256 x 256."""
    import torch
    rng = np.random.default_rng(75 + col0)
    M, K, N = 2051, 256, 4613
    p, Qw, sw, b, A, gate = case(rng, orc, M, K, N, G=256)
    R = workloads.gaussian_activations(rng, M, N, 0.0, 1.0, workloads.BF16)
    Yf = orc.epilogue(A, p.s, sw, b, 1.0, oracle.F32, threads=THREADS)
    want = orc.gated_residual(Yf, gate, R, 0.37, oracle.BF16, threads=THREADS)
    post = cr.GatedResidual(dev(gate), dev_x(R), 0.37)
    # along the features: [other | this | other]
    width = col0 + N + extra
    D = torch.full((M, width), 3.0, dtype=torch.bfloat16, device="cuda:0")
    say("gated concat columns", col0, width)
    cr.int8_linear_post(dev(p.q), dev(p.s), dev(Qw), dev(sw), dev(b), 1.0, post,
                        Y=D[:, col0:col0 + N])
    got = host(D)
    check_y(np.ascontiguousarray(got[:, col0:col0 + N]), want, oracle.BF16, "concat columns")
    assert np.all(got[:, :col0] == 0x4040) and np.all(got[:, col0 + N:] == 0x4040), "wrote outside its columns"
    # along the tokens: rows [r0, r0 + M) of a taller tensor
    r0 = 5
    T = torch.full((r0 + M + 2, N), 3.0, dtype=torch.bfloat16, device="cuda:0")
    say("gated concat rows", r0)
    cr.int8_linear_post(dev(p.q), dev(p.s), dev(Qw), dev(sw), dev(b), 1.0, post, Y=T[r0:r0 + M])
    got = host(T)
    check_y(np.ascontiguousarray(got[r0:r0 + M]), want, oracle.BF16, "concat rows")
    assert np.all(got[:r0] == 0x4040) and np.all(got[r0 + M:] == 0x4040), "wrote outside its rows"


def test_gated_residual_workload(orc):
    """The DiT output projection with its gated residual in place, at full
    size from a GPU-quantized packed tensor, every output compared."""
    w = workloads.WORKLOADS["proj_gated"]
    inp = workloads.make_inputs(w)
    Qw, sw = orc.weight_prep(inp.W[0], w.G, threads=THREADS)
    say("proj_gated")
    packed = cr.convrot_quantize_rows(dev_x(inp.X), w.G)
    qx, sx = cr.packed_parts(packed, w.M, w.K)
    Y = dev_x(inp.residual)
    cr.int8_linear_post(qx, sx, dev(Qw), dev(sw), dev(inp.b[0]), 1.0,
                        cr.GatedResidual(dev(inp.gate), Y), Y=Y, M=w.M)
    Yf = orc.linear(inp.X, w.G, Qw, sw, inp.b[0], 1.0, oracle.F32, threads=THREADS)
    want = orc.gated_residual(Yf, inp.gate, inp.residual, 1.0, oracle.BF16, threads=THREADS)
    check_y(host(Y), want, oracle.BF16, "proj_gated Y")
