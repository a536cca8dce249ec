"""The Norm -> Mul(weight) producer fused into the quantization pass (page
"ggml operator extensions", section "sd.cpp integration": the Norm -> Mul ->
ConvRot fusion), against the oracle's Norm and quantizer, and its linear.
Packed bytes are compared bit for bit; outputs bit for bit (after the error
gate of the linear tests)."""
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


def want_packed(orc, X, G, alpha, eps, w, K=None):
    Y = orc.norm_rows(X, eps, w, K=K, threads=THREADS)
    return orc.quantize_rows(Y, G, alpha, threads=THREADS).raw


def pre(eps, w):
    return cr.NormMul(eps, None if w is None else dev(w))


def offset_rows(rng, M, K, dtype, spread=3.0):
    """Gaussian rows with outliers, each shifted by its own mean drawn from
    N(0, spread), so that centring changes every value."""
    X = workloads.gaussian_activations(rng, M, K, 0.01, 30.0, workloads.F32)
    X = (X + (rng.standard_normal((M, 1)) * spread).astype(np.float32)).astype(np.float32)
    return workloads.f32_to_bf16_bits(X) if dtype == workloads.BF16 else X


# rows of 1 to 128 quads: one 64-feature block per quad span (K % 256 != 0) up
# to 128 blocks per row (K = 32768, the longest row this producer takes)
SHAPES = [(1, 64), (5, 256), (3, 320), (33, 1280), (129, 3072), (9, 4096), (7, 12288),
          (2, 32768)]


@pytest.mark.parametrize("dtype", [workloads.F32, workloads.BF16])
def test_norm_quantize_bit_exact(orc, dtype):
    rng = np.random.default_rng(71)
    for (M, K) in SHAPES:
        X = offset_rows(rng, M, K, dtype)
        w = workloads.norm_weight(rng, K)
        G = 256 if K % 256 == 0 else 64
        for ww in (w, None):
            for eps in (1e-6, 0.5):
                say("norm quantize", M, K, G, dtype, ww is not None, eps)
                got = host(cr.convrot_quantize_rows_pre(dev_x(X), pre(eps, ww), G))
                assert_bits_equal(got, want_packed(orc, X, G, 1.0, eps, ww),
                                  f"M={M} K={K} {dtype} w={ww is not None} eps={eps}")
        for G2 in (4, 16):
            say("norm quantize G", M, K, G2, dtype)
            got = host(cr.convrot_quantize_rows_pre(dev_x(X), pre(1e-6, w), G2, 0.3))
            assert_bits_equal(got, want_packed(orc, X, G2, 0.3, 1e-6, w),
                              f"M={M} K={K} G={G2} {dtype} alpha 0.3")


def test_norm_special_rows(orc):
    """Rows alternating c + a and c - a (exactly +-1 after the Norm with
    eps = 0), rows with a mean 10^4 times their deviation, zero-mean pair
    rows, magnitudes 2^40 and 2^-40, a single outlier on a constant row, and
    (eps > 0 only) constant and zero rows, which normalize to zeros."""
    K = 3072
    rng = np.random.default_rng(72)
    sign = np.tile(np.array([1.0, -1.0], np.float32), K // 2)
    pair = rng.standard_normal(K).astype(np.float32)
    pair[1::2] = -pair[0::2]
    rows = [np.float32(3.0) + np.float32(0.125) * sign, np.float32(-96.0) + np.float32(2.0) * sign,
            (np.float32(1e4) + rng.standard_normal(K).astype(np.float32)).astype(np.float32),
            pair,
            (rng.standard_normal(K) * 2.0 ** 40).astype(np.float32),
            (rng.standard_normal(K) * 2.0 ** -40).astype(np.float32),
            np.where(np.arange(K) == 1234, 500.0, 2.0).astype(np.float32)]
    flat = [np.zeros(K, np.float32), np.full(K, -7.5, np.float32)]
    w = workloads.norm_weight(rng, K)
    for eps, sel in ((0.0, rows), (1e-6, rows + flat)):
        X = np.stack(sel)
        for Xs in (X, workloads.f32_to_bf16_bits(X)):
            say("norm special rows", Xs.dtype, eps)
            got = host(cr.convrot_quantize_rows_pre(dev_x(Xs), pre(eps, w), 256))
            assert_bits_equal(got, want_packed(orc, Xs, 256, 1.0, eps, w),
                              f"special rows eps={eps} {Xs.dtype}")


def test_norm_workload_and_stride(orc):
    """mlp_up's Norm-fused pass in full, and strided rows."""
    w = workloads.WORKLOADS["mlp_up_norm"]
    inp = workloads.make_inputs(w)
    say("mlp_up_norm packed")
    got = host(cr.convrot_quantize_rows_pre(dev_x(inp.X), pre(w.rms_eps, inp.norm_weight), w.G))
    assert_bits_equal(got, want_packed(orc, inp.X, w.G, 1.0, w.rms_eps, inp.norm_weight),
                      "mlp_up_norm packed")
    rng = np.random.default_rng(73)
    for dtype in (workloads.F32, workloads.BF16):
        wide = offset_rows(rng, 37, 3072 + 64, dtype)
        nw = workloads.norm_weight(rng, 3072)
        say("norm ldx", dtype)
        got = host(cr.convrot_quantize_rows_pre(dev_x(wide), pre(1e-6, nw), 256, K=3072))
        assert_bits_equal(got, want_packed(orc, wide, 256, 1.0, 1e-6, nw, K=3072),
                          f"norm strided rows {dtype}")


@pytest.mark.parametrize("name", ["mlp_up_norm", "qkv"])
def test_norm_shared_linear(orc, name):
    """The fused entry with the producer: each linear's output in full
    against the oracle's Norm -> linear."""
    w = workloads.WORKLOADS[name]
    inp = workloads.make_inputs(w)
    rng = np.random.default_rng(74)
    nw = inp.norm_weight if w.norm else workloads.norm_weight(rng, w.K)
    preps = [orc.weight_prep(W, w.G, threads=THREADS) for W in inp.W]
    yd = oracle.BF16 if w.y_dtype == workloads.BF16 else oracle.F32
    lins = [dict(Qw=dev(q), s_w=dev(s), bias=dev(b), input_scale=a, y_dtype=yd)
            for (q, s), b, a in zip(preps, inp.b, w.input_scales)]
    say("norm shared", name)
    outs = [host(y) for y in cr.convrot_int8_linear_shared_pre(dev_x(inp.X), pre(w.rms_eps, nw), w.G,
                                                               lins)]
    Xp = orc.norm_rows(inp.X, w.rms_eps, nw, threads=THREADS)
    for j, (y, a) in enumerate(zip(outs, w.input_scales)):
        Qw, sw = preps[j]
        want = orc.linear(Xp, w.G, Qw, sw, inp.b[j], a, yd, threads=THREADS)
        check_y(y, want, yd, f"{name} norm linear {j}")
