"""The Modulate producer fused into the quantization pass, against the
oracle's Modulate followed by its quantizer and its linear (page "ggml
operator extensions", section "sd.cpp integration": Modulate, and its fusion
with ConvRot).  Packed bytes are compared bit for bit; outputs bit for bit
(after the error gate of the linear tests)."""
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


def want_packed(orc, X, G, alpha, sc, sh, K=None):
    return orc.quantize_rows(orc.modulate_rows(X, sc, sh, K=K, threads=THREADS), G, alpha,
                             threads=THREADS).raw


SHAPES = [(1, 64), (5, 256), (3, 320), (129, 3072), (9, 4096), (7, 12288)]


@pytest.mark.parametrize("dtype", [workloads.F32, workloads.BF16])
def test_modulated_quantize_bit_exact(orc, dtype):
    rng = np.random.default_rng(51)
    for (M, K) in SHAPES:
        X = workloads.gaussian_activations(rng, M, K, 0.01, 30.0, dtype)
        sc, sh = workloads.modulation(rng, K)
        for G in (4, 16, 64, 256):
            if K % G:
                continue
            for shift in (sh, None):
                for alpha in (1.0, 0.3):
                    say("modulated quantize", M, K, G, dtype, shift is not None, alpha)
                    got = host(cr.convrot_quantize_rows_pre(
                        dev_x(X), cr.Modulate(dev(sc), None if shift is None else dev(shift)),
                        G, alpha))
                    assert_bits_equal(got, want_packed(orc, X, G, alpha, sc, shift),
                                      f"M={M} K={K} G={G} {dtype} shift={shift is not None} a={alpha}")



def test_modulated_vectors_at_lds_limit(orc):
    """The workgroup quantizer stages the Modulate scale and shift in LDS when
    both fit in 48 KB: K = 6144 is the largest such row (both paths of the
    launch rule meet there), K = 6208 the smallest row past it.  Six rows, so
    that the last workgroup also holds pad rows."""
    rng = np.random.default_rng(54)
    for dtype in (workloads.F32, workloads.BF16):
        for K, G in ((6144, 256), (6208, 64)):
            X = workloads.gaussian_activations(rng, 6, K, 0.01, 30.0, dtype)
            sc, sh = workloads.modulation(rng, K)
            for shift in (sh, None):
                say("modulated quantize at the LDS limit", K, G, dtype, shift is not None)
                got = host(cr.convrot_quantize_rows_pre(
                    dev_x(X), cr.Modulate(dev(sc), None if shift is None else dev(shift)), G))
                assert_bits_equal(got, want_packed(orc, X, G, 1.0, sc, shift),
                                  f"K={K} G={G} {dtype} shift={shift is not None}")

def test_modulated_quantize_workload_and_stride(orc):
    """mlp_up's producer-fused pass in full, and strided rows."""
    w = workloads.WORKLOADS["mlp_up_mod"]
    inp = workloads.make_inputs(w)
    say("mlp_up_mod packed")
    got = host(cr.convrot_quantize_rows_pre(dev_x(inp.X), cr.Modulate(dev(inp.mod_scale),
                                                                      dev(inp.mod_shift)), w.G))
    assert_bits_equal(got, want_packed(orc, inp.X, w.G, 1.0, inp.mod_scale, inp.mod_shift),
                      "mlp_up_mod packed")
    rng = np.random.default_rng(52)
    for dtype in (workloads.F32, workloads.BF16):
        wide = workloads.gaussian_activations(rng, 37, 3072 + 64, 0.005, 30.0, dtype)
        sc, sh = workloads.modulation(rng, 3072)
        say("modulated ldx", dtype)
        got = host(cr.convrot_quantize_rows_pre(dev_x(wide), cr.Modulate(dev(sc), dev(sh)), 256,
                                                K=3072))
        assert_bits_equal(got, want_packed(orc, wide, 256, 1.0, sc, sh, K=3072),
                          f"modulated strided rows {dtype}")


def test_modulated_identity(orc):
    """scale = 0 and no shift give the unmodulated pass, bit for bit."""
    rng = np.random.default_rng(53)
    X = workloads.gaussian_activations(rng, 33, 3072, 0.005, 30.0, workloads.BF16)
    Xd = dev_x(X)
    say("modulate identity")
    got = host(cr.convrot_quantize_rows_pre(Xd, cr.Modulate(dev(np.zeros(3072, np.float32))), 256))
    assert_bits_equal(got, host(cr.convrot_quantize_rows(Xd, 256)), "scale 0")


@pytest.mark.parametrize("name", ["mlp_up_mod", "qkv"])
def test_modulated_shared_linear(orc, name):
    """The fused entry with the producer: each linear's output in full
    against the oracle's Modulate -> linear."""
    w = workloads.WORKLOADS[name]
    inp = workloads.make_inputs(w)
    rng = np.random.default_rng(54)
    sc, sh = ((inp.mod_scale, inp.mod_shift) if w.modulate else workloads.modulation(rng, w.K))
    preps = [orc.weight_prep(W, w.G, threads=THREADS) for W in inp.W]
    yd = oracle.BF16 if w.y_dtype == workloads.BF16 else oracle.F32
    lins = [dict(Qw=dev(q), s_w=dev(s), bias=dev(b), input_scale=a, y_dtype=yd)
            for (q, s), b, a in zip(preps, inp.b, w.input_scales)]
    say("modulated shared", name)
    outs = [host(y) for y in cr.convrot_int8_linear_shared_pre(
        dev_x(inp.X), cr.Modulate(dev(sc), dev(sh)), w.G, lins)]
    Xm = orc.modulate_rows(inp.X, sc, sh, threads=THREADS)
    for j, (y, a) in enumerate(zip(outs, w.input_scales)):
        Qw, sw = preps[j]
        want = orc.linear(Xm, w.G, Qw, sw, inp.b[j], a, yd, threads=THREADS)
        check_y(y, want, yd, f"{name} modulated linear {j}")
