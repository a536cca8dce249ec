"""The gated activation producer fused into the quantization pass (page
"ggml operator extensions", section "sd.cpp integration": SiLU/Sigmoid ->
Mul -> ConvRot, SwiGLU -> ConvRot with packed, swapped or separate gate/up
inputs), against the oracle's gated activation, quantizer and linear, bit for
bit; and the device build of its correctly rounded exp against the oracle's."""
import numpy as np
import pytest

import int8_hadamard_rotated_amd as cr
import oracle
import workloads
from gpu_util import THREADS, assert_bits_equal, dev, dev_x, host, say
from test_gpu_linear import check_y

pytestmark = pytest.mark.gpu

ACTS = {"silu": (cr.ACT_SILU, oracle.ACT_SILU), "sigmoid": (cr.ACT_SIGMOID, oracle.ACT_SIGMOID)}


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def test_device_expf(orc):
    """2^24 random binary32 arguments over exp's finite range and beyond, plus
    the range ends, zeros and subnormals: device exp == oracle exp, bit for bit."""
    import torch
    rng = np.random.default_rng(81)
    bits = rng.integers(0, 2 ** 32, size=1 << 24, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = np.where(np.isfinite(x), x, np.float32(1.0)).astype(np.float32)
    x = np.clip(x, -200.0, 200.0).astype(np.float32)
    special = np.array([0.0, -0.0, 89.0, -104.0, 88.72283, 88.72284, -103.97208, -103.97207,
                        1e-45, -1e-45, 1.0, -1.0, 0.5], np.float32)
    x[: special.size] = special
    say("device expf", x.size)
    got = host(cr.convrot_expf(dev(x)))
    want = orc.expf_array(x, threads=THREADS)
    assert_bits_equal(got, want, "device expf")
    say("device expf in place")
    xd = dev(x[:4096])
    cr.convrot_expf(xd, xd)
    assert_bits_equal(host(xd), want[:4096], "device expf in place")


def want_packed(orc, G, U, act, Gsz, alpha=1.0, K=None):
    z = orc.gated_act_rows(G, U, act, K=K, threads=THREADS)
    return orc.quantize_rows(z, Gsz, alpha, threads=THREADS).raw


SHAPES = [(1, 64), (5, 256), (3, 320), (33, 1280), (129, 3072), (7, 12288), (2, 32768)]


@pytest.mark.parametrize("act", sorted(ACTS))
@pytest.mark.parametrize("dtype", [workloads.F32, workloads.BF16])
def test_gated_quantize_bit_exact(orc, act, dtype):
    ca, oa = ACTS[act]
    rng = np.random.default_rng(82)
    for (M, K) in SHAPES:
        G = workloads.gaussian_activations(rng, M, K, 0.01, 30.0, dtype)
        U = workloads.gaussian_activations(rng, M, K, 0.01, 30.0, dtype)
        Gsz = 256 if K % 256 == 0 else 64
        say("gated quantize", act, M, K, dtype)
        got = host(cr.convrot_quantize_rows_pre(dev_x(G), cr.GatedAct(dev_x(U), ca), Gsz))
        assert_bits_equal(got, want_packed(orc, G, U, oa, Gsz), f"{act} M={M} K={K} {dtype}")
        say("gated quantize G=16 alpha 0.3", act, M, K, dtype)
        got = host(cr.convrot_quantize_rows_pre(dev_x(G), cr.GatedAct(dev_x(U), ca), 16, 0.3))
        assert_bits_equal(got, want_packed(orc, G, U, oa, 16, 0.3), f"{act} M={M} K={K} G=16")


@pytest.mark.parametrize("act", sorted(ACTS))
def test_gated_packed_and_swapped(orc, act):
    """A packed [gate | up] tensor and the swapped [up | gate] one, read as views
    of one allocation (row stride 2K): both equal the separate inputs."""
    ca, oa = ACTS[act]
    rng = np.random.default_rng(83)
    M, K = 70, 3072
    G = workloads.gaussian_activations(rng, M, K, 0.005, 30.0, workloads.BF16)
    U = workloads.gaussian_activations(rng, M, K, 0.005, 30.0, workloads.BF16)
    want = want_packed(orc, G, U, oa, 256)
    for name, both in (("packed", np.concatenate([G, U], axis=1)), ("swapped", np.concatenate([U, G], axis=1))):
        d = dev_x(both)
        g, u = (d[:, :K], d[:, K:]) if name == "packed" else (d[:, K:], d[:, :K])
        say("gated", act, name)
        got = host(cr.convrot_quantize_rows_pre(g, cr.GatedAct(u, ca), 256, K=K))
        assert_bits_equal(got, want, f"{act} {name}")


def test_gated_special_values(orc):
    """Gates at the ends of exp's range and beyond, zeros, signed zeros in up."""
    K = 256
    g = np.concatenate([np.linspace(-150.0, 150.0, K - 8, dtype=np.float32),
                        np.array([0.0, -0.0, 17.0, -17.0, 88.9, -103.9, 1e-30, -1e-30], np.float32)])
    G = np.stack([g, -g, np.zeros(K, np.float32)]).astype(np.float32)
    U = np.stack([np.ones(K, np.float32), -np.ones(K, np.float32), np.ones(K, np.float32)])
    for act in sorted(ACTS):
        ca, oa = ACTS[act]
        say("gated special", act)
        got = host(cr.convrot_quantize_rows_pre(dev_x(G), cr.GatedAct(dev_x(U), ca), 16))
        assert_bits_equal(got, want_packed(orc, G, U, oa, 16), f"{act} special values")


def test_gated_workload(orc):
    """mlp_down_glu's fused pass in full, and its linear through the shared
    entry in full."""
    w = workloads.WORKLOADS["mlp_down_glu"]
    inp = workloads.make_inputs(w)
    say("mlp_down_glu packed")
    Gd, Ud = dev_x(inp.X), dev_x(inp.up)
    got = host(cr.convrot_quantize_rows_pre(Gd, cr.GatedAct(Ud, cr.ACT_SILU), w.G))
    assert_bits_equal(got, want_packed(orc, inp.X, inp.up, oracle.ACT_SILU, w.G), "mlp_down_glu packed")
    Qw, sw = orc.weight_prep(inp.W[0], w.G, threads=THREADS)
    say("mlp_down_glu linear")
    Y = host(cr.convrot_int8_linear_shared_pre(Gd, cr.GatedAct(Ud, cr.ACT_SILU), w.G,
                                               [dict(Qw=dev(Qw), s_w=dev(sw), bias=dev(inp.b[0]),
                                                     y_dtype=oracle.BF16)])[0])
    z = orc.gated_act_rows(inp.X, inp.up, oracle.ACT_SILU, threads=THREADS)
    want = orc.linear(z, w.G, Qw, sw, inp.b[0], 1.0, oracle.BF16, threads=THREADS)
    check_y(Y, want, oracle.BF16, "mlp_down_glu Y")
