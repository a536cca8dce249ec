"""The RMSNorm -> Mul(weight) -> Modulate producer fused into the quantization
pass (page "ggml operator extensions", section "sd.cpp integration": the
RMSNorm -> Mul(weight) -> Mul(modulation) -> Add -> Add(shift) -> ConvRot
fusion), against the oracle's RMSNorm, Modulate and quantizer, and its linear.
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


def producer_out(orc, X, eps, w, sc, sh, K=None):
    Y = orc.rmsnorm_rows(X, eps, w, K=K, threads=THREADS)
    return Y if sc is None else orc.modulate_rows(Y, sc, sh, threads=THREADS)


def want_packed(orc, X, G, alpha, eps, w, sc, sh, K=None):
    return orc.quantize_rows(producer_out(orc, X, eps, w, sc, sh, K=K), G, alpha,
                             threads=THREADS).raw


def pre(eps, w, sc, sh):
    return cr.RMSNormModulate(eps, None if w is None else dev(w), None if sc is None else dev(sc),
                              None if sh is None else dev(sh))


# rows of 1 to 128 quads: one 64-feature block per quad span (K % 256 != 0) up
# to 128 blocks per row (K = 32768, the longest row this producer takes)
SHAPES = [(1, 64), (5, 256), (3, 320), (33, 1280), (129, 3072), (9, 4096), (7, 12288),
          (2, 32768)]


@pytest.mark.parametrize("dtype", [workloads.F32, workloads.BF16])
def test_rmsnorm_quantize_bit_exact(orc, dtype):
    rng = np.random.default_rng(61)
    for (M, K) in SHAPES:
        X = workloads.gaussian_activations(rng, M, K, 0.01, 30.0, dtype)
        w = workloads.norm_weight(rng, K)
        sc, sh = workloads.modulation(rng, K)
        G = 256 if K % 256 == 0 else 64
        for (ww, s1, s2) in ((w, sc, sh), (w, sc, None), (w, None, None), (None, None, None)):
            for eps in (1e-6, 0.5):
                say("rmsnorm quantize", M, K, G, dtype, ww is not None, s1 is not None,
                    s2 is not None, eps)
                got = host(cr.convrot_quantize_rows_pre(dev_x(X), pre(eps, ww, s1, s2), G))
                assert_bits_equal(got, want_packed(orc, X, G, 1.0, eps, ww, s1, s2),
                                  f"M={M} K={K} {dtype} w={ww is not None} sc={s1 is not None} "
                                  f"sh={s2 is not None} eps={eps}")
        for G2 in (4, 16):
            say("rmsnorm quantize G", M, K, G2, dtype)
            got = host(cr.convrot_quantize_rows_pre(dev_x(X), pre(1e-6, w, sc, sh), G2, 0.3))
            assert_bits_equal(got, want_packed(orc, X, G2, 0.3, 1e-6, w, sc, sh),
                              f"M={M} K={K} G={G2} {dtype} alpha 0.3")



def test_rmsnorm_vectors_at_lds_limit(orc):
    """With a Modulate, the RMSNorm weight is staged in LDS beside the scale
    and shift when all three fit in 48 KB: K = 4096 is the largest such row,
    K = 4160 the smallest past it."""
    rng = np.random.default_rng(62)
    for dtype in (workloads.F32, workloads.BF16):
        for K, G in ((4096, 256), (4160, 64)):
            X = workloads.gaussian_activations(rng, 6, K, 0.01, 30.0, dtype)
            w = workloads.norm_weight(rng, K)
            sc, sh = workloads.modulation(rng, K)
            for (ww, s1, s2) in ((w, sc, sh), (None, sc, sh)):
                say("rmsnorm quantize at the LDS limit", K, G, dtype, ww is not None)
                got = host(cr.convrot_quantize_rows_pre(dev_x(X), pre(1e-6, ww, s1, s2), G))
                assert_bits_equal(got, want_packed(orc, X, G, 1.0, 1e-6, ww, s1, s2),
                                  f"K={K} G={G} {dtype} w={ww is not None}")

def test_rmsnorm_special_rows(orc):
    """Zero rows (eps > 0), constant rows of +-2^k (eps = 0), magnitudes up to
    2^40 and down to 2^-40, and a single outlier."""
    K = 3072
    rng = np.random.default_rng(62)
    rows = [np.zeros(K, np.float32), np.full(K, 2.0 ** 12, np.float32),
            np.full(K, -2.0 ** -9, np.float32),
            (rng.standard_normal(K) * 2.0 ** 40).astype(np.float32),
            (rng.standard_normal(K) * 2.0 ** -40).astype(np.float32),
            np.where(np.arange(K) == 1234, 500.0, 0.0).astype(np.float32)]
    X = np.stack(rows)
    w = workloads.norm_weight(rng, K)
    for dtype_x in (X, workloads.f32_to_bf16_bits(X)):
        for eps in (1e-6, 0.0):
            if eps == 0.0:
                sel = dtype_x[1:]          # a zero row needs eps > 0
            else:
                sel = dtype_x
            say("rmsnorm special rows", sel.dtype, eps)
            got = host(cr.convrot_quantize_rows_pre(dev_x(sel), pre(eps, w, None, None), 256))
            assert_bits_equal(got, want_packed(orc, sel, 256, 1.0, eps, w, None, None),
                              f"special rows eps={eps} {sel.dtype}")


def test_rmsnorm_workload_and_stride(orc):
    """mlp_up's RMSNorm-fused pass in full, and strided rows."""
    w = workloads.WORKLOADS["mlp_up_rms"]
    inp = workloads.make_inputs(w)
    say("mlp_up_rms packed")
    got = host(cr.convrot_quantize_rows_pre(
        dev_x(inp.X), pre(w.rms_eps, inp.norm_weight, inp.mod_scale, inp.mod_shift), w.G))
    assert_bits_equal(got, want_packed(orc, inp.X, w.G, 1.0, w.rms_eps, inp.norm_weight,
                                       inp.mod_scale, inp.mod_shift), "mlp_up_rms packed")
    rng = np.random.default_rng(63)
    for dtype in (workloads.F32, workloads.BF16):
        wide = workloads.gaussian_activations(rng, 37, 3072 + 64, 0.005, 30.0, dtype)
        nw = workloads.norm_weight(rng, 3072)
        sc, sh = workloads.modulation(rng, 3072)
        say("rmsnorm ldx", dtype)
        got = host(cr.convrot_quantize_rows_pre(dev_x(wide), pre(1e-6, nw, sc, sh), 256, K=3072))
        assert_bits_equal(got, want_packed(orc, wide, 256, 1.0, 1e-6, nw, sc, sh, K=3072),
                          f"rmsnorm strided rows {dtype}")


@pytest.mark.parametrize("name", ["mlp_up_rms", "qkv"])
def test_rmsnorm_shared_linear(orc, name):
    """The fused entry with the producer: each linear's output in full
    against the oracle's RMSNorm -> Modulate -> linear."""
    w = workloads.WORKLOADS[name]
    inp = workloads.make_inputs(w)
    rng = np.random.default_rng(64)
    nw = inp.norm_weight if w.rmsnorm else workloads.norm_weight(rng, w.K)
    sc, sh = ((inp.mod_scale, inp.mod_shift) if w.modulate else workloads.modulation(rng, w.K))
    preps = [orc.weight_prep(W, w.G, threads=THREADS) for W in inp.W]
    yd = oracle.BF16 if w.y_dtype == workloads.BF16 else oracle.F32
    lins = [dict(Qw=dev(q), s_w=dev(s), bias=dev(b), input_scale=a, y_dtype=yd)
            for (q, s), b, a in zip(preps, inp.b, w.input_scales)]
    say("rmsnorm shared", name)
    outs = [host(y) for y in cr.convrot_int8_linear_shared_pre(
        dev_x(inp.X), pre(w.rms_eps, nw, sc, sh), w.G, lins)]
    Xp = producer_out(orc, inp.X, w.rms_eps, nw, sc, sh)
    for j, (y, a) in enumerate(zip(outs, w.input_scales)):
        Qw, sw = preps[j]
        want = orc.linear(Xp, w.G, Qw, sw, inp.b[j], a, yd, threads=THREADS)
        check_y(y, want, yd, f"{name} rmsnorm linear {j}")
