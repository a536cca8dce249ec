"""GPU contraction and reconstruction against the CPU oracle.

The int32 accumulator must match bit for bit; Y is checked bit for bit as well
(the gate the task sets is a max relative error of 1e-5 for fp32 and 1e-2 for
bf16 outputs; the reported error is printed and asserted against that gate,
then exactness is asserted on top)."""
import numpy as np
import pytest

import int8_hadamard_rotated_amd as cr
import oracle
import workloads
from gpu_util import THREADS, assert_bits_equal, bf16_to_f32, dev, dev_x, host, max_rel_err, say

pytestmark = pytest.mark.gpu

F32_GATE, BF16_GATE = 1e-5, 1e-2


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def check_y(got, want, y_dtype, what):
    if y_dtype == oracle.BF16:
        err = max_rel_err(bf16_to_f32(got), bf16_to_f32(want))
        assert err <= BF16_GATE, f"{what}: max rel err {err}"
    else:
        err = max_rel_err(got, want)
        assert err <= F32_GATE, f"{what}: max rel err {err}"
    assert_bits_equal(got, want, what)


# Beyond the small and ragged shapes: (4096 + 13) x 3072 x (4096 + 7) is a
# grid of 289 tiles of 256 x 256 whose 48 K steps run the peeled steady-state
# loop with an int32 output, ragged in M and N.
GEMM_SHAPES = [(1, 64, 1), (3, 128, 17), (129, 192, 250), (257, 3072, 300), (64, 12288, 96),
               (4096 + 13, 128, 4096 + 7), (4096 + 13, 3072, 4096 + 7)]


@pytest.mark.parametrize("M,K,N", GEMM_SHAPES)
def test_gemm_i32_bit_exact(orc, M, K, N):
    rng = np.random.default_rng(M + K + N)
    Qx = workloads.random_codes(rng, (M, K))
    Qw = workloads.random_codes(rng, (N, K))
    say("gemm_i32", M, K, N)
    A = host(cr.convrot_int8_gemm_i32(dev(Qx), dev(Qw)))
    assert_bits_equal(A, orc.gemm_i32(Qx, Qw, threads=THREADS), f"A {M}x{K}x{N}")


# The contraction at the full size of each workload, in the tile configuration
# its linear runs (256 x 256 tiles, steady-state loop over every K step);
# uniform codes over [-127, 127] give larger sums than quantized activations.
FULL_GEMMS = {"mlp_up": (4096, 3072, 12288), "qkv": (4096, 3072, 3072),
              "attn": (1024, 3072, 3072), "mlp_down": (16384, 12288, 3072)}


@pytest.mark.parametrize("name", sorted(FULL_GEMMS))
def test_gemm_i32_full_size(orc, name):
    M, K, N = FULL_GEMMS[name]
    rng = np.random.default_rng(K + N + 11)
    Qx = workloads.random_codes(rng, (M, K))
    Qw = workloads.random_codes(rng, (N, K))
    say("gemm_i32 full size", name, M, K, N)
    A = host(cr.convrot_int8_gemm_i32(dev(Qx), dev(Qw)))
    assert_bits_equal(A, orc.gemm_i32(Qx, Qw, threads=THREADS), f"A {name} {M}x{K}x{N}")


def test_gemm_i32_extreme_k(orc):
    """The largest K with an exact int32 result, at the extreme codes."""
    K = 133120
    Qx = np.full((4, K), 127, np.int8)
    Qx[1] = -127
    Qw = np.full((70, K), 127, np.int8)
    Qw[3::2] = -127
    say("gemm_i32 max K")
    A = host(cr.convrot_int8_gemm_i32(dev(Qx), dev(Qw)))
    want = orc.gemm_i32(Qx, Qw, threads=THREADS)
    assert abs(int(want[0, 0])) == K * 127 * 127
    assert_bits_equal(A, want, "A at max K")


@pytest.mark.parametrize("y_dtype", [oracle.F32, oracle.BF16])
@pytest.mark.parametrize("M,K,N", [(129, 192, 250), (1024 + 3, 256, 4096 + 5)])
def test_int8_linear_bit_exact(orc, y_dtype, M, K, N):
    rng = np.random.default_rng(3 * M + N)
    X = workloads.gaussian_activations(rng, M, K, 0.01, 30.0, workloads.F32)
    W, b = workloads.gaussian_weights(rng, N, K)
    G = 64
    Qw, sw = orc.weight_prep(W, G, threads=THREADS)
    for alpha in (1.0, 0.5, 0.3):
        p = orc.quantize_rows(X, G, alpha, threads=THREADS)
        A = orc.gemm_i32(p.q, Qw, threads=THREADS)
        Qx_d, sx_d, Qw_d, sw_d, b_d = dev(p.q), dev(p.s), dev(Qw), dev(sw), dev(b)
        for use_sw, use_b in ((True, True), (False, True), (True, False), (False, False)):
            say("int8_linear", M, K, N, y_dtype, alpha, use_sw, use_b)
            want = orc.epilogue(A, p.s, sw if use_sw else None, b if use_b else None, alpha,
                                y_dtype, threads=THREADS)
            Y = cr.int8_linear(Qx_d, sx_d, Qw_d, sw_d if use_sw else None, b_d if use_b else None,
                               alpha, y_dtype=y_dtype)
            check_y(host(Y), want, y_dtype, f"Y {M}x{K}x{N} a={alpha} sw={use_sw} b={use_b}")


# Grids of at least 160 tiles of 256 x 256 take the 256 x 256 kernels; with an
# input scale that is not a power of two those carry the unscale division.
# 2051 x 5125 is 9 x 21 = 189 such tiles; K = 512 gives 8 steps, so the
# steady-state loop runs as well.
BIG_GRID = (2051, 512, 5125)


@pytest.mark.parametrize("alpha", [0.3, 0.5, 2.0 ** -20])
@pytest.mark.parametrize("y_dtype", [oracle.F32, oracle.BF16])
def test_int8_linear_big_grid_unscale(orc, y_dtype, alpha):
    """The 256 x 256 kernels with the unscale: a correctly rounded division
    for 0.3, a multiplication by the exact reciprocal for the powers of two."""
    M, K, N = BIG_GRID
    rng = np.random.default_rng(91 + y_dtype)
    X = workloads.gaussian_activations(rng, M, K, 0.005, 30.0, workloads.BF16)
    W, b = workloads.gaussian_weights(rng, N, K)
    Qw, sw = orc.weight_prep(W, 256, threads=THREADS)
    p = orc.quantize_rows(X, 256, alpha, threads=THREADS)
    A = orc.gemm_i32(p.q, Qw, threads=THREADS)
    want = orc.epilogue(A, p.s, sw, b, alpha, y_dtype, threads=THREADS)
    say("int8_linear big grid", M, K, N, y_dtype, alpha)
    Y = cr.int8_linear(dev(p.q), dev(p.s), dev(Qw), dev(sw), dev(b), alpha, y_dtype=y_dtype)
    check_y(host(Y), want, y_dtype, f"Y {M}x{K}x{N} alpha={alpha}")
    # and the fused entry, which quantizes with the same alpha on the GPU
    say("fused big grid", M, K, N, y_dtype, alpha)
    Yf = cr.convrot_int8_linear(dev_x(X), 256, alpha, dev(Qw), dev(sw), dev(b), y_dtype=y_dtype)
    check_y(host(Yf), want, y_dtype, f"fused Y {M}x{K}x{N} alpha={alpha}")


@pytest.mark.parametrize("M,K,Ns", [(515, 768, (130, 64, 257)), (1030, 512, (3072, 3072, 3072))])
def test_int8_linear_grouped(orc, M, K, Ns):
    """Several linears on one packed input in one launch, each with its own
    divisor, output dtype and row stride; the second shape is 180 tiles of
    256 x 256 (the 256 x 256 kernel with the division compiled in)."""
    import torch
    rng = np.random.default_rng(M + K)
    G = 256
    X = workloads.gaussian_activations(rng, M, K, 0.005, 30.0, workloads.BF16)
    p = orc.quantize_rows(X, G, threads=THREADS)
    alphas = (1.0, 0.3, 1.0)
    dtypes = (oracle.BF16, oracle.F32, oracle.F32)
    lins, wants = [], []
    for N, a, yd in zip(Ns, alphas, dtypes):
        W, b = workloads.gaussian_weights(rng, N, K)
        Qw, sw = orc.weight_prep(W, G, threads=THREADS)
        A = orc.gemm_i32(p.q, Qw, threads=THREADS)
        wants.append(orc.epilogue(A, p.s, sw, b, a, yd, threads=THREADS))
        lins.append(dict(Qw=dev(Qw), s_w=dev(sw), bias=dev(b), input_scale=a, y_dtype=yd))
    # the last output strided inside a wider buffer
    wide = torch.full((M, Ns[2] + 5), -7.0, dtype=torch.float32, device="cuda:0")
    lins[2]["Y"] = wide[:, :Ns[2]]
    say("int8_linear_grouped", M, K, Ns)
    outs = cr.int8_linear_grouped(dev(p.q), dev(p.s), lins)
    for j, (y, want, yd) in enumerate(zip(outs, wants, dtypes)):
        check_y(np.ascontiguousarray(host(y)), want, yd, f"grouped linear {j}")
    assert np.all(host(wide)[:, Ns[2]:] == -7.0), "wrote past N"


@pytest.mark.parametrize("M,K,Ns", [(515, 768, (130, 64, 257)), (1030, 512, (3072, 3072, 3072))])
def test_int8_linear_grouped_own_inputs(orc, M, K, Ns):
    """Linears of one launch reading different packed tensors: the pages'
    path for several input scales (a quantization pass per scale, the
    division by it in the reconstruction).  The second shape is 180 tiles of
    256 x 256: the kernel with the division compiled in, which its alpha = 1
    tiles skip and its alpha = 0.5 tiles replace by the exact reciprocal."""
    rng = np.random.default_rng(M + 7 * K)
    G = 256
    X = workloads.gaussian_activations(rng, M, K, 0.005, 30.0, workloads.BF16)
    alphas = (1.0, 0.3, 0.5)
    packs = {a: orc.quantize_rows(X, G, a, threads=THREADS) for a in set(alphas)}
    dpacks = {a: (dev(p.q), dev(p.s)) for a, p in packs.items()}
    lins, wants = [], []
    for N, a in zip(Ns, alphas):
        W, b = workloads.gaussian_weights(rng, N, K)
        Qw, sw = orc.weight_prep(W, G, threads=THREADS)
        A = orc.gemm_i32(packs[a].q, Qw, threads=THREADS)
        wants.append(orc.epilogue(A, packs[a].s, sw, b, a, oracle.F32, threads=THREADS))
        lin = dict(Qw=dev(Qw), s_w=dev(sw), bias=dev(b), input_scale=a, y_dtype=oracle.F32)
        if a != 1.0:
            lin["Qx"], lin["s_x"] = dpacks[a]
        lins.append(lin)
    say("int8_linear_grouped own inputs", M, K, Ns)
    qx, sx = dpacks[1.0]
    outs = cr.int8_linear_grouped(qx, sx, lins)
    for j, (y, want) in enumerate(zip(outs, wants)):
        assert_bits_equal(host(y), want, f"grouped linear {j} alpha={alphas[j]}")


GROUPED_SIXTEEN = [(300, 256, (0, 1, 17, 64, 130, 256, 257, 3, 0, 96, 33, 512, 5, 128, 200, 64)),
                   (1030, 256, (520, 600, 257, 512, 700, 1, 513, 640, 300, 768, 129, 512, 64, 900, 256,
                                500))]


@pytest.mark.parametrize("M,K,Ns", GROUPED_SIXTEEN)
def test_int8_linear_grouped_sixteen(orc, M, K, Ns):
    """Sixteen linears in one launch (the most it takes): empty, one-column
    and ragged outputs, both output dtypes, five input scales.  Even linears
    read the call's packed tensor (alpha = 1), odd ones their own.  The
    first shape runs 128 x 128 tiles; the second is 180 tiles of 256 x 256
    with the division compiled in."""
    rng = np.random.default_rng(M + 3 * K)
    G = 256
    X = workloads.gaussian_activations(rng, M, K, 0.005, 30.0, workloads.BF16)
    own = (0.3, 0.5, 2.0, 0.7)
    packs = {a: orc.quantize_rows(X, G, a, threads=THREADS) for a in (1.0, *own)}
    dpacks = {a: (dev(p.q), dev(p.s)) for a, p in packs.items()}
    lins, wants = [], []
    for j, N in enumerate(Ns):
        a = 1.0 if j % 2 == 0 else own[(j // 2) % len(own)]
        yd = oracle.BF16 if j % 3 == 0 else oracle.F32
        if N == 0:
            Qw, sw = np.zeros((0, K), np.int8), np.zeros(0, np.float32)
            b = np.zeros(0, np.float32)
            wants.append(None)
        else:
            W, b = workloads.gaussian_weights(rng, N, K)
            Qw, sw = orc.weight_prep(W, G, threads=THREADS)
            A = orc.gemm_i32(packs[a].q, Qw, threads=THREADS)
            wants.append(orc.epilogue(A, packs[a].s, sw, b, a, yd, threads=THREADS))
        lin = dict(Qw=dev(Qw), s_w=dev(sw), bias=dev(b), input_scale=a, y_dtype=yd)
        if j % 2 == 1:
            lin["Qx"], lin["s_x"] = dpacks[a]
        lins.append(lin)
    say("int8_linear_grouped sixteen", M, K, Ns)
    qx, sx = dpacks[1.0]
    outs = cr.int8_linear_grouped(qx, sx, lins)
    for j, (y, want) in enumerate(zip(outs, wants)):
        if want is None:
            assert tuple(y.shape) == (M, 0)
            continue
        check_y(host(y), want, lins[j]["y_dtype"], f"grouped linear {j} N={Ns[j]}")


@pytest.mark.parametrize("dtype", [workloads.F32, workloads.BF16])
def test_shared_sixteen_scales(orc, dtype):
    """convrot_int8_linear_shared with sixteen linears of sixteen distinct
    input scales: sixteen packed tensors in the workspace (binary32 rows two
    scales per pass, bf16 rows one), then one grouped launch over all of
    them, against the oracle's literal path."""
    import torch
    rng = np.random.default_rng(99 + (dtype == workloads.BF16))
    M, K, G = 130, 512, 64
    X = workloads.gaussian_activations(rng, M, K, 0.005, 30.0, dtype)
    scales = [0.3, 0.7, 1.0, 1.3, 0.11, 3.7, 0.9, 1.1, 0.6, 2.5, 0.45, 6.0, 0.35, 1.7, 0.15, 4.2]
    Ns = [64, 17, 130, 1, 96, 256, 33, 128, 5, 64, 200, 48, 3, 160, 80, 32]
    preps, lins = [], []
    for a, N in zip(scales, Ns):
        W, b = workloads.gaussian_weights(rng, N, K)
        Qw, sw = orc.weight_prep(W, G, threads=THREADS)
        preps.append((Qw, sw, b))
        lins.append(dict(Qw=dev(Qw), s_w=dev(sw), bias=dev(b), input_scale=a, y_dtype=oracle.F32))
    ws = torch.empty(cr.convrot_workspace_bytes(M, K, len(scales)), dtype=torch.uint8, device="cuda:0")
    say("shared sixteen scales", dtype)
    outs = [host(y) for y in cr.convrot_int8_linear_shared(dev_x(X), G, lins, workspace=ws)]
    for (Qw, sw, b), a, y in zip(preps, scales, outs):
        want = orc.linear(X, G, Qw, sw, b, a, oracle.F32, threads=THREADS)
        check_y(y, want, oracle.F32, f"alpha={a}")


def test_shared_mixed_scales_big_grid(orc):
    """convrot_int8_linear_shared with alpha = 1 and alpha = 0.3 linears: two
    quantization passes, then one grouped launch of 180 tiles of 256 x 256
    over both packed tensors (the division kernel, skipped on the alpha = 1
    tiles), against the oracle's literal path."""
    import torch
    rng = np.random.default_rng(77)
    M, K, G = 1030, 512, 256
    X = workloads.gaussian_activations(rng, M, K, 0.005, 30.0, workloads.F32)
    alphas, Ns = (1.0, 0.3, 1.0), (3072, 3072, 3072)
    preps, lins = [], []
    for a, N in zip(alphas, Ns):
        W, b = workloads.gaussian_weights(rng, N, K)
        Qw, sw = orc.weight_prep(W, G, threads=THREADS)
        preps.append((Qw, sw, b))
        lins.append(dict(Qw=dev(Qw), s_w=dev(sw), bias=dev(b), input_scale=a, y_dtype=oracle.F32))
    ws = torch.empty(cr.convrot_workspace_bytes(M, K, 2), dtype=torch.uint8, device="cuda:0")
    say("shared mixed scales", M, K, Ns)
    outs = [host(y) for y in cr.convrot_int8_linear_shared(dev_x(X), G, lins, workspace=ws)]
    for (Qw, sw, b), a, y in zip(preps, alphas, outs):
        want = orc.linear(X, G, Qw, sw, b, a, oracle.F32, threads=THREADS)
        assert_bits_equal(y, want, f"alpha={a}")


@pytest.mark.parametrize("dtype", [workloads.F32, workloads.BF16])
def test_fused_group_one(orc, dtype):
    """G = 1 (no rotation) through the fused entry, weights prepared at G = 1
    too, on a ragged shape of both tile sizes' grids, against the oracle."""
    rng = np.random.default_rng(81)
    for (M, K, N) in ((257, 512, 300), (1030, 768, 3072 + 17)):
        X = workloads.gaussian_activations(rng, M, K, 0.005, 30.0, dtype)
        W, b = workloads.gaussian_weights(rng, N, K)
        Qw, sw = orc.weight_prep(W, 1, threads=THREADS)
        for a in (1.0, 0.3):
            say("fused G=1", M, K, N, dtype, a)
            Y = host(cr.convrot_int8_linear(dev_x(X), 1, a, dev(Qw), dev(sw), dev(b)))
            want = orc.linear(X, 1, Qw, sw, b, a, threads=THREADS)
            check_y(Y, want, oracle.F32, f"G=1 M={M} N={N} {dtype} alpha={a}")


def test_int8_linear_strided_output(orc):
    """ldy > N, and an output whose rows do not allow vector stores."""
    rng = np.random.default_rng(5)
    import torch
    M, K, N = 70, 256, 61
    Qx = workloads.random_codes(rng, (M, K))
    Qw = workloads.random_codes(rng, (N, K))
    sx = workloads.random_scales(rng, M)
    sw = workloads.random_scales(rng, N)
    b = (rng.standard_normal(N) * 0.1).astype(np.float32)
    want = orc.epilogue(orc.gemm_i32(Qx, Qw), sx, sw, b)
    for ld in (N, 64, 67):
        big = torch.full((M, ld), -7.0, dtype=torch.float32, device="cuda:0")
        Y = big[:, :N]
        say("strided Y", ld)
        cr.int8_linear(dev(Qx), dev(sx), dev(Qw), dev(sw), dev(b), 1.0, Y=Y)
        got = host(big)
        assert_bits_equal(np.ascontiguousarray(got[:, :N]), want, f"Y ldy={ld}")
        assert np.all(got[:, N:] == -7.0), "wrote past N"


@pytest.mark.parametrize("name", ["tiny", "attn", "mlp_up", "mlp_down"])
def test_fused_workload(orc, name):
    """The fused entry at each workload's full size, in the configuration the
    benchmark runs; every output compared with the oracle."""
    w = workloads.WORKLOADS[name]
    inp = workloads.make_inputs(w)
    Qw, sw = orc.weight_prep(inp.W[0], w.G, threads=THREADS)
    yd = oracle.BF16 if w.y_dtype == workloads.BF16 else oracle.F32
    say("fused", name)
    Y = host(cr.convrot_int8_linear(dev_x(inp.X), w.G, 1.0, dev(Qw), dev(sw), dev(inp.b[0]),
                                    y_dtype=yd))
    want = orc.linear(inp.X, w.G, Qw, sw, inp.b[0], 1.0, yd, threads=THREADS)
    check_y(Y, want, yd, f"{name} Y")


def test_shared_qkv(orc):
    """Three linears sharing one packed input plus one at input scale 0.5:
    each output against the oracle, against separate fused calls, and the
    0.5 linear against the same weights at scale 1 (bit-identical, since
    multiplying by 2^-1 before the rotation and dividing after are exact)."""
    w = workloads.WORKLOADS["qkv"]
    inp = workloads.make_inputs(w)
    Xd = dev_x(inp.X)
    preps = [orc.weight_prep(W, w.G, threads=THREADS) for W in inp.W]
    lins = [dict(Qw=dev(q), s_w=dev(s), bias=dev(b), input_scale=a)
            for (q, s), b, a in zip(preps, inp.b, w.input_scales)]
    say("shared qkv")
    outs = [host(y) for y in cr.convrot_int8_linear_shared(Xd, w.G, lins)]
    for j, (y, a) in enumerate(zip(outs, w.input_scales)):
        Qw, sw = preps[j]
        want = orc.linear(inp.X, w.G, Qw, sw, inp.b[j], a, threads=THREADS)
        check_y(y, want, oracle.F32, f"qkv linear {j}")
        say("separate", j)
        sep = host(cr.convrot_int8_linear(Xd, w.G, a, lins[j]["Qw"], lins[j]["s_w"],
                                          lins[j]["bias"]))
        assert_bits_equal(y, sep, f"shared vs separate, linear {j}")
    say("alpha 0.5 vs 1")
    one = host(cr.convrot_int8_linear(Xd, w.G, 1.0, lins[3]["Qw"], lins[3]["s_w"],
                                      lins[3]["bias"]))
    assert_bits_equal(outs[3], one, "input scale 0.5 vs 1")


def test_shared_power_of_two_scales(orc):
    """Input scales 2^k (|k| <= 16) read the alpha = 1 packed tensor and skip
    the division; every output must still equal the oracle's literal path
    (pre-scale, own quantization, division) bit for bit.  Six linears need
    three packed tensors: {1, 0.5, 4, 2^-16}, {2^17} and {0.3}."""
    import torch
    rng = np.random.default_rng(41)
    M, K, G = 257, 768, 256
    X = workloads.gaussian_activations(rng, M, K, 0.005, 30.0, workloads.BF16)
    scales = [1.0, 0.5, 4.0, 2.0 ** -16, 2.0 ** 17, 0.3]
    Ns = [96, 64, 130, 32, 80, 17]
    Xd = dev_x(X)
    preps, lins = [], []
    for a, N in zip(scales, Ns):
        W, b = workloads.gaussian_weights(rng, N, K)
        Qw, sw = orc.weight_prep(W, G, threads=THREADS)
        preps.append((Qw, sw, b))
        lins.append(dict(Qw=dev(Qw), s_w=dev(sw), bias=dev(b), input_scale=a, y_dtype=oracle.BF16))
    ws = torch.empty(cr.convrot_workspace_bytes(M, K, 3), dtype=torch.uint8, device="cuda:0")
    say("shared power-of-two scales")
    outs = [host(y) for y in cr.convrot_int8_linear_shared(Xd, G, lins, workspace=ws)]
    for (Qw, sw, b), a, y in zip(preps, scales, outs):
        want = orc.linear(X, G, Qw, sw, b, a, oracle.BF16, threads=THREADS)
        check_y(y, want, oracle.BF16, f"alpha={a}")


def test_fused_output_may_alias_input(orc):
    import torch
    rng = np.random.default_rng(12)
    M, K, N = 40, 512, 256
    X = workloads.gaussian_activations(rng, M, K, 0.01, 20.0, workloads.F32)
    W, b = workloads.gaussian_weights(rng, N, K)
    Qw, sw = orc.weight_prep(W, 64)
    want = orc.linear(X, 64, Qw, sw, b)
    Xd = dev_x(X)
    Y = Xd[:, :N]                 # Y overwrites X's storage (row stride K)
    say("alias")
    cr.convrot_int8_linear(Xd, 64, 1.0, dev(Qw), dev(sw), dev(b), Y=Y)
    assert_bits_equal(np.ascontiguousarray(host(Xd)[:, :N]), want, "aliased Y")


def test_empty_shapes(orc):
    import torch
    Qw = torch.zeros((0, 256), dtype=torch.int8, device="cuda:0")
    Qx = torch.zeros((5, 256), dtype=torch.int8, device="cuda:0")
    sx = torch.ones(5, dtype=torch.float32, device="cuda:0")
    say("empty N")
    Y = cr.int8_linear(Qx, sx, Qw)
    assert Y.shape == (5, 0)
    X = torch.zeros((0, 256), dtype=torch.float32, device="cuda:0")
    say("empty M")
    Y = cr.convrot_int8_linear(X, 16, 1.0, torch.zeros((8, 256), dtype=torch.int8, device="cuda:0"))
    assert Y.shape == (0, 8)


def test_signed_zero_outputs(orc):
    """Zero rows (A = 0) against negative weight scales give -0 before the
    bias; without a bias the output must keep that sign, with one it must be
    the bias (the oracle skips the missing operations)."""
    rng = np.random.default_rng(32)
    M, K, N = 12, 256, 40
    Qx = workloads.random_codes(rng, (M, K))
    Qx[3] = 0
    Qx[7] = 0
    Qw = workloads.random_codes(rng, (N, K))
    sx = workloads.random_scales(rng, M)
    sw = -workloads.random_scales(rng, N)
    b = (rng.standard_normal(N) * 0.1).astype(np.float32)
    A = orc.gemm_i32(Qx, Qw)
    for y_dtype in (oracle.F32, oracle.BF16):
        for bias in (None, b):
            say("signed zeros", y_dtype, bias is None)
            want = orc.epilogue(A, sx, sw, bias, 1.0, y_dtype)
            got = host(cr.int8_linear(dev(Qx), dev(sx), dev(Qw), dev(sw),
                                      None if bias is None else dev(bias), 1.0, y_dtype=y_dtype))
            assert_bits_equal(got, want, f"signed zeros dtype={y_dtype} bias={bias is not None}")
            if bias is None:
                zero_bits = want[3].view(np.uint32 if y_dtype == oracle.F32 else np.uint16)
                assert np.all(zero_bits == (0x80000000 if y_dtype == oracle.F32 else 0x8000))


def test_bf16_output_subnormal_range(orc):
    """Outputs around the binary32 / bf16 subnormal boundary: the kernel's bf16
    conversion must round exactly like the oracle's (nearest, ties to even)."""
    rng = np.random.default_rng(31)
    M, K, N = 64, 256, 96
    Qx = workloads.random_codes(rng, (M, K))
    Qw = workloads.random_codes(rng, (N, K))
    A = orc.gemm_i32(Qx, Qw)
    for sx_scale in (1e-36, 1e-39, 1e-41, 3e-43):
        sx = (workloads.random_scales(rng, M, 0.5, 2.0) * np.float32(sx_scale)).astype(np.float32)
        sw = workloads.random_scales(rng, N, 1e-3, 1e-1)
        for y_dtype in (oracle.F32, oracle.BF16):
            say("subnormal outputs", sx_scale, y_dtype)
            want = orc.epilogue(A, sx, sw, None, 1.0, y_dtype)
            got = host(cr.int8_linear(dev(Qx), dev(sx), dev(Qw), dev(sw), None, 1.0, y_dtype=y_dtype))
            assert_bits_equal(got, want, f"subnormal-range Y scale={sx_scale} dtype={y_dtype}")
