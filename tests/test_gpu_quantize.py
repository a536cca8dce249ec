"""GPU rotate + quantize + pack against the CPU oracle: the whole packed tensor
(codes, pad rows, scale tail) must be identical byte for byte."""
import numpy as np
import pytest

import int8_hadamard_rotated_amd as cr
import oracle
import pins
import workloads
from gpu_util import THREADS, assert_bits_equal, dev, dev_x, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def gpu_packed(X: np.ndarray, G: int, alpha: float = 1.0, K=None):
    Xd = dev_x(X)
    return host(cr.convrot_quantize_rows(Xd, G, alpha, K=K))


@pytest.mark.parametrize("name", ["tiny", "attn", "mlp_up", "qkv", "mlp_down"])
def test_workload_packed_bit_exact(orc, name):
    w = workloads.WORKLOADS[name]
    rng = np.random.default_rng(w.seed)
    X = workloads.gaussian_activations(rng, w.M, w.K, w.outlier_p, w.outlier_f, w.x_dtype)
    for alpha in sorted(set(w.input_scales)):
        say(name, w.M, w.K, w.G, w.x_dtype, "alpha", alpha)
        want = orc.quantize_rows(X, w.G, alpha, threads=THREADS).raw
        got = gpu_packed(X, w.G, alpha)
        assert_bits_equal(got, want, f"{name} packed (alpha={alpha})")


# Rows of 1 to 256 quad spans in both kernels: binary32 rows whose workgroups
# need at most 256 threads take the LDS-staged kernel (K = 4096 and 8192 fill
# its 4 waves), longer binary32 rows and every bf16 row the workgroup kernel;
# spans of 64, 128 and 256 elements (K % 256 != 0 takes the shorter ones).
EDGE_SHAPES = [(1, 64), (3, 128), (4, 192), (5, 256), (127, 320), (13, 512), (17, 768),
               (33, 1280), (11, 1536), (129, 3072), (9, 4096), (3, 6144), (6, 8192), (7, 12288),
               (2, 65536)]


@pytest.mark.parametrize("G", [1, 4, 16, 64, 256])
@pytest.mark.parametrize("dtype", [workloads.F32, workloads.BF16])
def test_edge_shapes(orc, G, dtype):
    rng = np.random.default_rng(100 + G)
    for (M, K) in EDGE_SHAPES:
        if K % G:
            continue
        X = workloads.gaussian_activations(rng, M, K, 0.01, 30.0, dtype)
        for alpha in (1.0, 0.5, 0.3):
            say("edge", M, K, G, dtype, alpha)
            assert_bits_equal(gpu_packed(X, G, alpha), orc.quantize_rows(X, G, alpha).raw,
                              f"M={M} K={K} G={G} {dtype} alpha={alpha}")



# Several input scales of one X in one call: binary32 rows of the staged
# kernel read X once per two scales (five scales: two such launches and one
# single pass), other
# rows (bf16; binary32 rows of 32 768 in the workgroup kernel) one pass per
# scale.  Each packed tensor must equal its own pass byte for byte, pad rows
# and scale tail included, and nothing past it may change.
SCALES_CASES = [(4096, 3072, workloads.F32, 256, (1.0, 0.5)),
                (129, 3072, workloads.F32, 256, (1.0, 0.3, 2.0 ** -20, 7.5, 0.5)),
                (33, 1280, workloads.F32, 64, (0.3, 1.0, 0.25)),
                (13, 512, workloads.F32, 16, (1.0, 0.5)),
                (17, 192, workloads.F32, 4, (3.0, 1.0)),
                (6, 8192, workloads.F32, 256, (1.0, 0.3)),
                (3, 32768, workloads.F32, 256, (1.0, 0.3)),
                (129, 3072, workloads.BF16, 256, (1.0, 0.5, 0.3)),
                # sixteen scales (the most a call takes): eight two-scale passes
                (77, 1024, workloads.F32, 256, (1.0, 0.3, 0.5, 0.7, 1.3, 2.0, 0.11, 3.7, 0.25, 5.0, 0.9,
                                                1.1, 0.6, 2.5, 0.45, 8.0)),
                (50, 768, workloads.BF16, 64, (0.3, 0.7, 1.0, 1.9, 0.5)),
                (5, 4096, workloads.F32, 16, (0.3, 0.7, 1.0)),
                (33, 1024, workloads.F32, 1, (1.0, 0.3)),
                (21, 640, workloads.BF16, 1, (0.3, 1.0))]


@pytest.mark.parametrize("M,K,dtype,G,scales", SCALES_CASES)
def test_quantize_rows_scales(orc, M, K, dtype, G, scales):
    import torch
    rng = np.random.default_rng(M + K + G)
    X = workloads.gaussian_activations(rng, M, K, 0.005, 30.0, dtype)
    pb = cr.convrot_packed_bytes(M, K)
    slot = (pb + 255) // 256 * 256 + 256
    buf = torch.full((slot * len(scales),), 0x5A, dtype=torch.uint8, device="cuda:0")
    outs = [buf[i * slot:i * slot + pb] for i in range(len(scales))]
    say("quantize_rows_scales", M, K, dtype, G, scales)
    cr.convrot_quantize_rows_scales(dev_x(X), G, scales, packed=outs)
    got = host(buf)
    for i, a in enumerate(scales):
        want = orc.quantize_rows(X, G, a, threads=THREADS).raw
        assert_bits_equal(got[i * slot:i * slot + pb], want, f"scale {a}")
        assert np.all(got[i * slot + pb:(i + 1) * slot] == 0x5A), f"wrote past packed tensor {i}"


# (rows, K, dtype, G): 131 073 bf16 rows of 256 make 2049 workgroups of 64
# rows (8196 waves) with three pad rows and 60 rows past the packed tensor in
# the last workgroup; 1025 binary32 rows of 32 768 take the workgroup kernel
# (512 threads, 8224 waves); 26 215 bf16 rows of 320 use spans of 64 elements
# (16 rows per workgroup, 8195 waves).
#   43 691 bf16 rows of 384 use spans of 128 elements (3 quads a row, 16 rows
# and 3 waves per workgroup, 2731 workgroups: 8193 waves, one pad row);
# 513 bf16 rows of 65 536 take 1024-thread workgroups of one row whose
# staging fills 64 KB of dynamic LDS on top of the kernel's static LDS
# (8256 waves, with three pad rows).
WAVE_STORE_SHAPES = [(131073, 256, workloads.BF16, 256), (1025, 32768, workloads.F32, 256),
                     (26215, 320, workloads.BF16, 64), (43691, 384, workloads.BF16, 64),
                     (513, 65536, workloads.BF16, 256)]


@pytest.mark.parametrize("M,K,dtype,G", WAVE_STORE_SHAPES)
def test_wave_stores_with_pad_rows(orc, M, K, dtype, G):
    """Passes of at least 8192 waves in whole waves store their codes through
    LDS, 1 KB per store instruction, with every lane storing pieces of other
    quads.  Bytes past the packed tensor must stay untouched."""
    rng = np.random.default_rng(107)
    X = workloads.gaussian_activations(rng, M, K, 0.005, 30.0, dtype)
    nb = cr.convrot_packed_bytes(M, K)
    Xd = dev_x(X)
    packed = dev(np.full(nb + 4096, 0x5A, dtype=np.uint8))
    say("wave stores", M, K, dtype, G)
    cr.convrot_quantize_rows(Xd, G, packed=packed)
    got = host(packed)
    assert_bits_equal(got[:nb], orc.quantize_rows(X, G).raw, f"wave-store packed M={M} K={K} {dtype}")
    assert np.all(got[nb:] == 0x5A), "bytes past the packed tensor were written"

def test_row_stride(orc):
    rng = np.random.default_rng(7)
    for dtype in (workloads.F32, workloads.BF16):
        wide = workloads.gaussian_activations(rng, 37, 3072 + 64, 0.005, 30.0, dtype)
        say("ldx", dtype)
        got = gpu_packed(wide, 256, K=3072)
        want = orc.quantize_rows(wide, 256, K=3072).raw
        assert_bits_equal(got, want, f"strided rows {dtype}")


def test_special_rows(orc):
    """Zero rows, the constructed rounding-tie row, constant rows, magnitudes
    near the contract's limits and a single isolated outlier."""
    vals, codes = pins.load_tie_row()
    tie = np.repeat(vals, 16).astype(np.float32)
    rng = np.random.default_rng(8)
    K = 256
    rows = [np.zeros(K, np.float32), tie, np.full(K, 3.25, np.float32),
            (rng.standard_normal(K) * 2.0 ** 90).astype(np.float32),
            (rng.standard_normal(K) * 2.0 ** -90).astype(np.float32),
            np.where(np.arange(K) == 77, 1000.0, 0.0).astype(np.float32),
            -tie]
    X = np.stack(rows)
    Xb = workloads.f32_to_bf16_bits(X)
    for G in (4, 16, 64, 256):
        for alpha in (1.0, 0.5):
            say("special rows", G, alpha)
            got = gpu_packed(X, G, alpha)
            want = orc.quantize_rows(X, G, alpha).raw
            assert_bits_equal(got, want, f"special rows G={G} alpha={alpha}")
            say("special rows bf16", G, alpha)
            assert_bits_equal(gpu_packed(Xb, G, alpha), orc.quantize_rows(Xb, G, alpha).raw,
                              f"special bf16 rows G={G} alpha={alpha}")
    # the tie row itself against the golden codes (G = 16 leaves it unrotated)
    p = oracle.Packed(gpu_packed(X, 16), X.shape[0], K)
    assert np.array_equal(p.q[1], np.repeat(codes, 16))
    assert p.s[1] == np.float32(1.0) and p.s[0] == 0 and np.all(p.q[0] == 0)


def test_weight_prep_on_gpu(orc):
    """The offline weight quantization is the same quantizer on W's rows."""
    w = workloads.WORKLOADS["attn"]
    rng = np.random.default_rng(9)
    W, _ = workloads.gaussian_weights(rng, 3072, 3072)
    say("weight prep")
    Qw, sw = orc.weight_prep(W, 256, threads=THREADS)
    p = oracle.Packed(gpu_packed(W, 256), 3072, 3072)
    assert_bits_equal(p.q, Qw, "Q_w")
    assert_bits_equal(p.s, sw, "s_w")


def test_empty_rows_enqueue_nothing():
    import torch
    X = torch.empty((0, 256), dtype=torch.float32, device="cuda:0")
    say("empty")
    out = cr.convrot_quantize_rows(X, 16)
    assert out.numel() == 0
