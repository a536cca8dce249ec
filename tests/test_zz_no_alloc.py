"""The no-allocation fused entry (convrot_int8_linear_noalloc) against the
fused entry with a caller workspace (convrot_int8_linear), which the parity
tests check against the oracle: two calls in a row, the second with a smaller
input, each bit for bit (and against the oracle as well)."""
import numpy as np
import pytest

import int8_hadamard_rotated_amd as cr
import oracle
import workloads
from gpu_util import THREADS, assert_bits_equal, dev, dev_x, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


# (M, K, N, G, x dtype, y dtype, input scale): a 256 x 256-tile call near the
# size of a DiT projection, then a smaller ragged one that reuses the same
# static buffer (its bytes past the second packed tensor still hold the
# first call's codes)
CALLS = [(2048 + 5, 3072, 2304, 256, workloads.BF16, oracle.BF16, 0.3),
         (300 + 1, 1024, 520, 64, workloads.F32, oracle.F32, 1.0)]


def test_noalloc_matches_workspace_entry(orc):
    for i, (M, K, N, G, xd, yd, a) in enumerate(CALLS):
        rng = np.random.default_rng(300 + i)
        X = workloads.gaussian_activations(rng, M, K, 0.005, 30.0, xd)
        W, b = workloads.gaussian_weights(rng, N, K)
        Qw, sw = orc.weight_prep(W, G, threads=THREADS)
        Xd, Qwd, swd, bd = dev_x(X), dev(Qw), dev(sw), dev(b)
        say("noalloc", i, M, K, N, G, xd, yd, a)
        got = host(cr.convrot_int8_linear_noalloc(Xd, G, a, Qwd, swd, bd, y_dtype=yd))
        say("workspace entry", i, M, K, N, G, xd, yd, a)
        ref = host(cr.convrot_int8_linear(Xd, G, a, Qwd, swd, bd, y_dtype=yd))
        assert_bits_equal(got, ref, f"noalloc call {i} vs convrot_int8_linear")
        want = orc.linear(X, G, Qw, sw, b, a, yd, threads=THREADS)
        assert_bits_equal(got, want, f"noalloc call {i} vs oracle")


def test_noalloc_rejects_beyond_static_buffer():
    import torch
    M, K = 8192, 8192
    assert cr.convrot_workspace_bytes(M, K, 1) > 64 << 20
    X = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda:0")
    Qw = torch.zeros((64, K), dtype=torch.int8, device="cuda:0")
    say("noalloc oversize")
    with pytest.raises(cr.ConvrotError) as e:
        cr.convrot_int8_linear_noalloc(X, 256, 1.0, Qw)
    assert e.value.status == cr.EWORKSPACE
