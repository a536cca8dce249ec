"""The entry points under HIP graph capture.

The library allocates nothing and issues no memory fills: every call only
enqueues its kernels on the caller's stream, so a captured call replays
them.  Each test captures calls once, then replays the graph several times
with new input contents copied into the captured input between replays and
eager work (the same calls, uncaptured) around each replay; every replay
must match the eager result bit for bit, and the eager result the oracle.
"""
import numpy as np
import pytest

import int8_hadamard_rotated_amd as cr
import oracle
import workloads
from gpu_util import THREADS, assert_bits_equal, dev, dev_x, host, say
from test_gpu_linear import check_y

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def capture(fn):
    """Run fn once on a side stream (warm-up), then capture it into a graph."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_fused_linear_replays(orc):
    """convrot_int8_linear (quantize + 256 x 256-tile GEMM) captured and
    replayed over three input sets."""
    import torch
    rng = np.random.default_rng(51)
    M, K, N, G = 2048 + 3, 512, 4608, 256
    Xs = [workloads.gaussian_activations(rng, M, K, 0.005, 30.0, workloads.BF16) for _ in range(3)]
    W, b = workloads.gaussian_weights(rng, N, K)
    Qw, sw = orc.weight_prep(W, G, threads=THREADS)
    Qwd, swd, bd = dev(Qw), dev(sw), dev(b)
    Xd = dev_x(Xs[0])
    Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    ws = torch.empty(cr.convrot_workspace_bytes(M, K, 1), dtype=torch.uint8, device="cuda:0")

    def call():
        cr.convrot_int8_linear(Xd, G, 1.0, Qwd, swd, bd, Y=Y, y_dtype=oracle.BF16, workspace=ws)

    say("graph capture: fused linear", M, K, N)
    g = capture(call)
    for rep in range(REPLAYS):
        for j, X in enumerate(Xs):
            Xd.copy_(dev_x(X))
            say("eager", rep, j)
            eager = host(cr.convrot_int8_linear(Xd, G, 1.0, Qwd, swd, bd, y_dtype=oracle.BF16))
            Y.fill_(-7.0)
            say("replay", rep, j)
            g.replay()
            assert_bits_equal(host(Y), eager, f"replay {rep} input {j}")
            if rep == 0:
                want = orc.linear(X, G, Qw, sw, b, 1.0, oracle.BF16, threads=THREADS)
                check_y(eager, want, oracle.BF16, f"eager input {j}")


def test_rmsnorm_swiglu_chain_replays(orc):
    """RMSNorm producer + quantize -> SwiGLU dual GEMM -> ConvRot of its
    output, three calls in one graph (128 x 128 tiles)."""
    import torch
    rng = np.random.default_rng(61)
    M, K, N, G, G2 = 300, 768, 520, 256, 64
    N2 = 512                                     # columns of Y that the second ConvRot reads
    Xs = [workloads.gaussian_activations(rng, M, K, 0.005, 30.0, workloads.F32) for _ in range(2)]
    Wg, _ = workloads.gaussian_weights(rng, N, K)
    Wu, _ = workloads.gaussian_weights(rng, N, K)
    Qg, sg = orc.weight_prep(Wg, G, threads=THREADS)
    Qu, su = orc.weight_prep(Wu, G, threads=THREADS)
    Qgd, sgd, Qud, sud = dev(Qg), dev(sg), dev(Qu), dev(su)
    weight = dev(workloads.norm_weight(rng, K))
    pre = cr.RMSNormModulate(1e-6, weight=weight)
    Xd = dev_x(Xs[0])
    packed = torch.empty(cr.convrot_packed_bytes(M, K), dtype=torch.uint8, device="cuda:0")
    Y = torch.empty((M, N), dtype=torch.float32, device="cuda:0")
    packed2 = torch.empty(cr.convrot_packed_bytes(M, N2), dtype=torch.uint8, device="cuda:0")

    def chain(Xt, pk, Yt, pk2):
        cr.convrot_quantize_rows_pre(Xt, pre, G, packed=pk)
        qx, s_x = cr.packed_parts(pk, M, K)
        cr.int8_swiglu_linear(qx, s_x, Qgd, sgd, Qud, sud, Y=Yt, y_dtype=oracle.F32, M=M)
        cr.convrot_quantize_rows(Yt, G2, packed=pk2, K=N2)

    say("graph capture: rmsnorm -> swiglu -> convrot", M, K, N)
    g = capture(lambda: chain(Xd, packed, Y, packed2))
    for rep in range(REPLAYS):
        for j, X in enumerate(Xs):
            Xd.copy_(dev_x(X))
            e_pk = torch.empty_like(packed)
            e_Y = torch.empty_like(Y)
            e_pk2 = torch.empty_like(packed2)
            say("eager", rep, j)
            chain(Xd, e_pk, e_Y, e_pk2)
            packed.fill_(0x5A)
            Y.fill_(-7.0)
            packed2.fill_(0x5A)
            say("replay", rep, j)
            g.replay()
            assert_bits_equal(host(packed), host(e_pk), f"packed, replay {rep} input {j}")
            assert_bits_equal(host(Y), host(e_Y), f"Y, replay {rep} input {j}")
            assert_bits_equal(host(packed2), host(e_pk2), f"packed output, replay {rep} input {j}")


def test_shared_entry_replays(orc):
    """convrot_int8_linear_shared with input scales {1, 0.5, 0.3}: one packed
    tensor for 1 and 0.5 (a power of two), one more for 0.3, one grouped GEMM."""
    import torch
    rng = np.random.default_rng(71)
    M, K, G = 513, 1024, 64
    Ns, scales = [384, 130, 256], [1.0, 0.5, 0.3]
    Xs = [workloads.gaussian_activations(rng, M, K, 0.005, 30.0, workloads.F32) for _ in range(2)]
    preps, lins, Ys = [], [], []
    for a, N in zip(scales, Ns):
        W, b = workloads.gaussian_weights(rng, N, K)
        Qw, sw = orc.weight_prep(W, G, threads=THREADS)
        preps.append((Qw, sw, b))
        Ys.append(torch.empty((M, N), dtype=torch.float32, device="cuda:0"))
        lins.append(dict(Qw=dev(Qw), s_w=dev(sw), bias=dev(b), input_scale=a))
    ws = torch.empty(cr.convrot_workspace_bytes(M, K, 2), dtype=torch.uint8, device="cuda:0")
    Xd = dev_x(Xs[0])
    cap = [dict(l, Y=y) for l, y in zip(lins, Ys)]

    say("graph capture: shared entry", M, K, Ns)
    g = capture(lambda: cr.convrot_int8_linear_shared(Xd, G, cap, workspace=ws))
    for rep in range(REPLAYS):
        for j, X in enumerate(Xs):
            Xd.copy_(dev_x(X))
            say("eager", rep, j)
            eager = [host(y) for y in cr.convrot_int8_linear_shared(Xd, G, lins)]
            for y in Ys:
                y.fill_(-7.0)
            say("replay", rep, j)
            g.replay()
            for d, (y, e) in enumerate(zip(Ys, eager)):
                assert_bits_equal(host(y), e, f"linear {d}, replay {rep} input {j}")
            if rep == 0:
                for d, ((Qw, sw, b), a) in enumerate(zip(preps, scales)):
                    want = orc.linear(X, G, Qw, sw, b, a, threads=THREADS)
                    check_y(eager[d], want, oracle.F32, f"eager linear {d} input {j}")


def test_scales_grouped_and_norm_replays(orc):
    """Two chains in one graph: the literal qkv-style step (one
    convrot_quantize_rows_scales call for input scales 1 and 0.3 on binary32
    rows, then one int8_linear_grouped launch whose second linear reads the
    0.3 tensor) and a Norm -> Mul(weight) producer pass at G = 1 feeding
    int8_linear; every replay against the eager calls, those against the
    oracle."""
    import torch
    rng = np.random.default_rng(81)
    M, K, G = 517, 1024, 256
    Ns, scales = [384, 200], [1.0, 0.3]
    Xs = [workloads.gaussian_activations(rng, M, K, 0.005, 30.0, workloads.F32) for _ in range(2)]
    Zs = [workloads.gaussian_activations(rng, M, K, 0.005, 30.0, workloads.BF16) for _ in range(2)]
    preps, lins, Ys = [], [], []
    for a, N in zip(scales, Ns):
        W, b = workloads.gaussian_weights(rng, N, K)
        Qw, sw = orc.weight_prep(W, G, threads=THREADS)
        preps.append((Qw, sw, b))
        Ys.append(torch.empty((M, N), dtype=torch.float32, device="cuda:0"))
        lins.append(dict(Qw=dev(Qw), s_w=dev(sw), bias=dev(b), input_scale=a))
    W1, b1 = workloads.gaussian_weights(rng, 300, K)
    Q1, s1 = orc.weight_prep(W1, 1, threads=THREADS)
    Q1d, s1d, b1d = dev(Q1), dev(s1), dev(b1)
    nw = workloads.norm_weight(rng, K)
    norm = cr.NormMul(1e-6, dev(nw))
    pb = cr.convrot_packed_bytes(M, K)
    Xd, Zd = dev_x(Xs[0]), dev_x(Zs[0])

    def chain(pks, ys, pk3, y3):
        cr.convrot_quantize_rows_scales(Xd, G, scales, packed=pks)
        qx, sx = cr.packed_parts(pks[0], M, K)
        q2, s2 = cr.packed_parts(pks[1], M, K)
        cr.int8_linear_grouped(qx, sx, [dict(lins[0], Y=ys[0]), dict(lins[1], Y=ys[1], Qx=q2, s_x=s2)], M=M)
        cr.convrot_quantize_rows_pre(Zd, norm, 1, packed=pk3)
        q3, s3 = cr.packed_parts(pk3, M, K)
        cr.int8_linear(q3, s3, Q1d, s1d, b1d, 1.0, Y=y3, M=M)

    def bufs():
        return ([torch.empty(pb, dtype=torch.uint8, device="cuda:0") for _ in scales],
                [torch.empty_like(y) for y in Ys], torch.empty(pb, dtype=torch.uint8, device="cuda:0"),
                torch.empty((M, 300), dtype=torch.float32, device="cuda:0"))

    cap_pks, _, cap_pk3, cap_y3 = bufs()
    say("graph capture: scales + grouped, norm at G=1", M, K, Ns)
    g = capture(lambda: chain(cap_pks, Ys, cap_pk3, cap_y3))
    for rep in range(REPLAYS):
        for j, (X, Z) in enumerate(zip(Xs, Zs)):
            Xd.copy_(dev_x(X))
            Zd.copy_(dev_x(Z))
            e_pks, e_ys, e_pk3, e_y3 = bufs()
            say("eager", rep, j)
            chain(e_pks, e_ys, e_pk3, e_y3)
            for y in Ys + [cap_y3]:
                y.fill_(-7.0)
            for pk in cap_pks + [cap_pk3]:
                pk.fill_(0x5A)
            say("replay", rep, j)
            g.replay()
            for d in range(2):
                assert_bits_equal(host(cap_pks[d]), host(e_pks[d]), f"packed {d}, replay {rep} input {j}")
                assert_bits_equal(host(Ys[d]), host(e_ys[d]), f"grouped linear {d}, replay {rep} input {j}")
            assert_bits_equal(host(cap_pk3), host(e_pk3), f"norm packed, replay {rep} input {j}")
            assert_bits_equal(host(cap_y3), host(e_y3), f"G=1 linear, replay {rep} input {j}")
            if rep == 0:
                for d, ((Qw, sw, b), a) in enumerate(zip(preps, scales)):
                    want = orc.linear(X, G, Qw, sw, b, a, threads=THREADS)
                    check_y(host(e_ys[d]), want, oracle.F32, f"eager grouped linear {d} input {j}")
                want = orc.linear(orc.norm_rows(Z, 1e-6, nw, threads=THREADS), 1, Q1, s1, b1, 1.0,
                                  threads=THREADS)
                check_y(host(e_y3), want, oracle.F32, f"eager norm G=1 linear input {j}")
