"""The C ABI on the host (no GPU): the library loads, exports every function
that include/convrot.h declares, and rejects bad arguments before anything is
enqueued.  Every call here fails validation (or is a no-op), so no HIP API is
reached; the pointers are fake, well-aligned addresses that are never touched."""
import ctypes
import os
import re
import subprocess

import pytest

import int8_hadamard_rotated_amd as cr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "convrot.h")

OK, EINVAL, EUNSUP, EOVF, EOVL, EWS = cr.OK, cr.EINVAL, cr.EUNSUPPORTED, cr.EOVERFLOW, cr.EOVERLAP, cr.EWORKSPACE
BASE = 0x7F00_0000_0000            # fake, 256-byte aligned device addresses
MB = 1 << 20


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    text = re.sub(r"typedef\s+(enum|struct)\s*\{.*?\}\s*\w+\s*;", "", text, flags=re.S)
    text = re.sub(r"#[^\n]*", "", text)
    names = re.findall(r"\b([A-Za-z_]\w*)\s*\([^;{}]*\)\s*;", text)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    return cr.library()


def test_header_declares_the_boundary():
    assert header_functions() == sorted([
        "convrot_packed_bytes", "convrot_quantize_rows", "int8_linear", "convrot_workspace_bytes",
        "convrot_int8_linear", "convrot_int8_linear_shared", "convrot_int8_gemm_i32",
        "convrot_status_string", "convrot_quantize_rows_pre", "convrot_int8_linear_shared_pre",
        "int4_linear", "convrot_int4_gemm_i32", "int8_linear_post", "convrot_expf",
        "int8_swiglu_linear", "convrot_int8_linear_noalloc", "int8_linear_grouped",
        "convrot_quantize_rows_scales"])


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", cr.LIBRARY], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in header_functions():
        assert name in exported, f"{name} not exported with C linkage"
        assert getattr(lib, name) is not None


def test_status_strings(lib):
    for code in (OK, EINVAL, EUNSUP, EOVF, EOVL, EWS, cr.EHIP):
        s = cr.convrot_status_string(code)
        assert s and s != "unknown status"
    assert cr.convrot_status_string(12345) == "unknown status"


def test_size_queries():
    assert cr.convrot_packed_bytes(5, 256) == 8 * 256 + 4 * 8
    assert cr.convrot_packed_bytes(4096, 3072) == 4096 * 3072 + 4 * 4096
    assert cr.convrot_packed_bytes(0, 3072) == 0
    assert cr.convrot_packed_bytes(-1, 3072) == 0
    assert cr.convrot_workspace_bytes(5, 256, 1) == 2304      # 2080 rounded up to 256
    assert cr.convrot_workspace_bytes(5, 256, 2) == 4608
    assert cr.convrot_workspace_bytes(4096, 3072, 2) == 2 * (4096 * 3072 + 4 * 4096)


def q(lib, X=BASE, dt=cr.F32, M=8, K=256, ldx=None, G=16, a=1.0, packed=BASE + 64 * MB):
    return lib.convrot_quantize_rows(ctypes.c_void_p(X), dt, M, K, K if ldx is None else ldx, G,
                                     ctypes.c_float(a), ctypes.c_void_p(packed), None)


def test_quantize_validation(lib):
    assert q(lib, G=8) == EUNSUP
    assert q(lib, G=2) == EUNSUP
    assert q(lib, G=1, M=0) == OK                        # 4^0: no rotation
    assert q(lib, G=1024, K=2048) == EUNSUP
    assert q(lib, K=100, G=4) == EUNSUP                  # K % 64
    assert q(lib, K=320, G=256) == EUNSUP                # K % G
    assert q(lib, K=65792, G=256) == EUNSUP              # longer than one workgroup's row
    assert q(lib, dt=7) == EUNSUP
    assert q(lib, M=-1) == EINVAL
    assert q(lib, K=0) == EINVAL
    assert q(lib, ldx=128) == EINVAL                     # ldx < K
    assert q(lib, ldx=258) == EINVAL                     # row stride not a 16-byte multiple
    assert q(lib, X=0) == EINVAL
    assert q(lib, X=BASE + 4) == EINVAL                  # X misaligned
    assert q(lib, packed=0) == EINVAL
    assert q(lib, packed=BASE + 8 + 64 * MB) == EINVAL   # packed misaligned
    for a in (0.0, -1.0, float("inf"), float("nan")):
        assert q(lib, a=a) == EINVAL
    assert q(lib, packed=BASE + 1024) == EOVL            # packed overlaps X
    assert q(lib, M=0) == OK                             # empty input: nothing enqueued
    assert q(lib, M=0, X=0, packed=0) == OK


def test_quantize_scales_validation(lib):
    """convrot_quantize_rows_scales: count, scales and the packed tensors'
    placement, all before any HIP call."""
    M, K = 8, 256
    pb = cr.convrot_packed_bytes(M, K)

    def call(scales, outs, n=None, X=BASE, G=16, M=M):
        sc = (ctypes.c_float * max(len(scales), 1))(*scales)
        ps = (ctypes.c_void_p * max(len(outs), 1))(*outs)
        return lib.convrot_quantize_rows_scales(ctypes.c_void_p(X), cr.F32, M, K, K, G,
                                                len(scales) if n is None else n, sc, ps, None)
    P0, P1 = BASE + 64 * MB, BASE + 96 * MB
    assert call([1.0, 0.5], [P0, P1], n=0) == EINVAL
    assert call([1.0] * 17, [P0] * 17) == EINVAL
    assert call([1.0, 0.0], [P0, P1]) == EINVAL          # a scale that is not positive
    assert call([1.0, float("nan")], [P0, P1]) == EINVAL
    assert call([1.0, 0.5], [P0, 0]) == EINVAL           # a missing packed tensor
    assert call([1.0, 0.5], [P0, P1 + 8]) == EINVAL      # misaligned
    assert call([1.0, 0.5], [P0, P0 + pb - 16]) == EOVL  # two packed tensors overlap
    assert call([1.0, 0.5], [P0, BASE + 1024]) == EOVL   # a packed tensor on X
    assert call([1.0, 0.5], [P0, P1], G=2) == EUNSUP
    assert call([1.0, 0.5], [P0, P1], M=0) == OK


def qpre(lib, kind=cr.PRE_MODULATE, sc=BASE + 96 * MB, sh=BASE + 97 * MB, M=8, K=256,
         packed=BASE + 64 * MB, raw=False, w=None, eps=0.0):
    d = None if raw else ctypes.byref(cr.PreDesc(kind, sc, sh, w, eps))
    return lib.convrot_quantize_rows_pre(ctypes.c_void_p(BASE), cr.F32, M, K, K, d, 16,
                                         ctypes.c_float(1.0), ctypes.c_void_p(packed), None)


def test_producer_validation(lib):
    assert qpre(lib, kind=7) == EUNSUP
    assert qpre(lib, sc=0) == EINVAL                     # modulation needs its scale
    assert qpre(lib, sc=BASE + 96 * MB + 4) == EINVAL    # 16-byte aligned vectors
    assert qpre(lib, sh=BASE + 97 * MB + 8) == EINVAL
    assert qpre(lib, sc=BASE + 64 * MB + 512) == EOVL    # packed overlaps the scale
    assert qpre(lib, sh=BASE + 64 * MB + 2048) == EOVL   # ... or the shift
    assert qpre(lib, M=0) == OK
    assert qpre(lib, M=0, raw=True) == OK                # NULL producer
    assert qpre(lib, kind=cr.PRE_NONE, sc=0, sh=0, M=0) == OK
    # RMSNorm -> Mul(weight) -> Modulate: scale optional, shift needs it,
    # eps finite and >= 0, aligned weight that packed does not overlap, rows
    # up to half the quantizer's K
    rms = cr.PRE_RMSNORM_MODULATE
    w = BASE + 98 * MB
    assert qpre(lib, kind=rms, w=w, eps=1e-6, M=0) == OK
    assert qpre(lib, kind=rms, sc=0, sh=0, w=0, eps=0.0, M=0) == OK     # plain RMSNorm
    assert qpre(lib, kind=rms, sc=0, w=w) == EINVAL                     # shift without scale
    assert qpre(lib, kind=rms, w=w, eps=-1e-6) == EINVAL
    assert qpre(lib, kind=rms, w=w, eps=float("inf")) == EINVAL
    assert qpre(lib, kind=rms, w=w, eps=float("nan")) == EINVAL
    assert qpre(lib, kind=rms, w=w + 8) == EINVAL
    assert qpre(lib, kind=rms, w=BASE + 64 * MB + 1024) == EOVL        # packed overlaps the weight
    assert qpre(lib, kind=rms, w=w, K=32768 + 256) == EUNSUP
    # Norm -> Mul(weight): no scale or shift, the same eps, weight and row rules
    nm = cr.PRE_NORM_MUL
    assert qpre(lib, kind=nm, sc=0, sh=0, w=w, eps=1e-6, M=0) == OK
    assert qpre(lib, kind=nm, sc=0, sh=0, w=0, eps=0.0, M=0) == OK       # Norm alone
    assert qpre(lib, kind=nm, sh=0, w=w) == EINVAL                      # a scale
    assert qpre(lib, kind=nm, sc=0, w=w) == EINVAL                      # a shift
    assert qpre(lib, kind=nm, sc=0, sh=0, w=w, eps=-1e-6) == EINVAL
    assert qpre(lib, kind=nm, sc=0, sh=0, w=w, eps=float("nan")) == EINVAL
    assert qpre(lib, kind=nm, sc=0, sh=0, w=w + 8) == EINVAL
    assert qpre(lib, kind=nm, sc=0, sh=0, w=BASE + 64 * MB + 1024) == EOVL   # packed on the weight
    assert qpre(lib, kind=nm, sc=0, sh=0, w=w, K=32768 + 256) == EUNSUP
    # gated activation: a second input with X's dtype, aligned, with a valid
    # stride, that packed does not overlap; SiLU or Sigmoid; same row limit
    def qact(up=BASE + 100 * MB, ld=256, act=cr.ACT_SILU, M=8, K=256, packed=BASE + 64 * MB):
        d = cr.PreDesc(cr.PRE_GATED_ACT, None, None, None, 0.0, up, ld, act)
        return lib.convrot_quantize_rows_pre(ctypes.c_void_p(BASE), cr.F32, M, K, K, ctypes.byref(d),
                                             16, ctypes.c_float(1.0), ctypes.c_void_p(packed), None)
    assert qact(M=0) == OK
    assert qact(up=BASE, M=0) == OK                                     # up may alias X
    assert qact(act=3) == EUNSUP
    assert qact(up=0) == EINVAL
    assert qact(up=BASE + 100 * MB + 4) == EINVAL
    assert qact(ld=200) == EINVAL                                       # below K
    assert qact(ld=257) == EINVAL                                       # stride not 16-byte
    assert qact(up=BASE + 64 * MB + 256) == EOVL                        # packed overlaps up
    assert qact(K=32768 + 256, ld=32768 + 256) == EUNSUP
    # the shared entry: the workspace must not overlap the vectors
    d = cr.LinearDesc(BASE + 16 * MB, None, None, 32, 1.0, BASE + 32 * MB, cr.F32, 32)
    pre = cr.PreDesc(cr.PRE_RMSNORM_MODULATE, None, None, BASE + 48 * MB + 512, 1e-6)
    f = lib.convrot_int8_linear_shared_pre
    assert f(ctypes.c_void_p(BASE), cr.F32, 8, 256, 256, ctypes.byref(pre), 16, 1, ctypes.byref(d),
             ctypes.c_void_p(BASE + 48 * MB), MB, None) == EOVL
    pre = cr.PreDesc(cr.PRE_MODULATE, BASE + 48 * MB + 256, None)
    f = lib.convrot_int8_linear_shared_pre
    assert f(ctypes.c_void_p(BASE), cr.F32, 8, 256, 256, ctypes.byref(pre), 16, 1, ctypes.byref(d),
             ctypes.c_void_p(BASE + 48 * MB), MB, None) == EOVL
    pre.kind = 9
    assert f(ctypes.c_void_p(BASE), cr.F32, 8, 256, 256, ctypes.byref(pre), 16, 1, ctypes.byref(d),
             ctypes.c_void_p(BASE + 48 * MB), MB, None) == EUNSUP


def test_swiglu_validation(lib):
    f = lib.int8_swiglu_linear
    def call(Qx=BASE, sx=BASE + 8 * MB, M=8, K=256, Wg=BASE + 16 * MB, sg=BASE + 24 * MB,
             Wu=BASE + 40 * MB, su=BASE + 48 * MB, N=32, a=1.0, Y=BASE + 32 * MB, dt=cr.F32):
        return f(ctypes.c_void_p(Qx), ctypes.c_void_p(sx), M, K, ctypes.c_void_p(Wg), ctypes.c_void_p(sg),
                 ctypes.c_void_p(Wu), ctypes.c_void_p(su), N, ctypes.c_float(a), ctypes.c_void_p(Y),
                 dt, N, None)
    assert call(M=0) == OK
    assert call(K=100) == EUNSUP
    assert call(Wu=0) == EINVAL
    assert call(Wg=BASE + 16 * MB + 4) == EINVAL
    assert call(Y=BASE + 40 * MB + 64) == EOVL                   # output on the up weights
    assert call(Y=BASE + 48 * MB) == EOVL                        # ... or the up scales
    assert call(a=-1.0) == EINVAL


def test_expf_validation(lib):
    f = lib.convrot_expf
    assert f(None, None, 0, None) == OK
    assert f(None, ctypes.c_void_p(BASE), 4, None) == EINVAL
    assert f(ctypes.c_void_p(BASE + 2), ctypes.c_void_p(BASE + MB), 4, None) == EINVAL
    assert f(ctypes.c_void_p(BASE), ctypes.c_void_p(BASE + 8), 4, None) == EOVL
    assert f(ctypes.c_void_p(BASE), ctypes.c_void_p(BASE + MB), -1, None) == EINVAL


def lin(lib, Qx=BASE, sx=BASE + 8 * MB, M=8, K=256, Qw=BASE + 16 * MB, sw=BASE + 24 * MB,
        b=BASE + 25 * MB, N=32, a=1.0, Y=BASE + 32 * MB, dt=cr.F32, ldy=None):
    return lib.int8_linear(ctypes.c_void_p(Qx), ctypes.c_void_p(sx), M, K, ctypes.c_void_p(Qw),
                           ctypes.c_void_p(sw), ctypes.c_void_p(b), N, ctypes.c_float(a),
                           ctypes.c_void_p(Y), dt, N if ldy is None else ldy, None)


def test_int8_linear_validation(lib):
    assert lin(lib, K=100) == EUNSUP
    assert lin(lib, K=133184) == EOVF                    # K * 127^2 would exceed int32
    assert lin(lib, K=0) == EINVAL
    assert lin(lib, M=-2) == EINVAL
    assert lin(lib, N=-1) == EINVAL
    assert lin(lib, ldy=16) == EINVAL
    assert lin(lib, dt=3) == EUNSUP
    assert lin(lib, Qx=0) == EINVAL
    assert lin(lib, sx=0) == EINVAL
    assert lin(lib, Qw=0) == EINVAL
    assert lin(lib, Y=0) == EINVAL
    assert lin(lib, Qw=BASE + 16 * MB + 4) == EINVAL
    assert lin(lib, Y=BASE + 32 * MB + 2) == EINVAL
    assert lin(lib, a=0.0) == EINVAL
    assert lin(lib, Y=BASE + 16 * MB + 256) == EOVL      # Y overlaps Qw
    assert lin(lib, Y=BASE + 24 * MB) == EOVL            # Y overlaps s_w
    assert lin(lib, Y=BASE + 8 * MB) == EOVL             # Y overlaps s_x
    assert lin(lib, Y=BASE) == EOVL                      # Y overlaps Qx
    assert lin(lib, M=0) == OK
    assert lin(lib, N=0) == OK
    # the largest K that is still exact passes the K check (then fails on Qx)
    assert lin(lib, K=133120, Qx=0) == EINVAL


def test_int4_linear_validation(lib):
    def l4(K=256, W4=BASE + 16 * MB, Y=BASE + 32 * MB, M=8, N=32):
        return lib.int4_linear(ctypes.c_void_p(BASE), ctypes.c_void_p(BASE + 8 * MB), M, K,
                               ctypes.c_void_p(W4), None, None, N, ctypes.c_float(1.0),
                               ctypes.c_void_p(Y), cr.F32, N, None)
    assert l4(K=132160) == EOVF                          # 16 * K * 127 * 8 would exceed int32
    assert l4(K=132096, W4=0) == EINVAL                  # the largest exact K passes the K check
    assert l4(K=96) == EUNSUP
    assert l4(W4=BASE + 16 * MB + 8) == EINVAL           # 16-byte aligned weights
    # Y overlapping the packed weights (N * K/2 bytes), not beyond them
    assert l4(Y=BASE + 16 * MB + 32 * 128 - 64) == EOVL
    assert l4(M=0) == OK
    f = lib.convrot_int4_gemm_i32
    assert f(ctypes.c_void_p(BASE), ctypes.c_void_p(BASE + MB), 4, 132160, 4,
             ctypes.c_void_p(BASE + 2 * MB), None) == EOVF
    assert f(None, None, 0, 64, 4, None, None) == OK


def test_post_validation(lib):
    Y = BASE + 32 * MB

    def lp(kind=cr.POST_GATED_RESIDUAL, scale=1.0, gate=BASE + 40 * MB, res=BASE + 44 * MB, ld=32,
           M=8, N=32):
        d = cr.PostDesc(kind, scale, gate, res, ld)
        return lib.int8_linear_post(ctypes.c_void_p(BASE), ctypes.c_void_p(BASE + 8 * MB), M, 256,
                                    ctypes.c_void_p(BASE + 16 * MB), None, None, N,
                                    ctypes.c_float(1.0), ctypes.byref(d), ctypes.c_void_p(Y),
                                    cr.F32, N, None)
    assert lp(kind=5) == EUNSUP
    assert lp(kind=5, M=0) == EUNSUP                     # checked before the empty-shape exit
    assert lp(scale=float("inf")) == EINVAL
    assert lp(gate=0) == EINVAL
    assert lp(gate=BASE + 40 * MB + 2) == EINVAL
    assert lp(res=0) == EINVAL
    assert lp(res=BASE + 44 * MB + 2) == EINVAL          # f32 residual must be 4-byte aligned
    assert lp(ld=16) == EINVAL                           # row stride below N
    assert lp(res=Y + 16) == EOVL                        # overlaps Y without being Y
    assert lp(res=Y, ld=48) == EOVL                      # Y's storage at another stride
    assert lp(gate=Y + 64) == EOVL
    assert lp(M=0) == OK


def test_gemm_i32_validation(lib):
    f = lib.convrot_int8_gemm_i32
    assert f(ctypes.c_void_p(BASE), ctypes.c_void_p(BASE + MB), 4, 133184, 4,
             ctypes.c_void_p(BASE + 2 * MB), None) == EOVF
    assert f(ctypes.c_void_p(BASE), ctypes.c_void_p(BASE + MB), 4, 96, 4,
             ctypes.c_void_p(BASE + 2 * MB), None) == EUNSUP
    assert f(ctypes.c_void_p(BASE), ctypes.c_void_p(BASE + MB), 4, 64, 4,
             ctypes.c_void_p(BASE + MB), None) == EOVL
    assert f(None, ctypes.c_void_p(BASE + MB), 4, 64, 4, ctypes.c_void_p(BASE + 2 * MB), None) == EINVAL
    assert f(None, None, 0, 64, 4, None, None) == OK


def desc(Qw, Y, N=32, a=1.0, sw=None, b=None, dt=cr.F32):
    d = cr.LinearDesc()
    d.Qw, d.Y, d.N, d.input_scale, d.s_w, d.bias, d.y_dtype, d.ldy = Qw, Y, N, a, sw, b, dt, N
    return d


def shared(lib, ds, ws=BASE + 512 * MB, ws_bytes=1 << 30, M=8, K=256, X=BASE, G=16):
    arr = (cr.LinearDesc * max(len(ds), 1))(*ds)
    return lib.convrot_int8_linear_shared(ctypes.c_void_p(X), cr.F32, M, K, K, G, len(ds), arr,
                                          ctypes.c_void_p(ws), ws_bytes, None)


def test_shared_validation(lib):
    W1, W2 = BASE + 64 * MB, BASE + 96 * MB
    Y1, Y2 = BASE + 128 * MB, BASE + 160 * MB
    good = [desc(W1, Y1), desc(W2, Y2, a=0.3)]
    need = cr.convrot_workspace_bytes(8, 256, 2)
    need1 = cr.convrot_workspace_bytes(8, 256, 1)
    assert shared(lib, []) == EINVAL
    assert shared(lib, [desc(W1, Y1)] * 17) == EINVAL
    assert shared(lib, good, ws=0) == EWS
    assert shared(lib, good, ws_bytes=need - 1) == EWS
    # a power-of-two input scale 2^k, |k| <= 16, reads the alpha = 1 packed
    # tensor, 2^17 needs a slot of its own (every call here fails validation
    # before any HIP call; the GPU tests run the passing case)
    assert shared(lib, [desc(W1, Y1), desc(W2, Y2, a=0.5)], ws_bytes=need1 - 1) == EWS
    assert shared(lib, [desc(W1, Y1), desc(W2, Y2, a=2.0 ** 17)], ws_bytes=need1) == EWS
    assert shared(lib, [desc(W1, Y1), desc(W2, Y1 + 64)]) == EOVL          # outputs overlap
    assert shared(lib, [desc(W1, Y1), desc(W2, W1 + 128)]) == EOVL         # output hits a weight
    assert shared(lib, good, ws=Y1) == EOVL                                 # workspace hits an output
    assert shared(lib, good, ws=BASE) == EOVL                               # workspace hits X
    assert shared(lib, [desc(W1, Y1, a=-1.0)]) == EINVAL
    assert shared(lib, good, G=2) == EUNSUP
    named = desc(W2, Y2)
    named.Qx, named.s_x = BASE + 192 * MB, BASE + 200 * MB
    assert shared(lib, [desc(W1, Y1), named]) == EINVAL                     # the entry quantizes X itself
    assert shared(lib, good, M=0) == OK


def test_fused_validation(lib):
    f = lib.convrot_int8_linear
    args = lambda Y, ws, wsb: (ctypes.c_void_p(BASE), cr.F32, 8, 256, 256, 16, ctypes.c_float(1.0),
                               ctypes.c_void_p(BASE + 64 * MB), None, None, 32, ctypes.c_void_p(Y),
                               cr.F32, 32, ctypes.c_void_p(ws), wsb, None)
    need = cr.convrot_workspace_bytes(8, 256, 1)
    assert f(*args(BASE + 128 * MB, BASE + 256 * MB, need - 16)) == EWS
    assert f(*args(BASE + 64 * MB, BASE + 256 * MB, need)) == EOVL          # Y on the weights
    assert f(*args(BASE + 256 * MB, BASE + 256 * MB, need)) == EOVL         # Y on the workspace


def test_grouped_validation(lib):
    """int8_linear_grouped: count, shapes and overlaps, before any HIP call."""
    f = lib.int8_linear_grouped
    Qx, sx = BASE, BASE + 16 * MB
    W1, W2, Y1, Y2 = BASE + 64 * MB, BASE + 96 * MB, BASE + 128 * MB, BASE + 192 * MB

    def desc(W, Y, N=32, a=1.0, ld=None):
        d = cr.LinearDesc()
        d.Qw, d.s_w, d.bias, d.N, d.input_scale = W, None, None, N, a
        d.Y, d.y_dtype, d.ldy = Y, cr.F32, N if ld is None else ld
        return d

    def call(ds, M=8, K=256, n=None, qx=Qx):
        arr = (cr.LinearDesc * max(len(ds), 1))(*ds)
        return f(ctypes.c_void_p(qx), ctypes.c_void_p(sx), M, K, len(ds) if n is None else n, arr, None)

    good = [desc(W1, Y1), desc(W2, Y2)]
    assert call(good, n=0) == EINVAL
    assert call(good, n=17) == EINVAL
    assert call(good, K=250) == EUNSUP
    assert call(good, K=133120 + 64) == EOVF
    assert call([desc(W1, Y1), desc(W2, Y1 + 64)]) == EOVL            # outputs overlap
    assert call([desc(W1, Y1), desc(W2, W1 + 128)]) == EOVL           # output on a weight
    assert call(good, qx=Y1) == EOVL                                   # output on Q_x
    assert call([desc(W1, Y1, a=0.0)]) == EINVAL
    assert call([desc(W1, Y1, ld=16)]) == EINVAL                       # ldy < N
    assert call(good, qx=0) == EINVAL

    def own(W, Y, qx, sx):                                             # a linear with its own input
        d = desc(W, Y)
        d.Qx, d.s_x = qx, sx
        return d
    Qx2, sx2 = BASE + 32 * MB, BASE + 48 * MB
    assert call([desc(W1, Y1), own(W2, Y2, Qx2, None)]) == EINVAL     # codes without scales
    assert call([desc(W1, Y1), own(W2, Y2, None, sx2)]) == EINVAL     # scales without codes
    assert call([desc(W1, Y1), own(W2, Y2, Qx2 + 8, sx2)]) == EINVAL  # codes not 16-byte aligned
    assert call([desc(W1, Y1), own(W2, Y2, Qx2, sx2 + 2)]) == EINVAL  # scales not 4-byte aligned
    assert call([desc(W1, Qx2 + 64), own(W2, Y2, Qx2, sx2)]) == EOVL  # output on another's codes
    assert call([desc(W1, sx2), own(W2, Y2, Qx2, sx2)]) == EOVL       # output on another's scales
    assert call(good, M=0) == OK


def test_noalloc_validation(lib):
    """The no-allocation entry validates like the fused one and rejects a
    packed tensor beyond its 64 MiB static buffer, all before any HIP call."""
    f = lib.convrot_int8_linear_noalloc
    args = lambda M, K, G=16, Y=BASE + 512 * MB, a=1.0: (
        ctypes.c_void_p(BASE), cr.F32, M, K, K, G, ctypes.c_float(a),
        ctypes.c_void_p(BASE + 384 * MB), None, None, 32, ctypes.c_void_p(Y), cr.F32, 32, None)
    assert cr.convrot_workspace_bytes(8192, 8192, 1) > 64 * MB
    assert f(*args(8192, 8192)) == EWS                  # beyond the static buffer
    assert f(*args(8, 256, G=2)) == EUNSUP
    assert f(*args(8, 256, a=0.0)) == EINVAL
    assert f(*args(8, 250)) == EUNSUP                   # K % 64
    assert f(*args(8, 256, Y=BASE + 384 * MB)) == EOVL  # Y on the weights
    assert f(*args(0, 256)) == OK                       # nothing to do


def test_build_refuses_register_spills():
    """The build reads hipcc's per-kernel resource report and refuses any
    kernel that spills registers (checked here on report text of both kinds)."""
    from int8_hadamard_rotated_amd import _build
    clean = ("x.hip:1:1: remark: Function Name: kern_a [-Rpass-analysis=kernel-resource-usage]\n"
             "x.hip:1:1: remark:     VGPRs: 103 [-Rpass-analysis=kernel-resource-usage]\n"
             "x.hip:1:1: remark:     SGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]\n"
             "x.hip:1:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]\n")
    spilling = clean + ("x.hip:9:1: remark: Function Name: kern_b [-Rpass-analysis=kernel-resource-usage]\n"
                        "x.hip:9:1: remark:     SGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]\n"
                        "x.hip:9:1: remark:     VGPRs Spill: 12 [-Rpass-analysis=kernel-resource-usage]\n")
    assert _build.register_spills(clean) == []
    assert _build.register_spills(spilling) == ["kern_b: VGPRs spill 12"]
    assert "-Rpass-analysis=kernel-resource-usage" in _build.RESOURCE_REMARKS
