"""MI355X (gfx950) INT8 convrot linear: Python binding over libconvrot.so.

Every entry point has the name and meaning of its C counterpart in
``include/convrot.h``; this module only marshals torch tensors (device
pointers) and the current HIP stream into those calls and raises on a
non-zero status.  All computation happens in the library's HIP kernels; there
is no fallback: if the library is not built, every call raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(_HERE, "libconvrot.so")

OK, EINVAL, EUNSUPPORTED, EOVERFLOW, EOVERLAP, EWORKSPACE, EHIP = 0, -1, -2, -3, -4, -5, -6
F32, BF16 = 0, 1
PRE_NONE, PRE_MODULATE, PRE_RMSNORM_MODULATE, PRE_GATED_ACT, PRE_NORM_MUL = 0, 1, 2, 3, 4
ACT_SILU, ACT_SIGMOID = 1, 2
POST_NONE, POST_GATED_RESIDUAL = 0, 1
MAX_LINEARS = 16

_lib = None


class ConvrotError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status} ({convrot_status_string(status)})")


class LinearDesc(ctypes.Structure):
    """Mirror of convrot_linear_desc."""
    _fields_ = [
        ("Qw", ctypes.c_void_p),
        ("s_w", ctypes.c_void_p),
        ("bias", ctypes.c_void_p),
        ("N", ctypes.c_int64),
        ("input_scale", ctypes.c_float),
        ("Y", ctypes.c_void_p),
        ("y_dtype", ctypes.c_int),
        ("ldy", ctypes.c_int64),
        ("Qx", ctypes.c_void_p),
        ("s_x", ctypes.c_void_p),
    ]


class PreDesc(ctypes.Structure):
    """Mirror of convrot_pre."""
    _fields_ = [
        ("kind", ctypes.c_int),
        ("scale", ctypes.c_void_p),
        ("shift", ctypes.c_void_p),
        ("norm_weight", ctypes.c_void_p),
        ("eps", ctypes.c_float),
        ("up", ctypes.c_void_p),
        ("ld_up", ctypes.c_int64),
        ("act", ctypes.c_int),
    ]


class Modulate:
    """The Modulate producer (x + x * scale) + shift with per-channel float32
    device vectors of K elements; shift may be None."""

    def __init__(self, scale, shift=None):
        self.scale = scale
        self.shift = shift

    def desc(self) -> PreDesc:
        return PreDesc(PRE_MODULATE, self.scale.data_ptr(),
                       None if self.shift is None else self.shift.data_ptr(), None, 0.0)


class RMSNormModulate:
    """RMSNorm -> Mul(weight) -> Modulate ahead of the quantizer: eps, and
    float32 device vectors of K elements, each optional (weight None: no
    weight multiplication; scale None: no modulation; shift needs scale)."""

    def __init__(self, eps: float, weight=None, scale=None, shift=None):
        self.eps = float(eps)
        self.weight, self.scale, self.shift = weight, scale, shift

    def desc(self) -> PreDesc:
        ptr = lambda t: None if t is None else t.data_ptr()
        return PreDesc(PRE_RMSNORM_MODULATE, ptr(self.scale), ptr(self.shift), ptr(self.weight),
                       self.eps)


class NormMul:
    """Norm (mean and variance) -> Mul(weight) ahead of the quantizer: eps, and
    an optional float32 device weight of K elements (None: no multiplication)."""

    def __init__(self, eps: float, weight=None):
        self.eps = float(eps)
        self.weight = weight

    def desc(self) -> PreDesc:
        return PreDesc(PRE_NORM_MUL, None, None, None if self.weight is None else self.weight.data_ptr(),
                       self.eps)


class GatedAct:
    """fl(act(x) * up) ahead of the quantizer (act: ACT_SILU or ACT_SIGMOID);
    up is a device tensor of X's dtype with K columns in use (a packed
    [gate | up] tensor gives both halves as views)."""

    def __init__(self, up, act: int = ACT_SILU):
        self.up, self.act = up, act

    def desc(self) -> PreDesc:
        return PreDesc(PRE_GATED_ACT, None, None, None, 0.0, self.up.data_ptr(),
                       _row_stride(self.up), self.act)


class PostDesc(ctypes.Structure):
    """Mirror of convrot_post."""
    _fields_ = [
        ("kind", ctypes.c_int),
        ("scale", ctypes.c_float),
        ("gate", ctypes.c_void_p),
        ("residual", ctypes.c_void_p),
        ("ld_residual", ctypes.c_int64),
    ]


class GatedResidual:
    """The gated-residual epilogue: fl(fl(fl(y * scale) * gate) + residual);
    gate float32 [N], residual [M, N] (row-contiguous last dimension) in the
    output dtype; the residual may be the output tensor itself."""

    def __init__(self, gate, residual, scale: float = 1.0):
        self.gate = gate
        self.residual = residual
        self.scale = scale

    def desc(self) -> PostDesc:
        ld = _row_stride(self.residual) if self.residual.shape[0] > 0 else self.residual.shape[1]
        return PostDesc(POST_GATED_RESIDUAL, self.scale, self.gate.data_ptr(),
                        self.residual.data_ptr(), ld)


def _pre(pre):
    return None if pre is None else ctypes.byref(pre.desc())


def library(path: str = LIBRARY) -> ctypes.CDLL:
    """Load libconvrot.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with int8_hadamard_rotated_amd._build.build()"
                           " (or __graft_entry__.build()); there is no fallback path")
    # torch first: the library must bind the HIP runtime torch already holds
    # (its own copy); loaded first, it would bind the system copy, and
    # launches on torch's streams would then fail
    _torch()
    lib = ctypes.CDLL(path)
    i64, i32, f32, vp, sz = ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
    sigs = {
        "convrot_packed_bytes": (sz, [i64, i64]),
        "convrot_quantize_rows": (i32, [vp, i32, i64, i64, i64, i32, f32, vp, vp]),
        "convrot_quantize_rows_scales": (i32, [vp, i32, i64, i64, i64, i32, i32, vp, vp, vp]),
        "convrot_quantize_rows_pre": (i32, [vp, i32, i64, i64, i64, ctypes.POINTER(PreDesc), i32,
                                            f32, vp, vp]),
        "int8_linear": (i32, [vp, vp, i64, i64, vp, vp, vp, i64, f32, vp, i32, i64, vp]),
        "convrot_workspace_bytes": (sz, [i64, i64, i32]),
        "convrot_int8_linear": (i32, [vp, i32, i64, i64, i64, i32, f32, vp, vp, vp, i64, vp, i32,
                                      i64, vp, sz, vp]),
        "convrot_int8_linear_noalloc": (i32, [vp, i32, i64, i64, i64, i32, f32, vp, vp, vp, i64, vp,
                                              i32, i64, vp]),
        "int8_linear_grouped": (i32, [vp, vp, i64, i64, i32, ctypes.POINTER(LinearDesc), vp]),
        "convrot_int8_linear_shared": (i32, [vp, i32, i64, i64, i64, i32, i32,
                                             ctypes.POINTER(LinearDesc), vp, sz, vp]),
        "convrot_int8_linear_shared_pre": (i32, [vp, i32, i64, i64, i64, ctypes.POINTER(PreDesc),
                                                 i32, i32, ctypes.POINTER(LinearDesc), vp, sz, vp]),
        "convrot_int8_gemm_i32": (i32, [vp, vp, i64, i64, i64, vp, vp]),
        "int4_linear": (i32, [vp, vp, i64, i64, vp, vp, vp, i64, f32, vp, i32, i64, vp]),
        "int8_linear_post": (i32, [vp, vp, i64, i64, vp, vp, vp, i64, f32,
                                   ctypes.POINTER(PostDesc), vp, i32, i64, vp]),
        "convrot_int4_gemm_i32": (i32, [vp, vp, i64, i64, i64, vp, vp]),
        "convrot_status_string": (ctypes.c_char_p, [i32]),
        "convrot_expf": (i32, [vp, vp, i64, vp]),
        "int8_swiglu_linear": (i32, [vp, vp, i64, i64, vp, vp, vp, vp, i64, f32, vp, i32, i64, vp]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


# ------------------------------------------------------------- marshalling

def _torch():
    import torch
    return torch


def _stream(stream, t):
    """The HIP stream to launch on: the given one, else torch's current
    stream on the device of tensor t."""
    if t.device.type != "cuda":
        raise ValueError(f"expected tensors in GPU memory, got one on {t.device}")
    if stream is None:
        return ctypes.c_void_p(_torch()._C._cuda_getCurrentRawStream(t.device.index))
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"expected float32 or bfloat16, got {t.dtype}")


def _torch_dtype(code: int):
    torch = _torch()
    return {F32: torch.float32, BF16: torch.bfloat16}[code]


def _row_stride(t) -> int:
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("expected a 2-D tensor with a contiguous last dimension")
    return t.stride(0)


def _check(fn: str, status: int):
    if status != OK:
        raise ConvrotError(fn, status)


# -------------------------------------------------------------- the entries

def convrot_status_string(status: int) -> str:
    return library().convrot_status_string(status).decode()


def convrot_packed_bytes(M: int, K: int) -> int:
    return int(library().convrot_packed_bytes(M, K))


def convrot_workspace_bytes(M: int, K: int, n_packed: int) -> int:
    return int(library().convrot_workspace_bytes(M, K, n_packed))


def packed_parts(packed, M: int, K: int):
    """Views of a packed tensor: (codes int8 [M_pad, K], scales float32 [M_pad])."""
    torch = _torch()
    m_pad = (M + 3) // 4 * 4
    q = packed[: m_pad * K].view(torch.int8).view(m_pad, K)
    s = packed[m_pad * K: m_pad * K + 4 * m_pad].view(torch.float32)
    return q, s


def convrot_quantize_rows(X, group_size: int, input_scale: float = 1.0, packed=None,
                          K: int | None = None, stream=None):
    """Rotate, quantize and pack the rows of X (first K columns); returns the
    packed uint8 tensor (allocated if not given)."""
    torch = _torch()
    M = X.shape[0]
    ldx = _row_stride(X) if M > 0 else X.shape[1]
    K = X.shape[1] if K is None else K
    if packed is None:
        packed = torch.empty(convrot_packed_bytes(M, K), dtype=torch.uint8, device=X.device)
    rc = library().convrot_quantize_rows(_ptr(X), _dtype_code(X), M, K, ldx, group_size,
                                         ctypes.c_float(input_scale), _ptr(packed), _stream(stream, X))
    _check("convrot_quantize_rows", rc)
    return packed


def convrot_quantize_rows_scales(X, group_size: int, input_scales, packed=None, stream=None):
    """convrot_quantize_rows for several input scales of the same X in one
    call; returns the packed tensors (allocated where ``packed`` is None)."""
    torch = _torch()
    M, K = X.shape
    ldx = _row_stride(X) if M > 0 else K
    n = len(input_scales)
    if packed is None:
        packed = [torch.empty(convrot_packed_bytes(M, K), dtype=torch.uint8, device=X.device)
                  for _ in range(n)]
    scales = (ctypes.c_float * max(n, 1))(*[float(a) for a in input_scales])
    ptrs = (ctypes.c_void_p * max(n, 1))(*[_ptr(p) for p in packed])
    rc = library().convrot_quantize_rows_scales(_ptr(X), _dtype_code(X), M, K, ldx, group_size, n,
                                                scales, ptrs, _stream(stream, X))
    _check("convrot_quantize_rows_scales", rc)
    return packed


def convrot_quantize_rows_pre(X, pre, group_size: int, input_scale: float = 1.0, packed=None,
                              K: int | None = None, stream=None):
    """convrot_quantize_rows with a producer (a Modulate, or None) applied to
    each element before the input scale and the rotation."""
    torch = _torch()
    M = X.shape[0]
    ldx = _row_stride(X) if M > 0 else X.shape[1]
    K = X.shape[1] if K is None else K
    if packed is None:
        packed = torch.empty(convrot_packed_bytes(M, K), dtype=torch.uint8, device=X.device)
    rc = library().convrot_quantize_rows_pre(_ptr(X), _dtype_code(X), M, K, ldx, _pre(pre),
                                             group_size, ctypes.c_float(input_scale), _ptr(packed),
                                             _stream(stream, X))
    _check("convrot_quantize_rows_pre", rc)
    return packed


def int8_linear(Qx, s_x, Qw, s_w=None, bias=None, input_scale: float = 1.0, Y=None,
                y_dtype: int = F32, M: int | None = None, stream=None):
    """Y = reconstruction of Q_x Q_w^T (Qx [M, K] int8 rows, s_x [M])."""
    torch = _torch()
    M = Qx.shape[0] if M is None else M
    K = Qx.shape[1]
    N = Qw.shape[0]
    if Y is None:
        Y = torch.empty((M, N), dtype=_torch_dtype(y_dtype), device=Qw.device)
    ldy = _row_stride(Y) if M > 0 and N > 0 else max(N, 1)
    rc = library().int8_linear(_ptr(Qx), _ptr(s_x), M, K, _ptr(Qw), _ptr(s_w), _ptr(bias), N,
                               ctypes.c_float(input_scale), _ptr(Y), _dtype_code(Y), ldy,
                               _stream(stream, Y))
    _check("int8_linear", rc)
    return Y


def int8_linear_post(Qx, s_x, Qw, s_w=None, bias=None, input_scale: float = 1.0, post=None,
                     Y=None, y_dtype: int = F32, M: int | None = None, stream=None):
    """int8_linear followed by an epilogue (a GatedResidual, or None)."""
    torch = _torch()
    M = Qx.shape[0] if M is None else M
    K = Qx.shape[1]
    N = Qw.shape[0]
    if Y is None:
        Y = torch.empty((M, N), dtype=_torch_dtype(y_dtype), device=Qw.device)
    ldy = _row_stride(Y) if M > 0 and N > 0 else max(N, 1)
    d = None if post is None else ctypes.byref(post.desc())
    rc = library().int8_linear_post(_ptr(Qx), _ptr(s_x), M, K, _ptr(Qw), _ptr(s_w), _ptr(bias), N,
                                    ctypes.c_float(input_scale), d, _ptr(Y), _dtype_code(Y), ldy,
                                    _stream(stream, Y))
    _check("int8_linear_post", rc)
    return Y


def int4_linear(Qx, s_x, W4, s_w=None, bias=None, input_scale: float = 1.0, Y=None,
                y_dtype: int = F32, M: int | None = None, stream=None):
    """int8_linear with convrot_w4a4 weights W4 (uint8 [N, K/2], two signed
    4-bit values per byte, low nibble first)."""
    torch = _torch()
    M = Qx.shape[0] if M is None else M
    K = Qx.shape[1]
    N = W4.shape[0]
    if Y is None:
        Y = torch.empty((M, N), dtype=_torch_dtype(y_dtype), device=W4.device)
    ldy = _row_stride(Y) if M > 0 and N > 0 else max(N, 1)
    rc = library().int4_linear(_ptr(Qx), _ptr(s_x), M, K, _ptr(W4), _ptr(s_w), _ptr(bias), N,
                               ctypes.c_float(input_scale), _ptr(Y), _dtype_code(Y), ldy,
                               _stream(stream, Y))
    _check("int4_linear", rc)
    return Y


def convrot_int4_gemm_i32(Qx, W4, A=None, M: int | None = None, stream=None):
    torch = _torch()
    M = Qx.shape[0] if M is None else M
    K = Qx.shape[1]
    N = W4.shape[0]
    if A is None:
        A = torch.empty((M, N), dtype=torch.int32, device=W4.device)
    rc = library().convrot_int4_gemm_i32(_ptr(Qx), _ptr(W4), M, K, N, _ptr(A), _stream(stream, A))
    _check("convrot_int4_gemm_i32", rc)
    return A


def int8_swiglu_linear(Qx, s_x, Qw_gate, s_w_gate, Qw_up, s_w_up, input_scale: float = 1.0,
                       Y=None, y_dtype: int = F32, M: int | None = None, stream=None):
    """Y = silu(gate reconstruction) * up reconstruction on one packed input."""
    torch = _torch()
    M = Qx.shape[0] if M is None else M
    K = Qx.shape[1]
    N = Qw_gate.shape[0]
    if Y is None:
        Y = torch.empty((M, N), dtype=_torch_dtype(y_dtype), device=Qw_gate.device)
    ldy = _row_stride(Y) if M > 0 and N > 0 else max(N, 1)
    rc = library().int8_swiglu_linear(_ptr(Qx), _ptr(s_x), M, K, _ptr(Qw_gate), _ptr(s_w_gate),
                                      _ptr(Qw_up), _ptr(s_w_up), N, ctypes.c_float(input_scale),
                                      _ptr(Y), _dtype_code(Y), ldy, _stream(stream, Qw_gate))
    _check("int8_swiglu_linear", rc)
    return Y


def convrot_expf(x, y=None, stream=None):
    """Correctly rounded binary32 exp of a float32 device tensor (the gated
    activation's exp); y may be x."""
    torch = _torch()
    if y is None:
        y = torch.empty_like(x)
    rc = library().convrot_expf(_ptr(x), _ptr(y), x.numel(), _stream(stream, x))
    _check("convrot_expf", rc)
    return y


def convrot_int8_gemm_i32(Qx, Qw, A=None, M: int | None = None, stream=None):
    torch = _torch()
    M = Qx.shape[0] if M is None else M
    K = Qx.shape[1]
    N = Qw.shape[0]
    if A is None:
        A = torch.empty((M, N), dtype=torch.int32, device=Qw.device)
    rc = library().convrot_int8_gemm_i32(_ptr(Qx), _ptr(Qw), M, K, N, _ptr(A), _stream(stream, A))
    _check("convrot_int8_gemm_i32", rc)
    return A


def convrot_int8_linear(X, group_size: int, input_scale: float, Qw, s_w=None, bias=None, Y=None,
                        y_dtype: int = F32, workspace=None, stream=None):
    torch = _torch()
    M, K = X.shape
    N = Qw.shape[0]
    ldx = _row_stride(X) if M > 0 else K
    if Y is None:
        Y = torch.empty((M, N), dtype=_torch_dtype(y_dtype), device=Qw.device)
    ldy = _row_stride(Y) if M > 0 and N > 0 else max(N, 1)
    if workspace is None:
        workspace = torch.empty(max(convrot_workspace_bytes(M, K, 1), 1), dtype=torch.uint8,
                                device=X.device)
    rc = library().convrot_int8_linear(_ptr(X), _dtype_code(X), M, K, ldx, group_size,
                                       ctypes.c_float(input_scale), _ptr(Qw), _ptr(s_w), _ptr(bias),
                                       N, _ptr(Y), _dtype_code(Y), ldy, _ptr(workspace),
                                       workspace.numel(), _stream(stream, X))
    _check("convrot_int8_linear", rc)
    return Y


def _descs(M: int, linears, device):
    torch = _torch()
    n = len(linears)
    descs = (LinearDesc * max(n, 1))()
    outs = []
    for i, lin in enumerate(linears):
        Qw = lin["Qw"]
        N = Qw.shape[0]
        Y = lin.get("Y")
        if Y is None:
            Y = torch.empty((M, N), dtype=_torch_dtype(lin.get("y_dtype", F32)), device=device)
        outs.append(Y)
        descs[i].Qw = Qw.data_ptr()
        descs[i].s_w = lin["s_w"].data_ptr() if lin.get("s_w") is not None else None
        descs[i].bias = lin["bias"].data_ptr() if lin.get("bias") is not None else None
        descs[i].N = N
        descs[i].input_scale = float(lin.get("input_scale", 1.0))
        descs[i].Y = Y.data_ptr()
        descs[i].y_dtype = _dtype_code(Y)
        descs[i].ldy = _row_stride(Y) if M > 0 and N > 0 else max(N, 1)
        if lin.get("Qx") is not None:
            descs[i].Qx = lin["Qx"].data_ptr()
            descs[i].s_x = lin["s_x"].data_ptr()
    return descs, outs


def int8_linear_grouped(Qx, s_x, linears, M: int | None = None, stream=None):
    """Several linears on quantized inputs in one GEMM launch.  ``linears``:
    dicts with Qw, s_w, bias, input_scale (the divisor) and optionally Y /
    y_dtype, and Qx / s_x for a linear that reads its own quantized input
    instead of the call's.  Returns the outputs."""
    M = Qx.shape[0] if M is None else M
    K = Qx.shape[1]
    descs, outs = _descs(M, linears, Qx.device)
    rc = library().int8_linear_grouped(_ptr(Qx), _ptr(s_x), M, K, len(linears), descs,
                                       _stream(stream, Qx))
    _check("int8_linear_grouped", rc)
    return outs


def convrot_int8_linear_noalloc(X, group_size: int, input_scale: float, Qw, s_w=None, bias=None,
                                Y=None, y_dtype: int = F32, stream=None):
    """convrot_int8_linear with the packed tensor in the library's static
    device buffer (no workspace argument, no allocation by the call; Y is
    allocated here only when not given)."""
    torch = _torch()
    M, K = X.shape
    N = Qw.shape[0]
    ldx = _row_stride(X) if M > 0 else K
    if Y is None:
        Y = torch.empty((M, N), dtype=_torch_dtype(y_dtype), device=Qw.device)
    ldy = _row_stride(Y) if M > 0 and N > 0 else max(N, 1)
    rc = library().convrot_int8_linear_noalloc(_ptr(X), _dtype_code(X), M, K, ldx, group_size,
                                               ctypes.c_float(input_scale), _ptr(Qw), _ptr(s_w),
                                               _ptr(bias), N, _ptr(Y), _dtype_code(Y), ldy,
                                               _stream(stream, X))
    _check("convrot_int8_linear_noalloc", rc)
    return Y


def _shared(X, group_size: int, linears, workspace, stream, pre):
    torch = _torch()
    M, K = X.shape
    ldx = _row_stride(X) if M > 0 else K
    n = len(linears)
    descs = (LinearDesc * max(n, 1))()
    outs = []
    scales = []
    for i, lin in enumerate(linears):
        Qw = lin["Qw"]
        N = Qw.shape[0]
        Y = lin.get("Y")
        if Y is None:
            Y = torch.empty((M, N), dtype=_torch_dtype(lin.get("y_dtype", F32)), device=Qw.device)
        outs.append(Y)
        a = float(lin.get("input_scale", 1.0))
        if a not in scales:
            scales.append(a)
        descs[i].Qw = Qw.data_ptr()
        descs[i].s_w = lin["s_w"].data_ptr() if lin.get("s_w") is not None else None
        descs[i].bias = lin["bias"].data_ptr() if lin.get("bias") is not None else None
        descs[i].N = N
        descs[i].input_scale = a
        descs[i].Y = Y.data_ptr()
        descs[i].y_dtype = _dtype_code(Y)
        descs[i].ldy = _row_stride(Y) if M > 0 and N > 0 else max(N, 1)
    if workspace is None:
        workspace = torch.empty(max(convrot_workspace_bytes(M, K, len(scales)), 1),
                                dtype=torch.uint8, device=X.device)
    if pre is None:
        rc = library().convrot_int8_linear_shared(_ptr(X), _dtype_code(X), M, K, ldx, group_size,
                                                  n, descs, _ptr(workspace), workspace.numel(),
                                                  _stream(stream, X))
        _check("convrot_int8_linear_shared", rc)
    else:
        rc = library().convrot_int8_linear_shared_pre(_ptr(X), _dtype_code(X), M, K, ldx,
                                                      _pre(pre), group_size, n, descs,
                                                      _ptr(workspace), workspace.numel(),
                                                      _stream(stream, X))
        _check("convrot_int8_linear_shared_pre", rc)
    return outs


def convrot_int8_linear_shared(X, group_size: int, linears, workspace=None, stream=None):
    """``linears``: sequence of dicts with keys Qw, s_w, bias, input_scale and
    optionally Y / y_dtype.  Returns the list of outputs."""
    return _shared(X, group_size, linears, workspace, stream, None)


def convrot_int8_linear_shared_pre(X, pre, group_size: int, linears, workspace=None,
                                   stream=None):
    """convrot_int8_linear_shared with a producer (a Modulate) applied in every
    quantization pass."""
    return _shared(X, group_size, linears, workspace, stream, pre)
