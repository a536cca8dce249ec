"""CPU oracle for the INT8 convrot linear layer (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may use
this package.  The product library never imports it, and it never imports the
product library: they share no code.

``convrot_oracle.c`` holds the arithmetic (plain binary32, no contraction);
this module builds it with gcc and wraps it for numpy arrays.  ``fp64`` holds
the dense binary64 helpers (H4 as printed on the "INT8 Convrot Safetensors"
page, its Kronecker powers, the closed form) used to pin the oracle.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "convrot_oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")

OK, EINVAL, EUNSUPPORTED, EOVERFLOW = 0, -1, -2, -3
F32, BF16 = 0, 1
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
          "-shared", "-Wall", "-Wextra"]


def build(source: str = SOURCE, output: str = LIBRARY) -> str:
    """Compile the oracle with gcc (always recompiles)."""
    tmp = output + ".tmp"
    cmd = ["gcc", *CFLAGS, source, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.replace(tmp, output)
    return output


class OracleError(RuntimeError):
    pass


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(x: np.ndarray) -> int:
    if x.dtype == np.float32:
        return F32
    if x.dtype == np.uint16:
        return BF16
    raise TypeError(f"activation must be float32 or uint16 (bf16 bits), got {x.dtype}")


@dataclass
class Packed:
    """Packed runtime activation tensor: int8 [M_pad][K] then float [M_pad]."""
    raw: np.ndarray      # uint8 [packed_bytes]
    M: int
    K: int

    @property
    def M_pad(self) -> int:
        return (self.M + 3) // 4 * 4

    @property
    def q_all(self) -> np.ndarray:
        return self.raw[: self.M_pad * self.K].view(np.int8).reshape(self.M_pad, self.K)

    @property
    def q(self) -> np.ndarray:
        return self.q_all[: self.M]

    @property
    def s_all(self) -> np.ndarray:
        return self.raw[self.M_pad * self.K:].view(np.float32)

    @property
    def s(self) -> np.ndarray:
        return self.s_all[: self.M]


ACT_SILU, ACT_SIGMOID = 1, 2


class Oracle:
    """ctypes wrapper over a built oracle shared library."""

    def __init__(self, path: str = LIBRARY):
        if not os.path.exists(path) or (path == LIBRARY and
                                        os.path.getmtime(SOURCE) > os.path.getmtime(path)):
            build(output=path)
        self.path = path
        lib = ctypes.CDLL(path)
        i64, i32, f32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_void_p
        sig = {
            "oracle_packed_bytes": (i64, [i64, i64]),
            "oracle_rotate_rows_f32": (i32, [vp, i64, i64, i32, vp]),
            "oracle_rotate_rows_f64": (i32, [vp, i64, i64, i32, vp]),
            "oracle_quantize_rows": (i32, [vp, i32, i64, i64, i64, i32, f32, vp, i32]),
            "oracle_modulate_rows": (i32, [vp, i32, i64, i64, i64, vp, vp, vp, i32]),
            "oracle_rmsnorm_rows": (i32, [vp, i32, i64, i64, i64, f32, vp, vp, i32]),
            "oracle_norm_rows": (i32, [vp, i32, i64, i64, i64, f32, vp, vp, i32]),
            "oracle_expf": (f32, [f32]),
            "oracle_expf_array": (i32, [vp, vp, i64, i32]),
            "oracle_gated_act_rows": (i32, [vp, i32, i64, i64, i64, vp, i64, i32, vp, i32]),
            "oracle_unpack_int4": (i32, [vp, i64, i64, vp]),
            "oracle_gated_residual": (i32, [vp, i64, i64, f32, vp, vp, i32, i64, i32, vp, i64, i32]),
            "oracle_gemm_i32": (i32, [vp, vp, i64, i64, i64, vp, i32]),
            "oracle_epilogue": (i32, [vp, i64, i64, vp, vp, vp, f32, i32, vp, i64, i32]),
            "oracle_linear": (i32, [vp, i32, i64, i64, i64, i32, f32, vp, vp, vp, i64, vp, i32,
                                    i64, i32]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        self.lib = lib

    @staticmethod
    def _check(rc: int, what: str):
        if rc != OK:
            raise OracleError(f"{what} failed with status {rc}")

    def packed_bytes(self, M: int, K: int) -> int:
        return int(self.lib.oracle_packed_bytes(M, K))

    def rotate_rows(self, X: np.ndarray, G: int) -> np.ndarray:
        X = np.ascontiguousarray(X, dtype=np.float32)
        M, K = X.shape
        Y = np.empty_like(X)
        self._check(self.lib.oracle_rotate_rows_f32(_p(X), M, K, G, _p(Y)), "rotate_rows_f32")
        return Y

    def rotate_rows_f64(self, X: np.ndarray, G: int) -> np.ndarray:
        X = np.ascontiguousarray(X, dtype=np.float64)
        M, K = X.shape
        Y = np.empty_like(X)
        self._check(self.lib.oracle_rotate_rows_f64(_p(X), M, K, G, _p(Y)), "rotate_rows_f64")
        return Y

    def quantize_rows(self, X: np.ndarray, G: int, alpha: float = 1.0, K: int | None = None,
                      threads: int = 1) -> Packed:
        """Quantize the rows of X ([M, ldx] with the first K columns used)."""
        code = _dtype_code(X)
        X = np.ascontiguousarray(X)
        M, ldx = X.shape
        K = ldx if K is None else K
        # filled with a marker so that bytes the oracle fails to write show up
        raw = np.full(self.packed_bytes(M, K), 0xA5, dtype=np.uint8)
        rc = self.lib.oracle_quantize_rows(_p(X), code, M, K, ldx, G, ctypes.c_float(alpha),
                                           _p(raw), threads)
        self._check(rc, "quantize_rows")
        return Packed(raw, M, K)

    def modulate_rows(self, X: np.ndarray, scale: np.ndarray, shift=None, K: int | None = None,
                      threads: int = 1) -> np.ndarray:
        """The Modulate producer on the first K columns of X: binary32 [M, K]."""
        code = _dtype_code(X)
        X = np.ascontiguousarray(X)
        M, ldx = X.shape
        K = ldx if K is None else K
        sc = np.ascontiguousarray(scale, dtype=np.float32)
        sh = None if shift is None else np.ascontiguousarray(shift, dtype=np.float32)
        assert sc.shape == (K,) and (sh is None or sh.shape == (K,))
        Y = np.empty((M, K), dtype=np.float32)
        rc = self.lib.oracle_modulate_rows(_p(X), code, M, K, ldx, _p(sc),
                                           None if sh is None else _p(sh), _p(Y), threads)
        self._check(rc, "modulate_rows")
        return Y

    def rmsnorm_rows(self, X: np.ndarray, eps: float, weight=None, K: int | None = None,
                     threads: int = 1) -> np.ndarray:
        """RMSNorm -> Mul(weight) on the first K columns of X: binary32 [M, K]."""
        code = _dtype_code(X)
        X = np.ascontiguousarray(X)
        M, ldx = X.shape
        K = ldx if K is None else K
        w = None if weight is None else np.ascontiguousarray(weight, dtype=np.float32)
        assert w is None or w.shape == (K,)
        Y = np.empty((M, K), dtype=np.float32)
        rc = self.lib.oracle_rmsnorm_rows(_p(X), code, M, K, ldx, ctypes.c_float(eps),
                                          None if w is None else _p(w), _p(Y), threads)
        self._check(rc, "rmsnorm_rows")
        return Y

    def norm_rows(self, X: np.ndarray, eps: float, weight=None, K: int | None = None,
                  threads: int = 1) -> np.ndarray:
        """Norm (mean and variance) -> Mul(weight) on the first K columns of X:
        binary32 [M, K]."""
        code = _dtype_code(X)
        X = np.ascontiguousarray(X)
        M, ldx = X.shape
        K = ldx if K is None else K
        w = None if weight is None else np.ascontiguousarray(weight, dtype=np.float32)
        assert w is None or w.shape == (K,)
        Y = np.empty((M, K), dtype=np.float32)
        rc = self.lib.oracle_norm_rows(_p(X), code, M, K, ldx, ctypes.c_float(eps),
                                       None if w is None else _p(w), _p(Y), threads)
        self._check(rc, "norm_rows")
        return Y

    def expf(self, x: float) -> float:
        """exp rounded once to binary32 (the oracle's exp)."""
        return float(self.lib.oracle_expf(ctypes.c_float(x)))

    def expf_array(self, x: np.ndarray, threads: int = 1) -> np.ndarray:
        x = np.ascontiguousarray(x, dtype=np.float32)
        y = np.empty_like(x)
        self._check(self.lib.oracle_expf_array(_p(x), _p(y), x.size, threads), "expf_array")
        return y

    def gated_act_rows(self, X: np.ndarray, U: np.ndarray, act: int, K: int | None = None,
                       threads: int = 1) -> np.ndarray:
        """fl(act(X) * U) on the first K columns (act: ACT_SILU or ACT_SIGMOID);
        X and U share their dtype.  Returns binary32 [M, K]."""
        code = _dtype_code(X)
        assert _dtype_code(U) == code
        X = np.ascontiguousarray(X)
        U = np.ascontiguousarray(U)
        M, ldx = X.shape
        K = ldx if K is None else K
        assert U.shape[0] == M and U.shape[1] >= K
        Y = np.empty((M, K), dtype=np.float32)
        rc = self.lib.oracle_gated_act_rows(_p(X), code, M, K, ldx, _p(U), U.shape[1], act, _p(Y),
                                            threads)
        self._check(rc, "gated_act_rows")
        return Y

    def unpack_int4(self, W4: np.ndarray, K: int) -> np.ndarray:
        """convrot_w4a4 packed weights [N, K/2] uint8 -> int8 [N, K]."""
        W4 = np.ascontiguousarray(W4, dtype=np.uint8)
        N = W4.shape[0]
        assert W4.shape == (N, K // 2)
        Qw = np.empty((N, K), dtype=np.int8)
        self._check(self.lib.oracle_unpack_int4(_p(W4), N, K, _p(Qw)), "unpack_int4")
        return Qw

    def weight_prep(self, W: np.ndarray, G: int, threads: int = 1):
        """Offline weight rotation + per-output-row quantization -> (Q_w, s_w)."""
        p = self.quantize_rows(np.ascontiguousarray(W, dtype=np.float32), G, 1.0, threads=threads)
        return np.ascontiguousarray(p.q), np.ascontiguousarray(p.s)

    def gemm_i32(self, Qx: np.ndarray, Qw: np.ndarray, threads: int = 1) -> np.ndarray:
        Qx = np.ascontiguousarray(Qx, dtype=np.int8)
        Qw = np.ascontiguousarray(Qw, dtype=np.int8)
        M, K = Qx.shape
        N, K2 = Qw.shape
        assert K == K2
        A = np.empty((M, N), dtype=np.int32)
        self._check(self.lib.oracle_gemm_i32(_p(Qx), _p(Qw), M, K, N, _p(A), threads), "gemm_i32")
        return A

    def epilogue(self, A: np.ndarray, s_x: np.ndarray, s_w, bias, alpha: float = 1.0,
                 y_dtype: int = F32, threads: int = 1) -> np.ndarray:
        A = np.ascontiguousarray(A, dtype=np.int32)
        M, N = A.shape
        s_x = np.ascontiguousarray(s_x, dtype=np.float32)
        sw = None if s_w is None else np.ascontiguousarray(s_w, dtype=np.float32)
        b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
        Y = np.empty((M, N), dtype=np.float32 if y_dtype == F32 else np.uint16)
        rc = self.lib.oracle_epilogue(_p(A), M, N, _p(s_x), None if sw is None else _p(sw),
                                      None if b is None else _p(b), ctypes.c_float(alpha),
                                      y_dtype, _p(Y), N, threads)
        self._check(rc, "epilogue")
        return Y

    def gated_residual(self, Y: np.ndarray, gate: np.ndarray, R: np.ndarray, scale: float = 1.0,
                       z_dtype: int = F32, threads: int = 1) -> np.ndarray:
        """The gated-residual epilogue on a binary32 reconstruction Y [M, N]:
        residual R [M, N] (float32 or bf16 bits), per-channel gate [N]."""
        Y = np.ascontiguousarray(Y, dtype=np.float32)
        M, N = Y.shape
        g = np.ascontiguousarray(gate, dtype=np.float32)
        code = _dtype_code(R)
        R = np.ascontiguousarray(R)
        assert g.shape == (N,) and R.shape == (M, N)
        Z = np.empty((M, N), dtype=np.float32 if z_dtype == F32 else np.uint16)
        rc = self.lib.oracle_gated_residual(_p(Y), M, N, ctypes.c_float(scale), _p(g), _p(R), code, N,
                                            z_dtype, _p(Z), N, threads)
        self._check(rc, "gated_residual")
        return Z

    def linear(self, X: np.ndarray, G: int, Qw: np.ndarray, s_w, bias, alpha: float = 1.0,
               y_dtype: int = F32, threads: int = 1) -> np.ndarray:
        code = _dtype_code(X)
        X = np.ascontiguousarray(X)
        M, K = X.shape
        Qw = np.ascontiguousarray(Qw, dtype=np.int8)
        N = Qw.shape[0]
        sw = None if s_w is None else np.ascontiguousarray(s_w, dtype=np.float32)
        b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
        Y = np.empty((M, N), dtype=np.float32 if y_dtype == F32 else np.uint16)
        rc = self.lib.oracle_linear(_p(X), code, M, K, K, G, ctypes.c_float(alpha), _p(Qw),
                                    None if sw is None else _p(sw), None if b is None else _p(b),
                                    N, _p(Y), y_dtype, N, threads)
        self._check(rc, "linear")
        return Y


_DEFAULT = None


def get() -> Oracle:
    """The oracle built from this directory's source (built on first use)."""
    global _DEFAULT
    if _DEFAULT is None:
        _DEFAULT = Oracle()
    return _DEFAULT
