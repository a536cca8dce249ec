"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError
when the oracle disagrees with something independent of it: the H4 entries
printed on the "INT8 Convrot Safetensors" page, numpy's Kronecker products and
binary64 matmuls, closed forms, exact invariants, exact rational arithmetic
with binary32 rounding written from the IEEE-754 definition, and brute-force
integer loops.  The mutation test runs the same functions against broken
copies of the oracle to show that each plausible mistake fails at least one.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np

import oracle as oracle_pkg
from oracle import fp64
import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
U32 = 2.0 ** -24            # unit roundoff of binary32


def load_h4_golden() -> np.ndarray:
    rows = []
    with open(os.path.join(GOLDEN, "h4.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([float(v) for v in line.split()])
    return np.array(rows) / 2.0


def load_tie_row() -> tuple[np.ndarray, np.ndarray]:
    vals, codes = [], []
    with open(os.path.join(GOLDEN, "tie_row_g16.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                v, c = line.split()
                vals.append(float(v))
                codes.append(int(c))
    return np.array(vals, dtype=np.float32), np.array(codes, dtype=np.int8)


# ---------------------------------------------------------------- exact IEEE

def rne_f32(q: Fraction) -> Fraction:
    """Round an exact rational to the nearest binary32 value, ties to even.

    Written from the definition: 24-bit significands for normal numbers,
    fixed 2^-149 spacing below 2^-126.  Overflow is outside the tests' range.
    """
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    # now 2^e <= a < 2^(e+1)
    e = max(e, -126)
    ulp = Fraction(2) ** (e - 23)
    k = a / ulp
    fl = k.numerator // k.denominator
    rem = k - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * ulp


def round_half_even(q: Fraction) -> int:
    fl = q.numerator // q.denominator
    rem = q - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return int(fl)


def F(x) -> Fraction:
    return Fraction(float(x))


def F_out(x) -> Fraction:
    """An oracle output as an exact rational; a non-finite one fails the pin."""
    assert np.isfinite(x), f"non-finite output {x}"
    return Fraction(float(x))


# ----------------------------------------------------------------- the pins

def pin_h4_entries(o):
    """The G=4 rotation of the unit vectors is the page's H4, exactly."""
    h4 = load_h4_golden()
    assert np.array_equal(fp64.H4, h4), "fp64 helper H4 differs from the page's matrix"
    R = o.rotate_rows(np.eye(4, dtype=np.float32), 4).astype(np.float64)
    assert np.array_equal(R, h4), f"oracle G=4 rotation is not H4:\n{R}"


def pin_kronecker_power(o):
    """For G = 16, 64, 256 the butterfly equals the Kronecker power, exactly."""
    for G in (16, 64, 256):
        Rk = fp64.kron_power(G, load_h4_golden())
        assert np.array_equal(Rk, fp64.closed_form(G)), f"kron chain != closed form, G={G}"
        R = o.rotate_rows(np.eye(G, dtype=np.float32), G).astype(np.float64)
        assert np.array_equal(R, Rk), f"oracle rotation != H4^(x)n for G={G}"


def pin_orthogonal_symmetric(o):
    """R R^T = I and R = R^T (exact); applying the oracle's rotation twice is
    the identity on small-integer rows (all intermediates are dyadic)."""
    for G in (4, 16, 256):
        R = fp64.kron_power(G, load_h4_golden())
        assert np.array_equal(R @ R.T, np.eye(G)), f"R R^T != I for G={G}"
        assert np.array_equal(R, R.T), f"R not symmetric for G={G}"
    rng = np.random.default_rng(11)
    for G in (4, 16, 64, 256):
        X = rng.integers(-8, 9, size=(6, 2 * G)).astype(np.float32)
        Y = o.rotate_rows(o.rotate_rows(X, G), G)
        assert np.array_equal(X, Y), f"rotation is not an involution, G={G}"


def pin_constant_group(o):
    """Regularity: a constant group rotates to itself, bit for bit."""
    rng = np.random.default_rng(12)
    for G in (4, 16, 64, 256):
        c = (rng.standard_normal(8) * 10).astype(np.float32)
        X = np.repeat(c, G).reshape(2, 4 * G)
        assert np.array_equal(o.rotate_rows(X, G), X), f"constant groups moved, G={G}"


def pin_one_hot(o):
    """An isolated value v is spread to magnitude v / sqrt(G) on its whole group
    (the rotation's stated purpose); the other groups stay zero."""
    for G, v in ((16, 20.0), (256, 20.0), (256, -30.0)):
        X = np.zeros((1, 2 * G), dtype=np.float32)
        X[0, G + 5] = v
        Y = o.rotate_rows(X, G)
        assert np.all(Y[0, :G] == 0)
        assert np.all(np.abs(Y[0, G:]) == np.float32(abs(v) / math.sqrt(G))), f"G={G}"
        assert np.array_equal(np.sign(Y[0, G:]) * np.sign(v),
                              np.sign(fp64.closed_form(G)[5])), f"sign pattern, G={G}"


def pin_fp64_error_bound(o):
    """Binary32 butterfly vs the dense binary64 R x: per group,
    ||y - R x||_2 <= 5 n u ||x||_2 (first-order bound; each stage is orthogonal)."""
    rng = np.random.default_rng(13)
    for G in (16, 64, 256):
        n = fp64.log4(G)
        X = workloads.gaussian_activations(rng, 16, 4 * G, 0.01, 30.0, workloads.F32)
        Y = o.rotate_rows(X, G).astype(np.float64)
        Yd = fp64.rotate_dense(X, G)
        err = np.linalg.norm((Y - Yd).reshape(-1, G), axis=1)
        bound = 5 * n * U32 * np.linalg.norm(X.astype(np.float64).reshape(-1, G), axis=1)
        assert np.all(err <= bound * 1.0001), f"G={G}: max err/bound {np.max(err / bound)}"
        # and it is a genuine rounding error, not zero-by-accident
        assert np.any(err > 0)


def pin_fp64_identity(o):
    """X_rot W_rot^T = X W^T in binary64 without quantization (the page's
    identity, from R R^T = I); the binary64 butterfly also equals dense X R."""
    rng = np.random.default_rng(14)
    for (M, K, N, G) in ((8, 256, 32, 16), (64, 3072, 3072, 256)):
        X = rng.standard_normal((M, K))
        W = rng.standard_normal((N, K)) * 0.02
        Xr = o.rotate_rows_f64(X, G)
        Wr = o.rotate_rows_f64(W, G)
        ref = X @ W.T
        rel = np.max(np.abs(Xr @ Wr.T - ref)) / np.max(np.abs(ref))
        assert rel <= 1e-12, f"identity violated ({M},{K},{N},G={G}): {rel}"
        d = np.max(np.abs(Xr - fp64.rotate_dense(X, G))) / np.max(np.abs(X))
        assert d <= 1e-14, f"binary64 butterfly != dense R: {d}"


def pin_quantizer_invariants(o):
    """Per row: the scale comes from the max over the WHOLE rotated row;
    codes lie in [-127, 127] and reach +-127; |y - s q| <= s/2 (+ rounding)."""
    rng = np.random.default_rng(15)
    for G, K in ((16, 256), (256, 3072), (64, 512)):
        X = workloads.gaussian_activations(rng, 33, K, 0.005, 30.0, workloads.F32)
        X[7] = 0.0
        p = o.quantize_rows(X, G)
        Y = o.rotate_rows(X, G)
        q, s = p.q.astype(np.int32), p.s
        amax = np.max(np.abs(Y), axis=1)
        assert np.array_equal(s, (amax / np.float32(127)).astype(np.float32)), "row scale"
        assert np.all(np.abs(q) <= 127)
        nz = amax > 0
        assert np.all(np.max(np.abs(q[nz]), axis=1) == 127)
        assert np.all(q[~nz] == 0) and np.all(s[~nz] == 0)
        s64 = s.astype(np.float64)[:, None]
        err = np.abs(Y.astype(np.float64) - s64 * q)
        assert np.all(err <= s64 * (0.5 + 127 * 4 * U32)), "quantization error above s/2"


def pin_quantizer_exact(o):
    """Codes and scales against exact rational arithmetic with binary32
    rounding at each step: s = fl(m / 127), inv = fl(127 / m),
    q = round_half_even(fl(y * inv)) (readings: reciprocal, ties to even)."""
    rng = np.random.default_rng(16)
    X = workloads.gaussian_activations(rng, 4, 256, 0.01, 20.0, workloads.F32)
    p = o.quantize_rows(X, 16)
    Y = o.rotate_rows(X, 16)
    for r in range(4):
        m = F(np.max(np.abs(Y[r])))
        assert F(p.s[r]) == rne_f32(m / 127), f"scale row {r}"
        inv = rne_f32(Fraction(127) / m)
        for i in range(256):
            want = round_half_even(rne_f32(F(Y[r, i]) * inv))
            want = max(-127, min(127, want))
            assert int(p.q[r, i]) == want, f"code ({r},{i}): {p.q[r, i]} vs {want}"


def pin_quantizer_group_one(o):
    """G = 1 (4^0) is the identity rotation: codes and scales of the widened
    input itself against exact rational arithmetic with binary32 rounding,
    for binary32 and bf16 rows, and the same packed bytes as rotating by
    nothing (the oracle's rotation at G = 1 returns its input)."""
    rng = np.random.default_rng(26)
    X = workloads.gaussian_activations(rng, 3, 192, 0.02, 20.0, workloads.F32)
    Xb = workloads.f32_to_bf16_bits(X)
    for src, xw in ((X, X), (Xb, workloads.bf16_bits_to_f32(Xb))):
        p = o.quantize_rows(src, 1)
        for r in range(3):
            m = F(np.max(np.abs(xw[r])))
            assert F(p.s[r]) == rne_f32(m / 127), f"G=1 scale row {r}"
            inv = rne_f32(Fraction(127) / m)
            for i in range(192):
                want = max(-127, min(127, round_half_even(rne_f32(F(xw[r, i]) * inv))))
                assert int(p.q[r, i]) == want, f"G=1 code ({r},{i}): {p.q[r, i]} vs {want}"
    assert np.array_equal(o.rotate_rows(X, 1), X)


def pin_tie_row(o):
    """Rounding rule, pinned on constructed ties (golden/tie_row_g16.txt)."""
    vals, codes = load_tie_row()
    X = np.repeat(vals, 16).reshape(1, 256).astype(np.float32)
    p = o.quantize_rows(X, 16)
    assert p.s[0] == np.float32(1.0)
    assert np.array_equal(p.q[0], np.repeat(codes, 16)), f"{p.q[0][::16]} vs {codes}"
    # the same row in bf16 (every value is exactly representable)
    pb = o.quantize_rows(workloads.f32_to_bf16_bits(X), 16)
    assert np.array_equal(pb.raw, p.raw)


def pin_packed_layout(o):
    """int8 [M_pad][K] codes, zero pad rows, then float [M_pad] scales (pad 0);
    each row is quantized independently; the row stride is honoured."""
    rng = np.random.default_rng(17)
    M, K, G = 5, 256, 16
    wide = workloads.gaussian_activations(rng, M, K + 64, 0.0, 1.0, workloads.F32)
    X = np.ascontiguousarray(wide[:, :K])
    p = o.quantize_rows(X, G)
    assert p.raw.size == 8 * K + 4 * 8 == o.packed_bytes(M, K)
    assert np.all(p.q_all[M:] == 0) and np.all(p.s_all[M:] == 0)
    for r in range(M):
        one = o.quantize_rows(X[r:r + 1], G)
        assert np.array_equal(one.q[0], p.q[r]) and one.s[0] == p.s[r], f"row {r}"
    strided = o.quantize_rows(wide, G, K=K)
    assert np.array_equal(strided.raw, p.raw), "row stride"


def pin_bf16_input(o):
    """bf16 input quantizes exactly like its (exact) fp32 widening."""
    rng = np.random.default_rng(18)
    Xb = workloads.gaussian_activations(rng, 12, 1024, 0.005, 30.0, workloads.BF16)
    Xf = workloads.bf16_bits_to_f32(Xb)
    for G in (4, 64, 256):
        assert np.array_equal(o.quantize_rows(Xb, G).raw, o.quantize_rows(Xf, G).raw), f"G={G}"


def pin_input_scale(o):
    """alpha pre-multiplies X once (binary32), and for alpha = 2^k the codes are
    unchanged, the scale is scaled exactly and the output is bit-identical."""
    rng = np.random.default_rng(19)
    M, K, N, G = 9, 512, 40, 64
    X = workloads.gaussian_activations(rng, M, K, 0.01, 20.0, workloads.F32)
    W, b = workloads.gaussian_weights(rng, N, K)
    Qw, sw = o.weight_prep(W, G)
    p1 = o.quantize_rows(X, G, 1.0)
    for a in (0.5, 0.25, 4.0):
        pa = o.quantize_rows(X, G, a)
        assert np.array_equal(pa.q, p1.q), f"codes change at alpha={a}"
        assert np.array_equal(pa.s, (p1.s * np.float32(a)).astype(np.float32)), f"alpha={a}"
        assert np.array_equal(o.linear(X, G, Qw, sw, b, a), o.linear(X, G, Qw, sw, b, 1.0))
    a = 0.3
    pa = o.quantize_rows(X, G, a)
    pre = (X * np.float32(a)).astype(np.float32)
    assert np.array_equal(pa.raw, o.quantize_rows(pre, G, 1.0).raw), "pre-scale"


def pin_gemm_bruteforce(o):
    """int32 contraction vs pure-Python integer loops (non-square, so a
    transposed operand cannot pass)."""
    rng = np.random.default_rng(20)
    M, K, N = 8, 256, 32
    Qx = workloads.random_codes(rng, (M, K))
    Qw = workloads.random_codes(rng, (N, K))
    Qx[0, :] = 127
    Qw[0, :] = -127
    A = o.gemm_i32(Qx, Qw)
    xl, wl = Qx.tolist(), Qw.tolist()
    for r in range(M):
        for c in range(N):
            want = sum(a * b for a, b in zip(xl[r], wl[c]))
            assert int(A[r, c]) == want, f"A[{r},{c}] = {A[r, c]} vs {want}"
    # the int32 range guard
    big = np.full((1, 133144), 127, dtype=np.int8)
    assert int(o.gemm_i32(big, big)[0, 0]) == 133144 * 127 * 127
    bigger = np.full((1, 133145), 127, dtype=np.int8)
    try:
        o.gemm_i32(bigger, bigger)
    except oracle_pkg.OracleError:
        pass
    else:
        raise AssertionError("int32 overflow not reported")


def pin_epilogue_exact(o):
    """Y = fl(fl(fl(fl(fl(A) * s_x) * s_w) / alpha) + b): exact rationals with
    binary32 rounding per step, in the order the pages state."""
    rng = np.random.default_rng(21)
    M, N = 6, 40
    A = rng.integers(-40_000_000, 40_000_000, size=(M, N)).astype(np.int32)
    A[0, :4] = [0, 1, -1, 2 ** 24 + 1]
    sx = workloads.random_scales(rng, M, 1e-3, 1e-1)
    sw = workloads.random_scales(rng, N, 1e-4, 1e-2)
    b = (rng.standard_normal(N) * 0.1).astype(np.float32)
    for alpha in (1.0, 0.3):
        Y = o.epilogue(A, sx, sw, b, alpha)
        for r in range(M):
            for c in range(N):
                t = rne_f32(Fraction(int(A[r, c])))
                t = rne_f32(t * F(sx[r]))
                t = rne_f32(t * F(sw[c]))
                if alpha != 1.0:
                    t = rne_f32(t / F(np.float32(alpha)))
                t = rne_f32(t + F(b[c]))
                assert F(Y[r, c]) == t, f"Y[{r},{c}] alpha={alpha}"
    # nullable scale and bias
    Y = o.epilogue(A, sx, None, None)
    assert F(Y[1, 3]) == rne_f32(rne_f32(Fraction(int(A[1, 3]))) * F(sx[1]))


def pin_epilogue_fp64_bound(o):
    """Independent of the order: |Y - Y64| <= 4u |A s_x s_w / alpha| + u |Y64|."""
    rng = np.random.default_rng(22)
    M, N = 16, 64
    A = rng.integers(-50_000_000, 50_000_000, size=(M, N)).astype(np.int32)
    sx = workloads.random_scales(rng, M)
    sw = workloads.random_scales(rng, N, 1e-4, 1e-2)
    b = (rng.standard_normal(N) * 0.1).astype(np.float32)
    for alpha in (1.0, 0.5, 0.3):
        Y = o.epilogue(A, sx, sw, b, alpha).astype(np.float64)
        a32 = np.float64(np.float32(alpha))
        P = A.astype(np.float64) * sx.astype(np.float64)[:, None] * sw.astype(np.float64)[None] / a32
        Y64 = P + b.astype(np.float64)[None]
        assert np.all(np.abs(Y - Y64) <= 4.01 * U32 * np.abs(P) + 1.01 * U32 * np.abs(Y64))


def pin_bf16_output(o):
    """bf16 output is the fp32 result rounded to nearest, ties to even; exact
    bf16 ties are constructed (257 lies halfway between 256 and 258)."""
    A = np.array([[257, 259, 261, 263, -257, -259, 1, 65535, 65537, 12345678]], dtype=np.int32)
    one = np.ones(1, dtype=np.float32)
    Yb = o.epilogue(A, one, None, None, 1.0, oracle_pkg.BF16)
    Yf = workloads.bf16_bits_to_f32(Yb)[0]
    assert list(Yf[:6]) == [256.0, 260.0, 260.0, 264.0, -256.0, -260.0], Yf
    rng = np.random.default_rng(23)
    A = rng.integers(-2 ** 30, 2 ** 30, size=(8, 64)).astype(np.int32)
    sx = workloads.random_scales(rng, 8)
    Yf32 = o.epilogue(A, sx, None, None)
    Yb = o.epilogue(A, sx, None, None, 1.0, oracle_pkg.BF16)
    assert np.array_equal(Yb, workloads.f32_to_bf16_bits(Yf32))


def pin_zero_row(o):
    """An all-zero row has scale 0 and codes 0, so its output is the bias."""
    rng = np.random.default_rng(24)
    X = workloads.gaussian_activations(rng, 4, 256, 0.0, 1.0, workloads.F32)
    X[2] = 0.0
    W, b = workloads.gaussian_weights(rng, 16, 256)
    Qw, sw = o.weight_prep(W, 16)
    Y = o.linear(X, 16, Qw, sw, b)
    assert np.array_equal(Y[2], b)


def pin_rotation_reduces_error(o):
    """Sanity of the method's stated purpose (not a parity gate): on inputs
    with isolated outliers the G=256 rotation lowers the quantized output's
    error against binary64 X W^T + b compared with no rotation (G = 1)."""
    rng = np.random.default_rng(25)
    X = workloads.gaussian_activations(rng, 32, 1024, 0.005, 30.0, workloads.F32)
    W, b = workloads.gaussian_weights(rng, 64, 1024)
    ref = X.astype(np.float64) @ W.T.astype(np.float64) + b
    errs = {}
    for G in (1, 256):
        Qw, sw = o.weight_prep(W, G)
        Y = o.linear(X, G, Qw, sw, b)
        errs[G] = np.linalg.norm(Y - ref) / np.linalg.norm(ref)
    assert errs[256] < 0.7 * errs[1], errs


def pin_modulate_exact(o):
    """The Modulate producer against exact rational arithmetic with binary32
    rounding at each step: fl(fl(x + fl(x * scale)) + shift), the vectors
    indexed by column (page "ggml operator extensions", the Modulate
    operator); with and without the shift, for binary32 and bf16 rows."""
    rng = np.random.default_rng(41)
    M, K = 3, 64
    X = workloads.gaussian_activations(rng, M, K, 0.05, 20.0, workloads.F32)
    sc = (rng.standard_normal(K) * 0.7).astype(np.float32)
    sh = (rng.standard_normal(K) * 0.7).astype(np.float32)
    Xb = workloads.f32_to_bf16_bits(X)
    for src, xw in ((X, X), (Xb, workloads.bf16_bits_to_f32(Xb))):
        for shift in (sh, None):
            Y = o.modulate_rows(src, sc, shift)
            for r in range(M):
                for i in range(K):
                    x = F(xw[r, i])
                    t = rne_f32(x + rne_f32(x * F(sc[i])))
                    if shift is not None:
                        t = rne_f32(t + F(shift[i]))
                    assert F(Y[r, i]) == t, f"modulate ({r},{i}) shift={shift is not None}"


def pin_modulate_special_cases(o):
    """scale = 0 without shift is the identity; scale = 1 doubles exactly, so the
    quantizer's codes are unchanged and its scales double; a row stride is
    honoured (only the first K columns are read)."""
    rng = np.random.default_rng(42)
    M, K, G = 6, 512, 64
    wide = workloads.gaussian_activations(rng, M, K + 32, 0.01, 20.0, workloads.F32)
    X = np.ascontiguousarray(wide[:, :K])
    zero = np.zeros(K, np.float32)
    assert np.array_equal(o.modulate_rows(X, zero).view(np.uint32), X.view(np.uint32))
    two = o.modulate_rows(X, np.ones(K, np.float32))
    assert np.array_equal(two, 2 * X)
    p1, p2 = o.quantize_rows(X, G), o.quantize_rows(two, G)
    assert np.array_equal(p1.q, p2.q) and np.array_equal(p2.s, 2 * p1.s)
    sc = (rng.standard_normal(K) * 0.3).astype(np.float32)
    assert np.array_equal(o.modulate_rows(wide, sc, K=K), o.modulate_rows(X, sc))


def sqrt_rn_f32(q: Fraction) -> Fraction:
    """The binary32 value nearest to sqrt(q) (q >= 0 rational), ties to even:
    the candidate whose rounding interval holds sqrt(q), decided by comparing
    q with the squares of the interval ends exactly."""
    if q == 0:
        return Fraction(0)
    c = np.float32(math.sqrt(float(q)))
    for cand in (np.nextafter(c, np.float32(0)), c, np.nextafter(c, np.float32(np.inf))):
        v = F(cand)
        lo = (v + F(np.nextafter(cand, np.float32(0)))) / 2
        hi = (v + F(np.nextafter(cand, np.float32(np.inf)))) / 2
        even = (int(np.float32(cand).view(np.uint32)) & 1) == 0
        if (lo * lo < q or (lo * lo == q and even)) and (q < hi * hi or (q == hi * hi and even)):
            return v
    raise AssertionError("no candidate holds the root")


def rmsnorm_exact(xw: np.ndarray, eps: float, w) -> list:
    """One row of RMSNorm -> Mul(weight) in exact rationals, rounded to
    binary32 after every operation, in the reading's order: pairwise sums of
    the squares inside 64-feature blocks, block sums left to right."""
    K = len(xw)
    S = None
    for b in range(0, K, 64):
        t = [rne_f32(F(x) * F(x)) for x in xw[b:b + 64]]
        while len(t) > 1:
            t = [rne_f32(t[2 * i] + t[2 * i + 1]) for i in range(len(t) // 2)]
        S = t[0] if S is None else rne_f32(S + t[0])
    mean = rne_f32(S / K)
    d = sqrt_rn_f32(rne_f32(mean + F(np.float32(eps))))
    r = rne_f32(1 / d)
    out = []
    for i, x in enumerate(xw):
        y = rne_f32(F(x) * r)
        if w is not None:
            y = rne_f32(y * F(w[i]))
        out.append(y)
    return out


def pin_rmsnorm_exact(o):
    """RMSNorm -> Mul(weight) against exact rational arithmetic with binary32
    rounding (and a correctly rounded square root) at each step, for binary32
    and bf16 rows, with and without the weight (page "ggml operator
    extensions", the RMSNorm -> Mul(weight) -> ... -> ConvRot chain)."""
    rng = np.random.default_rng(46)
    M, K = 2, 192
    X = workloads.gaussian_activations(rng, M, K, 0.05, 20.0, workloads.F32)
    w = (1.0 + rng.standard_normal(K) * 0.2).astype(np.float32)
    Xb = workloads.f32_to_bf16_bits(X)
    for src, xw in ((X, X), (Xb, workloads.bf16_bits_to_f32(Xb))):
        for weight in (w, None):
            for eps in (1e-6, 0.5):
                Y = o.rmsnorm_rows(src, eps, weight)
                for r in range(M):
                    want = rmsnorm_exact(xw[r], eps, weight)
                    for i in range(K):
                        assert F_out(Y[r, i]) == want[i], f"rmsnorm ({r},{i}) eps={eps} w={weight is not None}"


def pin_rmsnorm_closed_forms(o):
    """Constant rows of +-2^k normalize to +-1 exactly (eps = 0), times the
    weight with one; a zero row stays zero for eps > 0; with eps = 0 the
    result does not change when the row is scaled by a power of two; a row
    stride is honoured."""
    K = 256
    rows = [np.full(K, s * 2.0 ** k, np.float32) for s in (1, -1) for k in (-20, -3, 0, 7, 30)]
    X = np.stack(rows)
    Y = o.rmsnorm_rows(X, 0.0)
    assert np.array_equal(Y, np.sign(X)), "constant rows"
    rng = np.random.default_rng(47)
    w = rng.standard_normal(K).astype(np.float32)
    assert np.array_equal(o.rmsnorm_rows(X, 0.0, w), np.sign(X) * w), "constant rows, weight"
    assert np.array_equal(o.rmsnorm_rows(np.zeros((2, K), np.float32), 1e-5), np.zeros((2, K))), "zero row"
    R = workloads.gaussian_activations(rng, 4, K, 0.01, 20.0, workloads.F32)
    base = o.rmsnorm_rows(R, 0.0, w)
    for k in (-9, 5, 21):
        assert np.array_equal(o.rmsnorm_rows((R * 2.0 ** k).astype(np.float32), 0.0, w), base), f"2^{k}"
    wide = workloads.gaussian_activations(rng, 3, K + 64, 0.01, 20.0, workloads.F32)
    assert np.array_equal(o.rmsnorm_rows(wide, 1e-6, w, K=K),
                          o.rmsnorm_rows(np.ascontiguousarray(wide[:, :K]), 1e-6, w))


def pin_rmsnorm_fp64_bound(o):
    """Against x / sqrt(mean(x^2) + eps) * w in binary64: within the error bound
    of the binary32 steps (block sums (6 + K/64) roundings, halved by the root,
    plus 6 more), for eps well below and well above the mean square."""
    rng = np.random.default_rng(48)
    for K in (64, 1024, 3072):
        X = workloads.gaussian_activations(rng, 3, K, 0.005, 30.0, workloads.F32)
        w = (1.0 + rng.standard_normal(K) * 0.2).astype(np.float32)
        x64 = X.astype(np.float64)
        for eps in (1e-6, 4.0 * float(np.mean(x64 ** 2))):
            ref = x64 / np.sqrt(np.mean(x64 ** 2, axis=1, keepdims=True) + float(np.float32(eps))) * w
            got = o.rmsnorm_rows(X, eps, w).astype(np.float64)
            bound = ((6 + K / 64) / 2 + 6) * U32 * np.abs(ref) + 1e-30
            assert np.all(np.abs(got - ref) <= bound), f"K={K} eps={eps}: {np.max(np.abs(got - ref) / bound)}"


def tree_sum_f32(vals: list) -> Fraction:
    """The reading's sum order in exact rationals rounded to binary32 after
    every addition: pairwise inside each block of 64 (adjacent pairs first),
    then the block sums left to right."""
    S = None
    for b in range(0, len(vals), 64):
        t = list(vals[b:b + 64])
        while len(t) > 1:
            t = [rne_f32(t[2 * i] + t[2 * i + 1]) for i in range(len(t) // 2)]
        S = t[0] if S is None else rne_f32(S + t[0])
    return S


def norm_exact(xw: np.ndarray, eps: float, w) -> list:
    """One row of Norm -> Mul(weight) in exact rationals with binary32 rounding
    after every operation: the mean, the deviations, the mean of their
    squares, the correctly rounded root and reciprocal, then the products."""
    K = len(xw)
    mean = rne_f32(tree_sum_f32([F(x) for x in xw]) / K)
    d = [rne_f32(F(x) - mean) for x in xw]
    var = rne_f32(tree_sum_f32([rne_f32(v * v) for v in d]) / K)
    r = rne_f32(1 / sqrt_rn_f32(rne_f32(var + F(np.float32(eps)))))
    out = []
    for i, v in enumerate(d):
        y = rne_f32(v * r)
        if w is not None:
            y = rne_f32(y * F(w[i]))
        out.append(y)
    return out


def pin_norm_exact(o):
    """Norm -> Mul(weight) against exact rational arithmetic with binary32
    rounding (and a correctly rounded square root) at each step, for binary32
    and bf16 rows with a non-zero mean, with and without the weight (page
    "ggml operator extensions", the Norm -> Mul -> ConvRot fusion)."""
    rng = np.random.default_rng(146)
    M, K = 2, 192
    X = (workloads.gaussian_activations(rng, M, K, 0.05, 20.0, workloads.F32) +
         np.float32(2.5)).astype(np.float32)
    w = (1.0 + rng.standard_normal(K) * 0.2).astype(np.float32)
    Xb = workloads.f32_to_bf16_bits(X)
    for src, xw in ((X, X), (Xb, workloads.bf16_bits_to_f32(Xb))):
        for weight in (w, None):
            for eps in (1e-6, 0.5):
                Y = o.norm_rows(src, eps, weight)
                for r in range(M):
                    want = norm_exact(xw[r], eps, weight)
                    for i in range(K):
                        assert F_out(Y[r, i]) == want[i], f"norm ({r},{i}) eps={eps} w={weight is not None}"


def pin_norm_closed_forms(o):
    """Rows alternating c + a and c - a (c, a powers of two or zero, every sum
    exact) normalize to +-1 exactly with eps = 0, times the weight with one;
    constant rows and zero rows give zeros for eps > 0; with eps = 0 scaling a
    row by 2^k changes nothing; rows whose adjacent pairs are (v, -v) have
    mean 0 exactly and equal the RMSNorm chain bit for bit; a row stride is
    honoured."""
    K = 256
    sign = np.tile(np.array([1.0, -1.0], np.float32), K // 2)
    rows = [np.float32(c) + np.float32(a) * sign for c in (0.0, 3.0, -96.0, 2.0 ** 20)
            for a in (2.0 ** -3, 1.0, 2.0 ** 7)]
    X = np.stack(rows).astype(np.float32)
    assert np.all(np.abs(np.abs(X - X.mean(axis=1, keepdims=True)) - np.abs(X[:, :1] - X[:, 1:2]) / 2) == 0)
    assert np.array_equal(o.norm_rows(X, 0.0), np.broadcast_to(sign, X.shape)), "c +- a rows"
    rng = np.random.default_rng(147)
    w = rng.standard_normal(K).astype(np.float32)
    assert np.array_equal(o.norm_rows(X, 0.0, w), np.broadcast_to(sign * w, X.shape)), "c +- a rows, weight"
    C = np.stack([np.full(K, c, np.float32) for c in (0.0, 1.0, -7.5, 2.0 ** 40)])
    assert np.array_equal(o.norm_rows(C, 1e-5, w), np.zeros((4, K))), "constant rows"
    R = workloads.gaussian_activations(rng, 4, K, 0.01, 20.0, workloads.F32) + np.float32(1.5)
    base = o.norm_rows(R, 0.0, w)
    for k in (-9, 5, 21):
        assert np.array_equal(o.norm_rows((R * 2.0 ** k).astype(np.float32), 0.0, w), base), f"2^{k}"
    P = workloads.gaussian_activations(rng, 3, K, 0.01, 20.0, workloads.F32)
    P[:, 1::2] = -P[:, 0::2]
    for eps in (0.0, 1e-6, 0.5):
        assert np.array_equal(o.norm_rows(P, eps, w), o.rmsnorm_rows(P, eps, w)), f"zero-mean rows eps={eps}"
    wide = workloads.gaussian_activations(rng, 3, K + 64, 0.01, 20.0, workloads.F32)
    assert np.array_equal(o.norm_rows(wide, 1e-6, w, K=K),
                          o.norm_rows(np.ascontiguousarray(wide[:, :K]), 1e-6, w))


def pin_norm_fp64_bound(o):
    """Against (x - mean(x)) / sqrt(var(x) + eps) * w in binary64, for rows
    with means from 0 to several deviations, eps well below and well above
    the variance.  The binary32 steps err by at most (8 + K/64) units in the
    mean (in units of the mean absolute value) and in the variance; the bound
    adds the mean's error, carried by every deviation, to a relative error
    of the same order on each output."""
    rng = np.random.default_rng(148)
    for K in (64, 1024, 3072):
        for shift in (0.0, 4.0):
            X = (workloads.gaussian_activations(rng, 3, K, 0.005, 30.0, workloads.F32) +
                 np.float32(shift)).astype(np.float32)
            w = (1.0 + rng.standard_normal(K) * 0.2).astype(np.float32)
            x64 = X.astype(np.float64)
            mu = x64.mean(axis=1, keepdims=True)
            var = ((x64 - mu) ** 2).mean(axis=1, keepdims=True)
            for eps in (1e-6, 4.0 * float(var.mean())):
                sd = np.sqrt(var + float(np.float32(eps)))
                ref = (x64 - mu) / sd * w
                got = o.norm_rows(X, eps, w).astype(np.float64)
                g = 8 + K / 64
                mean_abs = np.abs(x64).mean(axis=1, keepdims=True)
                bound = (2 * g * U32 * mean_abs / sd * np.abs(w) + (g / 2 + 8) * U32 * np.abs(ref) + 1e-30)
                assert np.all(np.abs(got - ref) <= bound), \
                    f"K={K} shift={shift} eps={eps}: {np.max(np.abs(got - ref) / bound)}"


def exp_exact_f32(x: float) -> Fraction:
    """exp(x) to 60 significant digits (Python's decimal), then rounded to
    binary32 by the IEEE rule above: the correctly rounded binary32 exp."""
    from decimal import Decimal, localcontext
    with localcontext() as ctx:
        ctx.prec = 60
        return rne_f32(Fraction(Decimal(float(x)).exp()))


def expf_sample(rng, n):
    """Binary32 arguments over exp's finite range: random bit patterns inside
    [-103.9, 88.7], plus the ends, zeros, tiny values and small integers."""
    u = rng.integers(0, 2 ** 32, size=8 * n, dtype=np.uint64).astype(np.uint32).view(np.float32)
    u = u[np.isfinite(u) & (u > -103.9) & (u < 88.7)][:n]
    special = np.array([0.0, -0.0, 1.0, -1.0, 2.0 ** -30, -(2.0 ** -30), 88.72, -103.9, 0.5,
                        -0.5, 10.0, -10.0, 17.0, -17.0, 1e-7, 87.0, -87.0], np.float32)
    return np.concatenate([special, u]).astype(np.float32)


def pin_expf_correctly_rounded(o):
    """The oracle's exp equals the correctly rounded binary32 exp (decimal at
    60 digits) on random arguments over the whole finite range."""
    rng = np.random.default_rng(71)
    for x in expf_sample(rng, 6000):
        got = np.float32(o.expf(float(x)))
        want = exp_exact_f32(float(x))
        assert F_out(got) == want, f"exp({float(x)!r}) = {float(got)!r}, want {float(want)!r}"


def gated_exact(g: float, u: float, act: int) -> Fraction:
    e = exp_exact_f32(-float(g))
    sg = rne_f32(1 / rne_f32(1 + e))
    a = rne_f32(F(g) * sg) if act == oracle_pkg.ACT_SILU else sg
    return rne_f32(a * F(u))


def pin_gated_act_exact(o):
    """SiLU/Sigmoid -> Mul against exact rational arithmetic with binary32
    rounding after each step, exp correctly rounded (page "ggml operator
    extensions", SiLU/Sigmoid -> Mul -> ConvRot): binary32 and bf16 rows."""
    rng = np.random.default_rng(72)
    M, K = 3, 40
    G = (rng.standard_normal((M, K)) * 4.0).astype(np.float32)
    U = (rng.standard_normal((M, K)) * 2.0).astype(np.float32)
    Gb, Ub = workloads.f32_to_bf16_bits(G), workloads.f32_to_bf16_bits(U)
    for (gs, us, gw, uw) in ((G, U, G, U), (Gb, Ub, workloads.bf16_bits_to_f32(Gb), workloads.bf16_bits_to_f32(Ub))):
        for act in (oracle_pkg.ACT_SILU, oracle_pkg.ACT_SIGMOID):
            Y = o.gated_act_rows(gs, us, act)
            for r in range(M):
                for i in range(K):
                    assert F_out(Y[r, i]) == gated_exact(gw[r, i], uw[r, i], act), f"({r},{i}) act={act}"


def pin_gated_act_closed_forms(o):
    """sigmoid(0) = 1/2 and silu(0) = 0; silu(g) = g once exp(-g) is below half an
    ulp of 1 (g >= 17); sigmoid of a very negative g is 0; the up factor is
    indexed like the gate; a packed [gate | up] row and its swapped form read
    the right halves."""
    K = 64
    one = np.ones((1, K), np.float32)
    assert np.array_equal(o.gated_act_rows(np.zeros((1, K), np.float32), one, oracle_pkg.ACT_SIGMOID), 0.5 * one)
    assert np.array_equal(o.gated_act_rows(np.zeros((1, K), np.float32), one, oracle_pkg.ACT_SILU), 0 * one)
    big = np.linspace(17.0, 80.0, K, dtype=np.float32)[None, :]
    assert np.array_equal(o.gated_act_rows(big, one, oracle_pkg.ACT_SILU), big)
    assert np.all(o.gated_act_rows(-big - 100.0, one, oracle_pkg.ACT_SIGMOID) == 0.0)
    rng = np.random.default_rng(73)
    g = rng.standard_normal((2, K)).astype(np.float32)
    u = rng.standard_normal((2, K)).astype(np.float32)
    base = o.gated_act_rows(g, u, oracle_pkg.ACT_SILU)
    packed = np.concatenate([g, u], axis=1)
    assert np.array_equal(o.gated_act_rows(packed, np.ascontiguousarray(packed[:, K:]), oracle_pkg.ACT_SILU, K=K), base)
    swapped = np.concatenate([u, g], axis=1)
    assert np.array_equal(o.gated_act_rows(np.ascontiguousarray(swapped[:, K:]), swapped, oracle_pkg.ACT_SILU, K=K), base)
    ones = o.gated_act_rows(g, np.ones_like(g), oracle_pkg.ACT_SIGMOID)
    assert np.array_equal(o.gated_act_rows(g, 2 * np.ones_like(g), oracle_pkg.ACT_SIGMOID), 2 * ones)


def pin_gated_act_fp64_bound(o):
    """Against g / (1 + exp(-g)) * u and u / (1 + exp(-g)) in binary64: within
    five binary32 roundings."""
    rng = np.random.default_rng(74)
    G = (rng.standard_normal((4, 256)) * 6.0).astype(np.float32)
    U = rng.standard_normal((4, 256)).astype(np.float32)
    g64, u64 = G.astype(np.float64), U.astype(np.float64)
    sg = 1.0 / (1.0 + np.exp(-g64))
    for act, ref in ((oracle_pkg.ACT_SILU, g64 * sg * u64), (oracle_pkg.ACT_SIGMOID, sg * u64)):
        got = o.gated_act_rows(G, U, act).astype(np.float64)
        assert np.all(np.abs(got - ref) <= 5 * U32 * np.abs(ref) + 1e-38), f"act={act}"


def load_int4_golden():
    rows = []
    with open(os.path.join(GOLDEN, "int4_bytes.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                b, lo, hi = line.split()
                rows.append((int(b, 16), int(lo), int(hi)))
    return rows


def pin_int4_golden(o):
    """Packed 4-bit weights decode as the hand-written table says (low nibble is
    the even feature; two's complement), at every position of a row."""
    table = load_int4_golden()
    K = 2 * len(table)
    W4 = np.array([[b for b, _, _ in table], [b for b, _, _ in reversed(table)]], np.uint8)
    Q = o.unpack_int4(W4, K)
    want = [v for _, lo, hi in table for v in (lo, hi)]
    assert Q[0].tolist() == want
    assert Q[1].tolist() == [v for _, lo, hi in reversed(table) for v in (lo, hi)]


def pin_int4_roundtrip(o):
    """Decoding is a bijection from bytes onto pairs in [-8, 7]: re-encoding
    every decoded pair (two's complement nibbles, even feature low) gives the
    byte back, for all 256 bytes; and the contraction of decoded weights equals
    integer loops over the table-decoded values."""
    W4 = np.arange(256, dtype=np.uint8).reshape(2, 128)
    Q = o.unpack_int4(W4, 256)
    assert Q.min() == -8 and Q.max() == 7
    enc = ((Q[:, 0::2].astype(np.int64) & 15) | ((Q[:, 1::2].astype(np.int64) & 15) << 4))
    assert np.array_equal(enc.astype(np.uint8), W4)
    rng = np.random.default_rng(43)
    Qx = workloads.random_codes(rng, (3, 256))
    A = o.gemm_i32(Qx, Q)
    for r in range(3):
        for n in range(2):
            assert int(A[r, n]) == sum(int(Qx[r, k]) * int(Q[n, k]) for k in range(256))


def pin_gated_residual_exact(o):
    """The gated-residual epilogue against exact rational arithmetic with
    binary32 rounding at each step: fl(fl(fl(y * scale) * gate) + r), scale
    only when != 1, gate indexed by column; residual and output in binary32
    and bf16 (page "ggml operator extensions", INT8 gated residual)."""
    rng = np.random.default_rng(44)
    M, N = 3, 40
    Y = (rng.standard_normal((M, N)) * 3.0).astype(np.float32)
    g = (rng.standard_normal(N) * 0.7).astype(np.float32)
    Rf = rng.standard_normal((M, N)).astype(np.float32)
    Rb = workloads.f32_to_bf16_bits(Rf)
    for R, rw in ((Rf, Rf), (Rb, workloads.bf16_bits_to_f32(Rb))):
        for scale in (1.0, 0.37):
            for zd in (oracle_pkg.F32, oracle_pkg.BF16):
                Z = o.gated_residual(Y, g, R, scale, zd)
                for r in range(M):
                    for i in range(N):
                        t = F(Y[r, i])
                        if scale != 1.0:
                            t = rne_f32(t * F(np.float32(scale)))
                        t = rne_f32(rne_f32(t * F(g[i])) + F(rw[r, i]))
                        if zd == oracle_pkg.F32:
                            assert F(Z[r, i]) == t, f"gated residual ({r},{i})"
                        else:   # the bf16 cast itself is pinned by pin_bf16_output
                            tb = workloads.f32_to_bf16_bits(np.array([float(t)], np.float32))[0]
                            assert int(Z[r, i]) == int(tb), f"gated residual bf16 ({r},{i})"


def pin_gated_residual_special_cases(o):
    """gate = 0 leaves exactly the residual; gate = 1 with a zero residual and
    no scale leaves exactly the reconstruction."""
    rng = np.random.default_rng(45)
    M, N = 5, 64
    Y = (rng.standard_normal((M, N)) * 3.0).astype(np.float32)
    R = (rng.standard_normal((M, N)) + 0.5).astype(np.float32)
    assert np.array_equal(o.gated_residual(Y, np.zeros(N, np.float32), R), R)
    assert np.array_equal(o.gated_residual(Y, np.ones(N, np.float32), np.zeros((M, N), np.float32)), Y)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
