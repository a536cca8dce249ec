"""Seeded synthetic inputs for the INT8 convrot linear layer.

This module only draws random numbers and lays them out.  It holds none of
the layer's arithmetic (no rotation, no quantization, no GEMM, no
reconstruction), so the CPU oracle and the HIP path can both consume what it
produces without sharing any of the method's code.

Workloads are DiT-shaped linears (hidden width 3072, MLP width 12288, 4096
tokens per image), as in the "INT8 Convrot Safetensors" page, section "How INT8
convrot works" (G = 256 is the commonly used group size).  No dataset or
trained checkpoint is involved: activations are N(0, 1) with sparse large
outliers (the isolated large values that the rotation is meant to spread), and
weights are N(0, 0.02) floats that the caller rotates and quantizes per output
row (the page's "Weight quantization" section).

Recipe, per workload (fixed draw order):
    rng = numpy.random.default_rng(seed)                        # PCG64
    X   = rng.standard_normal((M, K), float32)
    X[rng.random((M, K), float32) < p] *= f                     # outliers
    X   = bf16(X) (round to nearest even) when the input dtype is bf16
    for each linear j:
        W_j = rng.standard_normal((N, K), float32) * 0.02
        b_j = rng.standard_normal(N, float32) * 0.1
    for 4-bit weights (convrot_w4a4) instead, per linear j:
        W4_j = rng.integers(0, 256, (N, K/2), uint8)            # every nibble value
        s_w_j = exp(rng.uniform(log 1e-3, log 1e-2, N)) as float32
        b_j = rng.standard_normal(N, float32) * 0.1
    when the workload has a gated-residual epilogue:
        gate = rng.standard_normal(N, float32) * 0.3
        residual = rng.standard_normal((M, N), float32), in the output dtype
    when the workload has a gated activation producer (X is the gate):
        up = rng.standard_normal((M, K), float32), outliers as for X, same dtype
    when the workload has an RMSNorm -> Mul(weight) or a Norm -> Mul(weight)
    producer (eps 1e-6):
        norm_weight = 1 + rng.standard_normal(K, float32) * 0.1
    when the workload has a Modulate producer (per-channel vectors, as the
    adaLN modulation of a DiT block supplies them):
        scale = rng.standard_normal(K, float32) * 0.3
        shift = rng.standard_normal(K, float32) * 0.3
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

F32 = "f32"
BF16 = "bf16"


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    K: int
    N: int
    G: int
    x_dtype: str
    y_dtype: str
    input_scales: tuple = (1.0,)      # one entry per linear reading the same X
    seed: int = 0
    outlier_p: float = 0.005
    outlier_f: float = 30.0
    modulate: bool = False            # a Modulate producer before the rotation
    w_bits: int = 8                   # 4: convrot_w4a4 packed weights
    gated: bool = False               # a gated-residual epilogue after the linear
    rmsnorm: bool = False             # RMSNorm -> Mul(weight) ahead of the Modulate
    norm: bool = False                # Norm (mean and variance) -> Mul(weight) ahead of the rotation
    rms_eps: float = 1e-6             # eps of either normalization
    glu: int = 0                      # 1 SiLU, 2 Sigmoid: fl(act(X) * up) ahead of the rotation
    swiglu: bool = False              # the two linears are a SwiGLU pair (gate, up), bias-free
    note: str = ""

    @property
    def n_linears(self) -> int:
        return len(self.input_scales)


WORKLOADS = {
    "tiny": Workload("tiny", 8, 256, 32, 16, F32, F32, (1.0,), seed=0,
                     outlier_p=0.01, outlier_f=20.0,
                     note="tiny oracle check, X [8,256], W [32,256], G=16"),
    "attn": Workload("attn", 1024, 3072, 3072, 256, F32, F32, (1.0,), seed=1,
                     note="DiT attention projection"),
    "mlp_up": Workload("mlp_up", 4096, 3072, 12288, 256, BF16, BF16, (1.0,), seed=2,
                       note="DiT MLP up-projection, bf16 in/out"),
    "qkv": Workload("qkv", 4096, 3072, 3072, 256, F32, F32, (1.0, 1.0, 1.0, 0.5), seed=3,
                    note="three linears sharing one packed input, plus one at input scale 0.5"),
    "mlp_up_mod": Workload("mlp_up_mod", 4096, 3072, 12288, 256, BF16, BF16, (1.0,), seed=5,
                           modulate=True,
                           note="DiT MLP up-projection with its Modulate producer fused"),
    "mlp_up_rms": Workload("mlp_up_rms", 4096, 3072, 12288, 256, BF16, BF16, (1.0,), seed=8,
                           modulate=True, rmsnorm=True,
                           note="DiT MLP up-projection with RMSNorm -> Mul(weight) -> Modulate fused"),
    "mlp_up_norm": Workload("mlp_up_norm", 4096, 3072, 12288, 256, BF16, BF16, (1.0,), seed=11,
                            norm=True,
                            note="DiT MLP up-projection with Norm -> Mul(weight) fused"),
    "mlp_up_w4": Workload("mlp_up_w4", 4096, 3072, 12288, 256, BF16, BF16, (1.0,), seed=6,
                          w_bits=4, note="DiT MLP up-projection with convrot_w4a4 weights"),
    "proj_gated": Workload("proj_gated", 4096, 3072, 3072, 256, BF16, BF16, (1.0,), seed=7,
                           gated=True,
                           note="DiT output projection with its gated residual, in place"),
    "mlp_up_swiglu": Workload("mlp_up_swiglu", 4096, 3072, 12288, 256, BF16, BF16, (1.0, 1.0),
                              seed=10, swiglu=True,
                              note="DiT SwiGLU MLP up-projection: gate and up weights, one dual GEMM"),
    "mlp_down_glu": Workload("mlp_down_glu", 4096, 12288, 3072, 256, BF16, BF16, (1.0,), seed=9,
                             glu=1, note="DiT MLP down-projection of silu(gate) * up, fused"),
    "mlp_down": Workload("mlp_down", 16384, 12288, 3072, 256, BF16, BF16, (1.0,), seed=4,
                         note="batched MLP down-projection, 4 images x 4096 tokens, bf16 in/out"),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bits (uint16) to fp32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def gaussian_activations(rng: np.random.Generator, M: int, K: int, p: float, f: float,
                         dtype: str) -> np.ndarray:
    """N(0,1) [M,K] with a Bernoulli(p) mask of entries multiplied by f.

    Returns float32 for F32, uint16 bf16 bits for BF16.
    """
    X = rng.standard_normal((M, K), dtype=np.float32)
    if p > 0:
        mask = rng.random((M, K), dtype=np.float32) < np.float32(p)
        X[mask] *= np.float32(f)
    if dtype == BF16:
        return f32_to_bf16_bits(X)
    if dtype != F32:
        raise ValueError(f"unknown dtype {dtype}")
    return X


def gaussian_weights(rng: np.random.Generator, N: int, K: int):
    """W ~ N(0, 0.02) [N,K] fp32 and bias ~ N(0, 0.1) [N] fp32."""
    W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    b = rng.standard_normal(N, dtype=np.float32) * np.float32(0.1)
    return W, b


@dataclass
class Inputs:
    workload: Workload
    X: np.ndarray                      # float32 or uint16 (bf16 bits), [M,K]
    W: list = field(default_factory=list)   # float32 [N,K] per linear
    b: list = field(default_factory=list)   # float32 [N] per linear
    s_w: list = field(default_factory=list) # float32 [N] per linear (4-bit weights only)
    norm_weight: np.ndarray | None = None   # float32 [K] (RMSNorm or Norm producer)
    up: np.ndarray | None = None            # like X, [M,K] (gated activation producer)
    mod_scale: np.ndarray | None = None     # float32 [K] (Modulate producer)
    mod_shift: np.ndarray | None = None     # float32 [K]
    gate: np.ndarray | None = None          # float32 [N] (gated residual)
    residual: np.ndarray | None = None      # [M,N] in the output dtype (gated residual)


def make_inputs(w: Workload, seed: int | None = None, M: int | None = None) -> Inputs:
    """Draw the workload's inputs in the fixed order documented above.

    ``M`` may override the row count (a smaller slice of the same recipe).
    """
    rng = np.random.default_rng(w.seed if seed is None else seed)
    rows = w.M if M is None else M
    X = gaussian_activations(rng, rows, w.K, w.outlier_p, w.outlier_f, w.x_dtype)
    inp = Inputs(w, X)
    for _ in range(w.n_linears):
        if w.w_bits == 4:
            inp.W.append(random_int4_packed(rng, w.N, w.K))
            inp.s_w.append(random_scales(rng, w.N, 1e-3, 1e-2))
            inp.b.append(rng.standard_normal(w.N, dtype=np.float32) * np.float32(0.1))
            continue
        W, b = gaussian_weights(rng, w.N, w.K)
        inp.W.append(W)
        inp.b.append(b)
    if w.glu:
        inp.up = gaussian_activations(rng, rows, w.K, w.outlier_p, w.outlier_f, w.x_dtype)
    if w.rmsnorm or w.norm:
        inp.norm_weight = norm_weight(rng, w.K)
    if w.modulate:
        inp.mod_scale, inp.mod_shift = modulation(rng, w.K)
    if w.gated:
        inp.gate = rng.standard_normal(w.N, dtype=np.float32) * np.float32(0.3)
        inp.residual = gaussian_activations(rng, rows, w.N, 0.0, 1.0, w.y_dtype)
    return inp


def norm_weight(rng: np.random.Generator, K: int, sigma: float = 0.1):
    """Normalization weight 1 + N(0, sigma), fp32 [K]."""
    return np.float32(1.0) + rng.standard_normal(K, dtype=np.float32) * np.float32(sigma)


def modulation(rng: np.random.Generator, K: int, sigma: float = 0.3):
    """Per-channel Modulate vectors (scale, shift), each N(0, sigma) fp32 [K]."""
    sc = rng.standard_normal(K, dtype=np.float32) * np.float32(sigma)
    sh = rng.standard_normal(K, dtype=np.float32) * np.float32(sigma)
    return sc, sh


def random_int4_packed(rng: np.random.Generator, N: int, K: int) -> np.ndarray:
    """Uniform bytes [N, K/2]: packed 4-bit weights covering every nibble value."""
    return rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)


def random_codes(rng: np.random.Generator, shape, lo: int = -127, hi: int = 127) -> np.ndarray:
    """Uniform int8 codes in [lo, hi] (for contraction-only tests)."""
    return rng.integers(lo, hi + 1, size=shape, dtype=np.int8)


def random_scales(rng: np.random.Generator, n: int, lo: float = 1e-3, hi: float = 1e-1) -> np.ndarray:
    """Positive fp32 scales, log-uniform in [lo, hi]."""
    return np.exp(rng.uniform(np.log(lo), np.log(hi), size=n)).astype(np.float32)
