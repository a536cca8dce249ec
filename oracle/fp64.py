"""Dense binary64 helpers that pin the oracle (test infrastructure only).

These follow the "INT8 Convrot Safetensors" page, section "How INT8 convrot
works": H4 as the page prints it, R_G as the normalized Kronecker power
H4 (x) ... (x) H4 (G = 4^n), applied block-diagonally to contiguous groups of
G features.  They use numpy's kron and matmul and share nothing with the
oracle's butterfly, so agreement between the two is evidence, not an echo.
"""
from __future__ import annotations

import numpy as np

# The page's matrix: [[1,1,1,-1],[1,1,-1,1],[1,-1,1,1],[-1,1,1,1]] / 2.
H4 = np.array([[1, 1, 1, -1],
               [1, 1, -1, 1],
               [1, -1, 1, 1],
               [-1, 1, 1, 1]], dtype=np.float64) / 2.0


def log4(G: int) -> int:
    n, g = 0, G
    while g > 1:
        if g % 4:
            raise ValueError(f"group size {G} is not a power of four")
        g //= 4
        n += 1
    return n


def kron_power(G: int, h4: np.ndarray = H4) -> np.ndarray:
    """R_G = h4 (x) h4 (x) ... (x) h4, n = log4(G) factors (R_1 = [[1]])."""
    R = np.ones((1, 1), dtype=np.float64)
    for _ in range(log4(G)):
        R = np.kron(R, h4)
    return R


def closed_form(G: int) -> np.ndarray:
    """R_G[i, j] = 2^-n * (-1)^(number of base-4 digit positions k with i_k + j_k = 3).

    Each factor H4[a, b] is +1/2 unless a + b = 3 (the anti-diagonal), where it
    is -1/2; a Kronecker entry is the product of the digit-wise factors.
    """
    n = log4(G)
    R = np.empty((G, G), dtype=np.float64)
    for i in range(G):
        for j in range(G):
            neg = 0
            a, b = i, j
            for _ in range(n):
                if (a % 4) + (b % 4) == 3:
                    neg += 1
                a //= 4
                b //= 4
            R[i, j] = (-1.0) ** neg * 2.0 ** (-n)
    return R


def rotate_dense(X: np.ndarray, G: int) -> np.ndarray:
    """X R in binary64 with the dense block-diagonal R (matmul per group)."""
    X = np.asarray(X, dtype=np.float64)
    M, K = X.shape
    R = kron_power(G)
    return (X.reshape(M, K // G, G) @ R).reshape(M, K)
