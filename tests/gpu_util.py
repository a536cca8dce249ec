"""Helpers for the GPU parity tests: numpy <-> device tensors and comparisons."""
from __future__ import annotations

import os
import sys

import numpy as np

DEV = "cuda:0"
THREADS = max(1, min(16, os.cpu_count() or 1))


def say(*a):
    """Name the case before each GPU step (flushed, so a fault still shows it)."""
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def dev_x(X: np.ndarray):
    import torch
    X = np.ascontiguousarray(X)
    if X.dtype == np.uint16:
        return torch.from_numpy(X.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(X).to(DEV)


def dev(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t) -> np.ndarray:
    import torch
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def assert_bits_equal(got: np.ndarray, want: np.ndarray, what: str):
    assert got.shape == want.shape, f"{what}: shape {got.shape} vs {want.shape}"
    if got.dtype == np.float32:
        g, w = got.view(np.uint32), want.view(np.uint32)
    else:
        g, w = got, want
    bad = np.argwhere(g != w)
    if bad.size:
        idx = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} of {g.size} differ; first at {idx}: "
                             f"{got[idx]!r} vs {want[idx]!r}")


def max_rel_err(got: np.ndarray, want: np.ndarray) -> float:
    """max |got - want| / max(|want|, 1e-6 * rms(want)), in binary64."""
    g, w = got.astype(np.float64), want.astype(np.float64)
    # (an all-zero reference still gives a finite ratio)
    floor = max(1e-6 * float(np.sqrt(np.mean(w * w))), np.finfo(np.float64).tiny) if w.size else 0.0
    return float(np.max(np.abs(g - w) / np.maximum(np.abs(w), floor))) if w.size else 0.0


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)
