"""Shared helpers of the GPU parity tests: tolerances and comparison metrics.

Tolerances (relative Frobenius error of the BF16 output against the fp64
oracle on the inputs the kernel consumed): BF16 path 1e-2, FP8 path 6e-2.
"""

import numpy as np
import torch

TOL = {"bf16": 1e-2, "fp8": 6e-2}


def rel_fro(out, ref) -> float:
    o = out.detach().to("cpu", torch.float64).numpy() if hasattr(out, "detach") else np.asarray(out, np.float64)
    r = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(o - r) / np.linalg.norm(r))


def per_head_rel_fro(out, ref):
    o = out.detach().to("cpu", torch.float64).numpy()
    r = np.asarray(ref, dtype=np.float64)
    num = np.sqrt(((o - r) ** 2).sum(axis=(0, 1, 3)))
    den = np.sqrt((r ** 2).sum(axis=(0, 1, 3)))
    return num / den


def sample_rows(N: int, count: int, seed: int) -> np.ndarray:
    """First and last rows, the rows around tile edges near the end, plus a
    seeded random sample; sorted, unique."""
    g = np.random.default_rng(seed)
    fixed = [0, 1, 31, 32, 63, 64, 127, 128, N // 2, N - 129, N - 128, N - 65, N - 64, N - 33, N - 32, N - 2, N - 1]
    rnd = g.integers(0, N, size=count)
    rows = np.unique(np.clip(np.concatenate([fixed, rnd]), 0, N - 1))
    return rows.astype(np.int64)
