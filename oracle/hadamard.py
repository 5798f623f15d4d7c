"""128-point Hadamard rotation along the head dimension -- test only.

The pages (legend in ``oracle/__init__.py``) report that rotating Q and K by a
Hadamard matrix before FP8 quantization roughly halves the input-quantization
error at a small time cost ([P3] "ZYFA 的 FP8 注意力有多准确？", [P2] "Accuracy and
Code").  They do not say which Hadamard matrix; the reading taken is
the plain Sylvester matrix H_128 with no random signs, applied as x <- x H_128,
with the 1/sqrt(128) normalisation folded into the per-head scale instead of
into the values.

Because the quantized codes are integers decided by fp32 arithmetic, the oracle
and the kernel must take that decision in the same precision with the same
operation order: the fast transform below is the textbook radix-2 butterfly on
fp32 values, stage widths 1, 2, 4, ..., 64, each butterfly (a, b) -> (a + b,
a - b).  Each fp32 add/sub is correctly rounded, so that order fixes every bit.
"""

from __future__ import annotations

import numpy as np


def sylvester_hadamard(n: int) -> np.ndarray:
    """Sylvester construction: H_1 = [1], H_2n = [[H, H], [H, -H]] (int64)."""
    if n < 1 or n & (n - 1):
        raise ValueError("n must be a power of two")
    h = np.ones((1, 1), dtype=np.int64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def fwht128_f32(x) -> np.ndarray:
    """Unnormalised fast Walsh-Hadamard transform over the last axis (size 128),
    in fp32, equal to x @ H_128 up to fp32 rounding (exactly equal whenever
    every partial sum is representable, e.g. small integers)."""
    y = np.array(x, dtype=np.float32, copy=True)
    if y.shape[-1] != 128:
        raise ValueError("last axis must have 128 entries")
    lead = y.shape[:-1]
    y = y.reshape(-1, 128)
    width = 1
    while width < 128:
        # pair index i with i + width inside each block of 2*width channels
        blocks = y.reshape(y.shape[0], 128 // (2 * width), 2, width)
        a = blocks[:, :, 0, :].copy()
        b = blocks[:, :, 1, :].copy()
        blocks[:, :, 0, :] = a + b  # fp32 + fp32 -> fp32 (numpy keeps float32)
        blocks[:, :, 1, :] = a - b
        y = blocks.reshape(-1, 128)
        width *= 2
    return y.reshape(*lead, 128)
