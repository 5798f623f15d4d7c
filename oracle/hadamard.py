"""Hadamard rotation along the head dimension -- test only.

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

Head dimension 192 (the multi-head-latent query/key width): the pages report the
rotation only at 128.  The reading taken here is the block-diagonal matrix of
three Sylvester H_64 (one transform per consecutive group of 64 channels, stage
widths 1, ..., 32), whose normalisation 1/8 is exact; Q and K get the same
matrix, so their dot products are preserved.
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


def fwht_f32(x, n: int) -> np.ndarray:
    """Unnormalised n-point fast Walsh-Hadamard transform of every consecutive
    group of n entries of the last axis, in fp32: x @ blockdiag(H_n, ..., H_n)
    up to fp32 rounding (exactly equal whenever every partial sum is
    representable, e.g. small integers)."""
    y = np.array(x, dtype=np.float32, copy=True)
    if n < 1 or n & (n - 1) or y.shape[-1] % n:
        raise ValueError("the last axis must split into groups of a power-of-two size n")
    shape = y.shape
    y = y.reshape(-1, n)
    width = 1
    while width < n:
        # pair index i with i + width inside each block of 2*width channels
        blocks = y.reshape(y.shape[0], n // (2 * width), 2, width)
        a = blocks[:, :, 0, :].copy()
        b = blocks[:, :, 1, :].copy()
        blocks[:, :, 0, :] = a + b  # fp32 + fp32 -> fp32 (numpy keeps float32)
        blocks[:, :, 1, :] = a - b
        y = blocks.reshape(-1, n)
        width *= 2
    return y.reshape(shape)


def fwht128_f32(x) -> np.ndarray:
    """The 128-point transform over a last axis of exactly 128 entries."""
    if np.shape(x)[-1] != 128:
        raise ValueError("last axis must have 128 entries")
    return fwht_f32(x, 128)


def hadamard_block(d: int) -> int:
    """Size of the Sylvester blocks that rotate a head dimension d: 128 for
    d = 128, 64 for d = 192 (three blocks)."""
    if d == 128:
        return 128
    if d == 192:
        return 64
    raise ValueError("the Hadamard rotation is defined for d = 128 and d = 192")


def hadamard_rotate_f32(x) -> np.ndarray:
    """Unnormalised rotation of the last axis (d = 128 or 192), in fp32."""
    return fwht_f32(x, hadamard_block(np.shape(x)[-1]))


def hadamard_norm_f32(d: int) -> np.float32:
    """fp32 normalisation of the rotation: 1/sqrt(block size), i.e.
    fp32(2^-3.5) for d = 128 and exactly 2^-3 for d = 192."""
    return np.float32(2.0 ** -3.5) if hadamard_block(d) == 128 else np.float32(0.125)
