"""FP8 e4m3fn quantization of attention inputs -- test only.

The pages (legend in ``oracle/__init__.py``) state that FP8 attention needs
per-tensor or per-head scale factors to bring values into the representable
range, and that finer scaling granularity is one of the places where accuracy
is won, with FP32 accumulation ([P1] "ZYFA's performance and accuracy data").
Two granularities are defined here; the steps and their fp32 rounding are
readings taken where the pages are silent.

Per (batch, head), ``quantize_ref`` (the workloads' amax/448 scales):

1. optional rotation x <- x H (unnormalised, fp32; ``hadamard.py``), Q and K only;
2. amax = max |x| over the (batch, head) slice [N, d];
3. inv = fp32(448 / amax), scale = fp32(amax / 448)   (correctly rounded);
   amax == 0 gives inv = scale = 1 (all codes 0);
4. y = fp32(x * inv), clamped to [-448, 448];
5. code = round-to-nearest-even e4m3fn(y);
6. with the rotation the stored scale is fp32(scale * norm), norm = fp32(2^-3.5)
   (d = 128) or 2^-3 (d = 192), which folds the normalisation of the matrix.

Per (batch, head, block of 64 positions), ``quantize_block64_ref``, with
power-of-two scales (the form the scaled matrix instructions of CDNA4 apply):

1. optional rotation z = fp32(fp32(x H) * norm) -- the normalisation goes into
   the values, since a power-of-two scale cannot hold 2^-3.5;
2. amax = max |z| over the block [64 positions, d] (the last block may be
   shorter);
3. e = the smallest integer with amax <= 448 * 2^e, but at least -126 (scales
   stay normal fp32 numbers); amax == 0 gives e = 0;
4. code = round-to-nearest-even e4m3fn(fp32(z * 2^-e)) (exact scaling, no clamp
   needed);
5. the stored scale is 2^e (fp32).

Dequantized value seen by attention: e4m3_decode(code) * stored scale, exact in
fp64 (4-bit times 24-bit significands fit in 53 bits).
"""

from __future__ import annotations

import math

import numpy as np

from .e4m3 import E4M3_MAX, e4m3_decode, e4m3_encode_rne_sat
from .hadamard import hadamard_norm_f32, hadamard_rotate_f32

INV_SQRT128_F32 = np.float32(2.0 ** -3.5)
BLOCK = 64  # positions per scale block of quantize_block64_ref


def _as_f32(x) -> np.ndarray:
    if hasattr(x, "detach"):
        import torch

        x = x.detach().to("cpu").to(torch.float32).numpy()
    return np.asarray(x, dtype=np.float32)


def quantize_ref(x, hadamard: bool = False):
    """x: [B, N, H, d] real (fp32 or bf16).  Returns (codes uint8 [B, N, H, d],
    scales float32 [B, H])."""
    x = _as_f32(x)
    if x.ndim != 4:
        raise ValueError("x must be [B, N, H, d]")
    if hadamard:
        x = hadamard_rotate_f32(x)
    B, N, H, d = x.shape
    codes = np.empty(x.shape, dtype=np.uint8)
    scales = np.empty((B, H), dtype=np.float32)
    f448 = np.float32(E4M3_MAX)
    for b in range(B):
        for h in range(H):
            xs = x[b, :, h, :]
            amax = np.float32(np.max(np.abs(xs))) if xs.size else np.float32(0)
            if amax == 0:
                inv = np.float32(1.0)
                scale = np.float32(1.0)
            else:
                inv = np.float32(f448 / amax)  # fp32 / fp32, correctly rounded
                scale = np.float32(amax / f448)
            y = np.clip((xs * inv).astype(np.float32), -f448, f448)
            codes[b, :, h, :] = e4m3_encode_rne_sat(y)
            if hadamard:
                scale = np.float32(scale * hadamard_norm_f32(d))
            scales[b, h] = scale
    return codes, scales


def dequantize_ref(codes, scales) -> np.ndarray:
    """fp64 [B, N, H, d] values = decode(code) * scale[b, h] (exact)."""
    vals = e4m3_decode(codes)
    s = np.asarray(scales, dtype=np.float64)
    return vals * s[:, None, :, None]


def block_exponent(amax: float) -> int:
    """Smallest integer e with amax <= 448 * 2^e, at least -126; 0 for amax == 0.
    Decided with exact fp64 comparisons (powers of two times 448 are exact)."""
    if amax == 0:
        return 0
    e = math.frexp(float(amax))[1] - 9  # 256 * 2^e <= amax < 512 * 2^e, so e - 1 is too small
    if float(amax) > math.ldexp(float(E4M3_MAX), e):
        e += 1  # 448 * 2^e < amax < 512 * 2^e
    return max(e, -126)


def quantize_block64_ref(x, hadamard: bool = False):
    """x: [B, N, H, d] real (fp32 or bf16).  Returns (codes uint8 [B, N, H, d],
    scales float32 [B, H, ceil(N / 64)], each a power of two)."""
    x = _as_f32(x)
    if x.ndim != 4:
        raise ValueError("x must be [B, N, H, d]")
    B, N, H, d = x.shape
    if hadamard:
        x = (hadamard_rotate_f32(x) * hadamard_norm_f32(d)).astype(np.float32)
    nb = -(-N // BLOCK)
    codes = np.empty(x.shape, dtype=np.uint8)
    scales = np.empty((B, H, nb), dtype=np.float32)
    for b in range(B):
        for h in range(H):
            for j in range(nb):
                xs = x[b, j * BLOCK:(j + 1) * BLOCK, h, :]
                e = block_exponent(np.max(np.abs(xs)))
                y = (xs * np.float32(math.ldexp(1.0, -e))).astype(np.float32)
                codes[b, j * BLOCK:(j + 1) * BLOCK, h, :] = e4m3_encode_rne_sat(y)
                scales[b, h, j] = np.float32(math.ldexp(1.0, e))
    return codes, scales


def dequantize_block64_ref(codes, scales) -> np.ndarray:
    """fp64 [B, N, H, d] values = decode(code) * scale[b, h, n // 64] (exact)."""
    vals = e4m3_decode(codes)
    s = np.asarray(scales, dtype=np.float64)  # [B, H, nb]
    N = vals.shape[1]
    per_pos = np.repeat(s, BLOCK, axis=2)[:, :, :N]  # [B, H, N]
    return vals * per_pos.transpose(0, 2, 1)[:, :, :, None]
