"""Per-(batch, head) FP8 e4m3fn quantization with amax/448 scales -- test only.

The pages (legend in ``oracle/__init__.py``) state that FP8 attention needs
per-tensor or per-head scale factors to bring values into the representable
range, with FP32 accumulation ([P1] "ZYFA's performance and accuracy data"); the
workloads fix one fp32 scale per (batch, head) equal to amax/448.  The steps and
their fp32 rounding are a reading where the pages are silent:

1. optional rotation x <- fwht128(x) (unnormalised, fp32), Q and K only;
2. amax = max |x| over the (batch, head) slice [N, d];
3. inv = fp32(448 / amax), scale = fp32(amax / 448)   (correctly rounded);
   amax == 0 gives inv = scale = 1 (all codes 0);
4. y = fp32(x * inv), clamped to [-448, 448];
5. code = round-to-nearest-even e4m3fn(y);
6. with the rotation the stored scale is fp32(scale * fp32(2^-3.5)), which folds
   the 1/sqrt(128) normalisation of the Hadamard matrix.

Dequantized value seen by attention: e4m3_decode(code) * stored_scale, exact in
fp64 (4-bit times 24-bit significands fit in 53 bits).
"""

from __future__ import annotations

import numpy as np

from .e4m3 import E4M3_MAX, e4m3_decode, e4m3_encode_rne_sat
from .hadamard import fwht128_f32

INV_SQRT128_F32 = np.float32(2.0 ** -3.5)


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
        x = fwht128_f32(x)
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
                scale = np.float32(scale * INV_SQRT128_F32)
            scales[b, h] = scale
    return codes, scales


def dequantize_ref(codes, scales) -> np.ndarray:
    """fp64 [B, N, H, d] values = decode(code) * scale[b, h] (exact)."""
    vals = e4m3_decode(codes)
    s = np.asarray(scales, dtype=np.float64)
    return vals * s[:, None, :, None]
