"""OCP FP8 e4m3fn code: decode and round-to-nearest-even encode -- test only.

Format (page legend in ``oracle/__init__.py``): e4m3 has one sign bit, four
exponent bits and three mantissa bits ([P1] "ZYFA's performance and accuracy
data").  Read as an unsigned integer, the code of a positive value grows by 8
each time the value doubles ([P3] "ZYFA 如何工作？", the lean-P paragraph).  The
pages say only "e4m3"; the workloads scale by amax/448, which fixes the OCP
"e4m3fn" variant: exponent bias 7, largest finite value 448 (code 0x7E), no
infinities, S.1111.111 is NaN.

Nothing here shares code with the HIP path.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """Value of each e4m3fn code byte, as fp64 (NaN for 0x7F / 0xFF).

    value = (-1)^s * 2^(e-7) * (1 + m/8)   for e >= 1
          = (-1)^s * 2^(-6)  * (m/8)       for e == 0 (subnormal)

    The formula is evaluated once for each of the 256 codes and the result
    indexed by the input (the same values, without evaluating it per element
    of large tensors).
    """
    return _decode_formula(np.arange(256, dtype=np.uint8))[np.asarray(codes, dtype=np.uint8)]


def _decode_formula(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(
        e == 0,
        np.ldexp(m.astype(np.float64) / 8.0, -6),
        np.ldexp(1.0 + m.astype(np.float64) / 8.0, (e - 7).astype(np.int64)),
    )
    mag = np.where((e == 0xF) & (m == 0x7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


# Non-negative finite codes 0x00..0x7E, ascending: code order equals value order.
_POS_VALUES = e4m3_decode(np.arange(0x7F, dtype=np.uint8))


def e4m3_encode_rne_sat(x) -> np.ndarray:
    """Encode real values to e4m3fn codes: round to nearest, ties to even,
    saturating at +-448.  NaN inputs give 0x7F.  The sign bit follows the sign
    of the input (negative values that round to zero give 0x80).

    Works on the exact value of ``x`` (upcast to fp64, which is exact for fp32
    and bf16 inputs), so the rounding decision is the one an IEEE conversion
    from fp32 makes.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    v = _POS_VALUES
    hi = np.searchsorted(v, a, side="left")  # first code whose value >= a
    hi = np.minimum(hi, v.size - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - v[lo]
    d_hi = v[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(v[hi] == a, hi, code)  # exactly representable
    code = code.astype(np.uint8)
    code = np.where(np.signbit(x), code | np.uint8(0x80), code).astype(np.uint8)
    code = np.where(np.isnan(x), np.uint8(0x7F), code).astype(np.uint8)
    return code
