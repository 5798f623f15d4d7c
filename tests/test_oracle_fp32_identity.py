"""An fp32 identity the quantizer's amax pass relies on (CPU, numpy fp32).

With the Hadamard rotation the amax pass does not form the last butterfly
stage: the larger magnitude of its outputs fl(a + b) and fl(a - b) equals
fl(|a| + |b|) exactly in IEEE fp32 (round-to-nearest-even), so the amax over
the rotated values is the same bits whichever way it is computed.  Checked
here on random pairs over the whole fp32 range, subnormals, zeros of both
signs, near-overflow values and equal or opposite magnitudes.
"""

import numpy as np
import pytest

pytestmark = pytest.mark.cpu


def _pairs(rng, n):
    mant = rng.uniform(1.0, 2.0, size=(2, n))
    expo = rng.integers(-149, 128, size=(2, n))
    sign = rng.choice([-1.0, 1.0], size=(2, n))
    x = (sign * mant * np.exp2(expo.astype(np.float64))).astype(np.float32)
    a, b = x[0], x[1]
    # close exponents, where the rounding of the sum matters most
    c = (sign[1] * rng.uniform(1.0, 2.0, n) * np.exp2(np.clip(expo[0] + rng.integers(-30, 31, n), -149, 127)))
    return np.concatenate([a, a]), np.concatenate([b, c.astype(np.float32)])


def test_max_of_butterfly_magnitudes_is_sum_of_magnitudes():
    rng = np.random.default_rng(0)
    a, b = _pairs(rng, 1_000_000)
    specials = np.array([0.0, -0.0, 1e-45, -1e-45, 1.17549435e-38, 3.4028235e38, -3.4028235e38, 1.0, -1.0, 2.0 ** -24],
                        dtype=np.float32)
    a = np.concatenate([a, np.repeat(specials, len(specials))])
    b = np.concatenate([b, np.tile(specials, len(specials))])
    with np.errstate(over="ignore"):
        lhs = np.maximum(np.abs(a + b), np.abs(a - b))
        rhs = np.abs(a) + np.abs(b)
    assert lhs.dtype == np.float32 and rhs.dtype == np.float32
    assert np.array_equal(lhs.view(np.uint32), rhs.view(np.uint32))
