"""Pins for the oracle's finer-granularity FP8 front end (CPU only): the
three-block Hadamard rotation at head dimension 192 against scipy's matrix, and
the per-64-position power-of-two block quantizer against its closed-form
exponent, torch's float8_e4m3fn conversion, block independence and the error
it saves on inputs whose magnitude varies along the sequence."""

import math

import numpy as np
import pytest
import scipy.linalg
import torch

from oracle import (
    attn_ref,
    block_exponent,
    dequantize_block64_ref,
    dequantize_ref,
    fwht_f32,
    hadamard_norm_f32,
    hadamard_rotate_f32,
    quantize_block64_ref,
    quantize_ref,
)

pytestmark = pytest.mark.cpu


def _x(shape, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32)


# ---- Hadamard at d = 192: three Sylvester H_64 blocks

def test_fwht192_is_block_diagonal_h64_on_integers():
    g = np.random.default_rng(0)
    x = g.integers(-500, 500, size=(200, 192)).astype(np.float32)
    h64 = scipy.linalg.hadamard(64)
    ref = x.astype(np.int64) @ scipy.linalg.block_diag(h64, h64, h64)
    assert np.array_equal(hadamard_rotate_f32(x).astype(np.int64), ref)
    assert np.array_equal(fwht_f32(x, 64).astype(np.int64), ref)


def test_normalised_rotation_preserves_dot_products():
    for d in (128, 192):
        q, k = _x((50, d), 1), _x((60, d), 2)
        n = float(hadamard_norm_f32(d))
        qr = hadamard_rotate_f32(q).astype(np.float64) * n
        kr = hadamard_rotate_f32(k).astype(np.float64) * n
        assert np.allclose(qr @ kr.T, q.astype(np.float64) @ k.astype(np.float64).T, rtol=0, atol=2e-4)
    assert hadamard_norm_f32(192) == np.float32(1 / 8) and hadamard_norm_f32(128) == np.float32(2 ** -3.5)


def test_per_head_hadamard_at_192_folds_one_eighth():
    x = _x((1, 200, 2, 192), 3)
    codes, scales = quantize_ref(x, hadamard=True)
    rot = hadamard_rotate_f32(x)
    amax = np.abs(rot[0, :, 1]).max()
    assert scales[0, 1] == np.float32(np.float32(amax / np.float32(448)) * np.float32(0.125))
    deq = dequantize_ref(codes, scales)
    ref = rot.astype(np.float64) / 8.0
    assert np.linalg.norm(deq - ref) / np.linalg.norm(ref) < 0.04


# ---- block exponent

def test_block_exponent_closed_form():
    for k in range(-100, 100, 7):
        base = math.ldexp(448.0, k)
        assert block_exponent(base) == k  # exactly on 448 * 2^k
        assert block_exponent(np.nextafter(base, np.inf)) == k + 1
        assert block_exponent(math.ldexp(base, -1) * 1.0000001) == k
    assert block_exponent(0.0) == 0
    assert block_exponent(1e-42) == -126 and block_exponent(math.ldexp(448.0, -130)) == -126
    g = np.random.default_rng(4)
    for a in g.uniform(-30, 30, 500):
        amax = float(np.float32(2.0 ** a))
        brute = min(e for e in range(-200, 200) if amax <= math.ldexp(448.0, e))
        assert block_exponent(amax) == max(brute, -126)


# ---- per-64-position block quantizer

def test_block_scales_are_tight_powers_of_two():
    x = _x((2, 300, 3, 128), 5, 3.0)
    x[0, 64:128, 1] *= 1000.0
    x[1, 256:, 2] *= 1e-3
    codes, scales = quantize_block64_ref(x)
    assert scales.shape == (2, 3, 5) and scales.dtype == np.float32
    m, _ = np.frexp(scales)
    assert np.all(m == 0.5)  # powers of two
    for b in range(2):
        for h in range(3):
            for j in range(5):
                amax = np.abs(x[b, 64 * j:64 * (j + 1), h]).max()
                r = amax / float(scales[b, h, j])
                assert 224 < r <= 448


def test_block_codes_match_torch_conversion():
    x = _x((1, 200, 2, 192), 6, 0.7)
    codes, scales = quantize_block64_ref(x)
    for h in range(2):
        for j in range(4):
            blk = torch.from_numpy(np.ascontiguousarray(x[0, 64 * j:64 * (j + 1), h]))
            ref = (blk * float(1 / scales[0, h, j])).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert np.array_equal(codes[0, 64 * j:64 * (j + 1), h], ref)


def test_block_independence_and_power_of_two_invariance():
    x = _x((1, 256, 2, 128), 7)
    c0, s0 = quantize_block64_ref(x)
    y = x.copy()
    y[0, 128:192, 0] *= np.float32(16.0)
    c1, s1 = quantize_block64_ref(y)
    assert np.array_equal(c0, c1)
    assert s1[0, 0, 2] == 16 * s0[0, 0, 2]
    mask = np.ones_like(s0, dtype=bool)
    mask[0, 0, 2] = False
    assert np.array_equal(s0[mask], s1[mask])


def test_zero_tiny_and_ragged_blocks():
    x = _x((1, 130, 1, 128), 8)
    x[0, 64:128] = 0
    x[0, 128:] *= np.float32(1e-38)
    codes, scales = quantize_block64_ref(x)
    assert scales.shape == (1, 1, 3)
    assert scales[0, 0, 1] == 1.0 and np.all(codes[0, 64:128] == 0)
    assert scales[0, 0, 2] == np.float32(2.0 ** -126)  # clamped exponent
    deq = dequantize_block64_ref(codes, scales)
    assert deq.shape == x.shape


def test_dequantize_block64_elementwise():
    x = _x((2, 100, 2, 128), 9)
    codes, scales = quantize_block64_ref(x)
    deq = dequantize_block64_ref(codes, scales)
    from oracle import e4m3_decode

    vals = e4m3_decode(codes)
    for b, n, h in [(0, 0, 0), (1, 63, 1), (1, 64, 0), (0, 99, 1)]:
        assert np.array_equal(deq[b, n, h], vals[b, n, h] * float(scales[b, h, n // 64]))


def test_block_hadamard_normalises_values():
    for d in (128, 192):
        x = _x((1, 128, 2, d), 10)
        codes, scales = quantize_block64_ref(x, hadamard=True)
        ref = hadamard_rotate_f32(x).astype(np.float64) * float(hadamard_norm_f32(d))
        deq = dequantize_block64_ref(codes, scales)
        assert np.linalg.norm(deq - ref) / np.linalg.norm(ref) < 0.04


def test_block_scales_cut_error_when_magnitude_varies_along_the_sequence():
    # one scale per head wastes e4m3 range on blocks far below the head's amax;
    # per-block scales keep every block in the normal range
    x = _x((1, 512, 1, 128), 12)
    mags = np.float32(10.0) ** np.array([0, -1, -2, -3, -4, -4.5, -2.5, -3.5], dtype=np.float32)
    x *= np.repeat(mags, 64)[None, :, None, None]
    def per_block_rel(deq):
        return [np.linalg.norm(deq[0, j:j + 64] - x[0, j:j + 64]) / np.linalg.norm(x[0, j:j + 64])
                for j in range(0, 512, 64)]

    r_head = per_block_rel(dequantize_ref(*quantize_ref(x)))
    r_blk = per_block_rel(dequantize_block64_ref(*quantize_block64_ref(x)))
    assert max(r_blk) < 0.04  # every block keeps e4m3's relative precision
    assert max(r_head) > 0.1  # blocks far below the head's amax fall into the subnormals
    # attention on block-quantized K/V stays close to attention on exact inputs
    q, k, v = _x((1, 512, 2, 128), 13), x, _x((1, 512, 1, 128), 14) * 3
    exact = attn_ref(q, k, v)
    blk = attn_ref(q, dequantize_block64_ref(*quantize_block64_ref(k)), dequantize_block64_ref(*quantize_block64_ref(v)))
    assert np.linalg.norm(blk - exact) / np.linalg.norm(exact) < 0.06
