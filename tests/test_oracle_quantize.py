"""Pins for the oracle's per-head FP8 quantizer (CPU only): the amax element
lands on the largest code, every value is within half an e4m3 step of its
input, the scale is amax/448, zero and power-of-two cases, and an independent
conversion through torch's float8_e4m3fn."""

import numpy as np
import pytest
import torch

from oracle import dequantize_ref, e4m3_decode, fwht128_f32, quantize_ref
from bf16_causal_prefill_flashattention_amd.inputs import WORKLOADS, make_qkv

pytestmark = pytest.mark.cpu


def _x(shape, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32)


def test_scale_and_amax_code():
    x = _x((2, 100, 3, 128), 0, 5.0)
    codes, scales = quantize_ref(x)
    assert codes.dtype == np.uint8 and scales.dtype == np.float32
    for b in range(2):
        for h in range(3):
            amax = np.abs(x[b, :, h]).max()
            assert scales[b, h] == np.float32(amax / np.float32(448))
            i = np.unravel_index(np.abs(x[b, :, h]).argmax(), x[b, :, h].shape)
            assert codes[b, :, h][i] & 0x7F == 0x7E


def test_within_half_step():
    x = _x((1, 500, 2, 128), 1, 2.0)
    codes, scales = quantize_ref(x)
    deq = dequantize_ref(codes, scales)
    y = x.astype(np.float64) / scales.astype(np.float64)[:, None, :, None]  # value in code units
    err = np.abs(deq / scales.astype(np.float64)[:, None, :, None] - y)
    # normal range: half a step is 2^-4 relative; subnormal: 2^-10 absolute
    bound = np.maximum(np.abs(y) * 2.0 ** -4, 2.0 ** -10) * (1 + 1e-6)
    assert np.all(err <= bound)


def test_matches_torch_conversion():
    x = _x((1, 300, 4, 128), 2, 0.3)
    codes, scales = quantize_ref(x)
    for h in range(4):
        t = torch.from_numpy(x[0, :, h])
        inv = torch.tensor(np.float32(448) / np.float32(np.abs(x[0, :, h]).max()))
        ref = (t * inv).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(codes[0, :, h], ref)


def test_zero_head_and_power_of_two_invariance():
    x = _x((1, 64, 2, 128), 3)
    x[0, :, 1] = 0
    codes, scales = quantize_ref(x)
    assert scales[0, 1] == 1.0 and np.all(codes[0, :, 1] == 0)
    c2, s2 = quantize_ref(x * np.float32(8.0))
    assert np.array_equal(c2[0, :, 0], codes[0, :, 0])
    assert s2[0, 0] == scales[0, 0] * 8


def test_bf16_input_is_upcast_exactly():
    x = torch.from_numpy(_x((1, 64, 2, 128), 4)).to(torch.bfloat16)
    c1, s1 = quantize_ref(x)
    c2, s2 = quantize_ref(x.float().numpy())
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


def test_hadamard_variant_dequantizes_to_normalised_rotation():
    x = _x((1, 256, 2, 128), 5)
    codes, scales = quantize_ref(x, hadamard=True)
    rot = fwht128_f32(x).astype(np.float64) / np.sqrt(128.0)
    deq = dequantize_ref(codes, scales)
    rel = np.linalg.norm(deq - rot) / np.linalg.norm(rot)
    assert rel < 0.04  # e4m3 rounding of Gaussian-like values
    # the folded normalisation is fp32(2^-3.5) applied to amax/448
    amax = np.abs(fwht128_f32(x)[0, :, 0]).max()
    assert scales[0, 0] == np.float32(np.float32(amax / np.float32(448)) * np.float32(2 ** -3.5))


def test_hadamard_halves_error_on_aligned_outliers():
    # the pages report that rotating Q and K roughly halves the input error on
    # activation-like inputs; with aligned outlier channels the rotation spreads
    # the large channels over all 128 coordinates
    w = WORKLOADS["fp8_gqa_n16k"].with_(N=512, Hq=4, Hkv=1)
    q, k, v = make_qkv(w)
    q, k = q.numpy(), k.numpy()
    from oracle import attn_ref

    exact = attn_ref(q, k, v.numpy())

    def run(had):
        cq, sq = quantize_ref(q, had)
        ck, sk = quantize_ref(k, had)
        cv, sv = quantize_ref(v.numpy(), False)
        return attn_ref(dequantize_ref(cq, sq), dequantize_ref(ck, sk), dequantize_ref(cv, sv))

    e0 = np.linalg.norm(run(False) - exact) / np.linalg.norm(exact)
    e1 = np.linalg.norm(run(True) - exact) / np.linalg.norm(exact)
    assert e1 < 0.6 * e0
