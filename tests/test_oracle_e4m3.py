"""Pins for the e4m3fn codec of the oracle (CPU only): torch's float8_e4m3fn
as a library routine, the published code table (tests/golden), the doubling
property the pages state, and exhaustive tie and saturation cases."""

import os

import numpy as np
import pytest
import torch

from oracle import e4m3_decode, e4m3_encode_rne_sat

pytestmark = pytest.mark.cpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3fn_codes.txt")


def test_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(ours[~nan], ref[~nan])


def test_golden_code_table():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                code, value = line.split()
                rows.append((int(code, 16), float(value)))
    assert len(rows) >= 10
    for code, value in rows:
        assert e4m3_decode(np.array([code], np.uint8))[0] == value, hex(code)
        assert e4m3_encode_rne_sat(np.array([value]))[0] == code, hex(code)


def test_code_grows_by_eight_per_doubling():
    # read as an integer, the code of 2^k is 56 + 8k over the normal range
    for k in range(-6, 9):
        assert int(e4m3_encode_rne_sat(np.array([2.0 ** k]))[0]) == 56 + 8 * k


def test_roundtrip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    back = e4m3_encode_rne_sat(e4m3_decode(codes))
    # +0 and -0 both decode to zero; -0.0 keeps its sign bit
    assert np.array_equal(back, codes)


def test_encode_matches_torch_on_random_fp32():
    g = np.random.default_rng(0)
    x = np.concatenate([
        g.standard_normal(200000).astype(np.float32) * s for s in (1e-4, 1e-2, 1.0, 30.0, 300.0)
    ]).astype(np.float32)
    x = np.clip(x, -448, 448)
    ours = e4m3_encode_rne_sat(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_ties_go_to_even_code():
    vals = e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2  # exact in fp64
    codes = e4m3_encode_rne_sat(mids)
    lo = np.arange(0x7E)
    expect = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(codes, expect.astype(np.uint8))
    ref = torch.from_numpy(mids.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)


def test_saturation_and_sign():
    x = np.array([448.0, 449.0, 464.0, 500.0, 1e30, -1e30, -448.0, -1e-30, 0.0, -0.0])
    c = e4m3_encode_rne_sat(x)
    assert list(c) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x80, 0x00, 0x80]
    assert e4m3_encode_rne_sat(np.array([np.nan]))[0] == 0x7F
