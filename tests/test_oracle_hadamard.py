"""Pins for the oracle's 128-point Hadamard rotation (CPU only): scipy's
Hadamard matrix (library routine), orthogonality, exactness on integer inputs,
and the dot-product preservation that makes rotating Q and K harmless."""

import numpy as np
import pytest
import scipy.linalg

from oracle import fwht128_f32, sylvester_hadamard

pytestmark = pytest.mark.cpu


def test_sylvester_matches_scipy():
    for n in (1, 2, 4, 64, 128):
        assert np.array_equal(sylvester_hadamard(n), scipy.linalg.hadamard(n))


def test_orthogonality():
    h = sylvester_hadamard(128)
    assert np.array_equal(h @ h.T, 128 * np.eye(128, dtype=np.int64))


def test_fwht_exact_on_small_integers():
    g = np.random.default_rng(0)
    x = g.integers(-1000, 1000, size=(300, 128)).astype(np.float32)
    ref = x.astype(np.int64) @ scipy.linalg.hadamard(128)
    assert np.array_equal(fwht128_f32(x).astype(np.int64), ref)


def test_fwht_close_to_fp64_product_on_gaussian():
    g = np.random.default_rng(1)
    x = (g.standard_normal((1000, 128)) * 3).astype(np.float32)
    ref = x.astype(np.float64) @ scipy.linalg.hadamard(128).astype(np.float64)
    y = fwht128_f32(x)
    assert y.dtype == np.float32
    # 7 rounded stages on values up to ~sqrt(128)*|x|: error within 7 ulp(|sum|)
    bound = 7 * np.spacing(np.abs(x).sum(axis=1, keepdims=True).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(y - ref) <= bound)


def test_fwht_keeps_leading_axes_and_preserves_dot_products():
    g = np.random.default_rng(2)
    q = g.standard_normal((2, 9, 3, 128)).astype(np.float32)
    k = g.standard_normal((2, 9, 3, 128)).astype(np.float32)
    qr, kr = fwht128_f32(q), fwht128_f32(k)
    assert qr.shape == q.shape
    lhs = np.einsum("bnhd,bmhd->bhnm", qr.astype(np.float64), kr.astype(np.float64)) / 128.0
    rhs = np.einsum("bnhd,bmhd->bhnm", q.astype(np.float64), k.astype(np.float64))
    np.testing.assert_allclose(lhs, rhs, rtol=1e-5, atol=1e-4)
