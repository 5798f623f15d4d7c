"""Pins for the fp64 attention oracle (CPU only).

Each check comes from outside the oracle's own code: a library routine
(torch's fp64 scaled_dot_product_attention on CPU, with GQA), brute force in
50-digit arithmetic (mpmath), or a property the definition fixes exactly.  A
plausible slip -- dropped or wrong softmax scale, off-by-one causal mask, wrong
grouped-query mapping, softmax over the wrong axis, a transposed operand --
fails at least one of them.
"""

import math

import mpmath
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attn_ref, attn_ref_rows, causal_weights_ref
from bf16_causal_prefill_flashattention_amd.inputs import WORKLOADS, make_qkv

pytestmark = pytest.mark.cpu


def _rand(shape, seed):
    g = np.random.default_rng(seed)
    return g.standard_normal(shape)


def _sdpa(q, k, v):
    # torch wants [B, H, N, d]; GQA maps query head h to kv head h // (Hq/Hkv)
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)
    kt = torch.from_numpy(k).permute(0, 2, 1, 3)
    vt = torch.from_numpy(v).permute(0, 2, 1, 3)
    o = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True, enable_gqa=True)
    return o.permute(0, 2, 1, 3).numpy()


@pytest.mark.parametrize(
    "B,N,Hq,Hkv,dqk,dv",
    [(1, 1, 1, 1, 8, 8), (2, 37, 2, 2, 16, 16), (1, 130, 4, 2, 128, 128),
     (1, 65, 8, 2, 128, 128), (1, 70, 2, 2, 192, 128), (1, 300, 6, 3, 32, 48)],
)
def test_matches_torch_sdpa_fp64(B, N, Hq, Hkv, dqk, dv):
    q = _rand((B, N, Hq, dqk), 1)
    k = _rand((B, N, Hkv, dqk), 2)
    v = _rand((B, N, Hkv, dv), 3)
    ref = _sdpa(q, k, v)
    out = attn_ref(q, k, v)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def _mp_attention(q, k, v, dps=50):
    mpmath.mp.dps = dps
    B, N, Hq, dqk = q.shape
    Hkv, dv = k.shape[2], v.shape[3]
    tau = mpmath.mpf(1) / mpmath.sqrt(dqk)
    out = np.zeros((B, N, Hq, dv))
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            for i in range(N):
                s = [tau * mpmath.fsum(mpmath.mpf(q[b, i, h, c]) * mpmath.mpf(k[b, j, g, c])
                                       for c in range(dqk)) for j in range(i + 1)]
                e = [mpmath.exp(x) for x in s]
                z = mpmath.fsum(e)
                for c in range(dv):
                    out[b, i, h, c] = float(mpmath.fsum(e[j] * mpmath.mpf(v[b, j, g, c])
                                                        for j in range(i + 1)) / z)
    return out


@pytest.mark.parametrize("N,Hq,Hkv,d", [(1, 1, 1, 2), (5, 2, 1, 4), (6, 2, 2, 3)])
def test_brute_force_mpmath(N, Hq, Hkv, d):
    q = _rand((1, N, Hq, d), 10) * 2.0
    k = _rand((1, N, Hkv, d), 11) * 2.0
    v = _rand((1, N, Hkv, d + 1), 12)
    ref = _mp_attention(q, k, v)
    out = attn_ref(q, k, v)
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-14)


def test_weights_rows_sum_to_one_and_causal_zeros():
    q = _rand((1, 200, 2, 64), 20) * 3
    k = _rand((1, 200, 2, 64), 21) * 3
    for h in range(2):
        w = causal_weights_ref(q, k, 0, h)
        assert np.all(np.abs(w.sum(axis=1) - 1.0) <= 1e-14)
        assert np.all(w[np.triu_indices(200, 1)] == 0.0)
        assert np.all(w >= 0)


def test_weights_of_two_keys_are_a_logistic_of_the_scaled_score_gap():
    """Closed form that fixes tau: row 1 sees keys 0 and 1, so its weight on key
    1 is 1 / (1 + exp(-tau (s1 - s0))), s_j = <q_1, k_j>; checked at the default
    tau = 1/sqrt(d) and at explicit scales."""
    rng = np.random.default_rng(40)
    d = 64
    q = rng.standard_normal((1, 2, 1, d))
    k = rng.standard_normal((1, 2, 1, d))
    gap = float(q[0, 1, 0] @ k[0, 1, 0] - q[0, 1, 0] @ k[0, 0, 0])
    for tau in (None, 0.05, 0.3, 1.0):
        t = 1.0 / math.sqrt(d) if tau is None else tau
        w = causal_weights_ref(q, k, softmax_scale=tau)
        assert w[0, 0] == 1.0 and w[0, 1] == 0.0
        assert abs(w[1, 1] - 1.0 / (1.0 + math.exp(-t * gap))) <= 1e-15
        assert abs(w[1, 0] - 1.0 / (1.0 + math.exp(t * gap))) <= 1e-15


def test_zero_queries_give_uniform_weights_and_weights_reproduce_the_output():
    """Q = 0: W[i, j] = 1 / (i + 1) for j <= i (any tau).  Random inputs with
    GQA: W @ V of each head equals attn_ref's output, which the SDPA and
    brute-force pins fix."""
    N = 40
    q0 = np.zeros((1, N, 2, 32))
    k = _rand((1, N, 1, 32), 41)
    w = causal_weights_ref(q0, k, 0, 1, softmax_scale=0.7)
    expect = np.tril(np.ones((N, N))) / np.arange(1, N + 1)[:, None]
    np.testing.assert_allclose(w, expect, rtol=0, atol=1e-15)
    q = _rand((1, N, 4, 32), 42)
    k = _rand((1, N, 2, 32), 43)
    v = _rand((1, N, 2, 16), 44)
    out = attn_ref(q, k, v)
    for h in range(4):
        w = causal_weights_ref(q, k, 0, h)
        np.testing.assert_allclose(w @ v[0, :, h // 2, :], out[0, :, h, :], rtol=1e-12, atol=1e-13)


def test_row_zero_is_first_value_row_exactly():
    q = _rand((2, 50, 4, 128), 30)
    k = _rand((2, 50, 2, 128), 31)
    v = _rand((2, 50, 2, 128), 32)
    out = attn_ref(q, k, v)
    for h in range(4):
        assert np.array_equal(out[:, 0, h, :], v[:, 0, h // 2, :])


def test_equal_scores_give_prefix_mean():
    N = 257
    q = np.zeros((1, N, 2, 128))
    k = _rand((1, N, 1, 128), 40)
    v = _rand((1, N, 1, 128), 41)
    out = attn_ref(q, k, v)
    prefix_mean = np.cumsum(v[0, :, 0, :], axis=0) / np.arange(1, N + 1)[:, None]
    for h in range(2):
        np.testing.assert_allclose(out[0, :, h, :], prefix_mean, rtol=1e-12, atol=1e-13)


def test_key_value_permutation_inside_window():
    N, kk = 90, 40
    q = _rand((1, N, 2, 32), 50)
    k = _rand((1, N, 2, 32), 51)
    v = _rand((1, N, 2, 16), 52)
    perm = np.random.default_rng(53).permutation(kk + 1)
    k2, v2 = k.copy(), v.copy()
    k2[:, : kk + 1] = k[:, perm]
    v2[:, : kk + 1] = v[:, perm]
    a = attn_ref(q, k, v)
    b = attn_ref(q, k2, v2)
    np.testing.assert_allclose(a[:, kk:], b[:, kk:], rtol=1e-12, atol=1e-13)
    assert not np.allclose(a[:, 1:kk], b[:, 1:kk])  # rows inside the window do change


def test_row_constant_score_shift_and_linearity_in_v():
    q = _rand((1, 64, 2, 32), 60)
    k = _rand((1, 64, 1, 32), 61)
    v = _rand((1, 64, 1, 32), 62)
    u = _rand((32,), 63)
    a = attn_ref(q, k, v)
    b = attn_ref(q, k + u, v)  # s_ij += tau <q_i, u>, constant in j
    np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-12)
    v2 = _rand((1, 64, 1, 32), 64)
    np.testing.assert_allclose(attn_ref(q, k, 2.0 * v - 3.0 * v2), 2.0 * a - 3.0 * attn_ref(q, k, v2),
                               rtol=1e-11, atol=1e-12)


def test_last_row_is_full_attention():
    from scipy.special import softmax

    q = _rand((1, 33, 1, 128), 70)
    k = _rand((1, 33, 1, 128), 71)
    v = _rand((1, 33, 1, 128), 72)
    s = (k[0, :, 0, :] @ q[0, -1, 0, :]) / math.sqrt(128)
    full = softmax(s) @ v[0, :, 0, :]
    np.testing.assert_allclose(attn_ref(q, k, v)[0, -1, 0], full, rtol=1e-12, atol=1e-13)


def test_one_hot_row_selects_value():
    # a key aligned with the query at a huge norm takes all the weight
    N, d = 20, 16
    q = np.zeros((1, N, 1, d))
    k = _rand((1, N, 1, d), 80) * 0.01
    v = _rand((1, N, 1, d), 81)
    q[0, 15, 0, 0] = 100.0
    k[0, 7, 0, 0] = 100.0
    out = attn_ref(q, k, v)
    np.testing.assert_allclose(out[0, 15, 0], v[0, 7, 0], rtol=0, atol=1e-12)


def test_rows_subset_equals_full():
    q = _rand((1, 300, 4, 128), 90)
    k = _rand((1, 300, 2, 128), 91)
    v = _rand((1, 300, 2, 128), 92)
    rows = np.array([0, 1, 63, 64, 200, 299])
    np.testing.assert_array_equal(attn_ref_rows(q, k, v, rows), attn_ref(q, k, v)[:, rows])


def test_workload_generator_outliers_are_aligned():
    w = WORKLOADS["bf16_gqa_n16k"].with_(N=64)
    q, k, v = make_qkv(w)
    # the 4 boosted channels of kv head g are the 4 largest-variance channels of
    # K[:, :, g] and of Q for every query head of g's group
    grp = w.Hq // w.Hkv
    for g in range(w.Hkv):
        kc = set(torch.topk(k[0, :, g, :].pow(2).mean(0), 4).indices.tolist())
        for h in range(g * grp, (g + 1) * grp):
            qc = set(torch.topk(q[0, :, h, :].pow(2).mean(0), 4).indices.tolist())
            assert qc == kc
    assert float(v.abs().max()) < 8.0
