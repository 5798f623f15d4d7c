"""Pins for the chunked-prefill oracle ``attn_chunk_ref_rows`` (CPU only).

Checks from outside the function's own code: torch's fp64
scaled_dot_product_attention with an explicit bottom-right causal mask, scipy's
logsumexp for the LSE, brute force in 50-digit arithmetic (mpmath), the plain
causal oracle (itself pinned) as the Nq == Nk special case, the closed form for
equal scores, and the split-and-merge identity that defines what an LSE is for.
A dropped query offset, an LSE without the max, a misplaced chunk (top-left
instead of bottom-right) or a wrong scale fails at least one of them.
"""

import math
import os
import types

import mpmath
import numpy as np
import pytest
import torch
import torch.nn.functional as F
from scipy.special import logsumexp

from oracle import attn_chunk_ref_rows, attn_ref_rows

pytestmark = pytest.mark.cpu
ORACLE = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _inputs(B, Nq, Nk, Hq, Hkv, dqk, dv, seed=0):
    return (_rand((B, Nq, Hq, dqk), seed), _rand((B, Nk, Hkv, dqk), seed + 1), _rand((B, Nk, Hkv, dv), seed + 2))


def _mask(Nq, Nk):
    # bottom-right alignment: row i is position i + Nk - Nq
    return np.arange(Nk)[None, :] <= (np.arange(Nq) + Nk - Nq)[:, None]


def _sdpa_masked(q, k, v, tau):
    Nq, Nk = q.shape[1], k.shape[1]
    qt, kt, vt = (torch.from_numpy(t).permute(0, 2, 1, 3) for t in (q, k, v))
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(_mask(Nq, Nk)), scale=tau,
                                       enable_gqa=True)
    return o.permute(0, 2, 1, 3).numpy()


def _lse_scipy(q, k, tau):
    B, Nq, Hq, _ = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    out = np.zeros((B, Hq, Nq))
    for b in range(B):
        for h in range(Hq):
            s = tau * (torch.from_numpy(q[b, :, h]) @ torch.from_numpy(k[b, :, h // (Hq // Hkv)]).T).numpy()
            out[b, h] = logsumexp(np.where(_mask(Nq, Nk), s, -np.inf), axis=1)
    return out


@pytest.mark.parametrize("B,Nq,Nk,Hq,Hkv,dqk,dv", [
    (1, 1, 1, 1, 1, 8, 8), (1, 1, 37, 2, 2, 16, 16), (2, 20, 57, 4, 2, 32, 32), (1, 130, 300, 2, 1, 128, 128),
    (1, 64, 64, 2, 2, 192, 128), (1, 257, 1000, 3, 3, 32, 48),
])
def test_matches_sdpa_and_logsumexp(B, Nq, Nk, Hq, Hkv, dqk, dv):
    q, k, v = _inputs(B, Nq, Nk, Hq, Hkv, dqk, dv)
    tau = 1 / math.sqrt(dqk)
    out, lse = attn_chunk_ref_rows(q, k, v)
    np.testing.assert_allclose(out, _sdpa_masked(q, k, v, tau), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse, _lse_scipy(q, k, tau), rtol=1e-12, atol=1e-12)


def test_explicit_softmax_scale():
    q, k, v = _inputs(1, 30, 70, 2, 1, 16, 16, seed=5)
    out, lse = attn_chunk_ref_rows(q, k, v, softmax_scale=0.7)
    np.testing.assert_allclose(out, _sdpa_masked(q, k, v, 0.7), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse, _lse_scipy(q, k, 0.7), rtol=1e-12, atol=1e-12)


def test_equal_lengths_is_plain_causal_oracle():
    q, k, v = _inputs(1, 90, 90, 4, 2, 32, 32, seed=3)
    out, _ = attn_chunk_ref_rows(q, k, v)
    np.testing.assert_allclose(out, attn_ref_rows(q, k, v), rtol=1e-14, atol=1e-15)


def test_equal_scores_closed_form():
    # Q = 0: every visible key has weight 1/(p+1), lse = log(p+1), p = i + Nk - Nq
    Nq, Nk = 25, 60
    q = np.zeros((1, Nq, 2, 16))
    k, v = _rand((1, Nk, 1, 16), 7), _rand((1, Nk, 1, 16), 8)
    out, lse = attn_chunk_ref_rows(q, k, v)
    pos = np.arange(Nq) + Nk - Nq
    prefix_mean = np.cumsum(v[0, :, 0], axis=0) / np.arange(1, Nk + 1)[:, None]
    for h in range(2):
        np.testing.assert_allclose(out[0, :, h], prefix_mean[pos], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(lse[0, h], np.log(pos + 1.0), rtol=1e-15, atol=1e-15)


def test_split_and_merge_identity():
    # one row against all its keys equals the LSE-weighted merge of the same row
    # against two disjoint key ranges (each range fully visible to that row)
    q, k, v = _inputs(1, 12, 80, 2, 1, 16, 16, seed=11)
    out, lse = attn_chunk_ref_rows(q, k, v)
    for i, a in ((11, 40), (3, 1), (0, 60), (7, 75)):
        p = i + 80 - 12
        qi = q[:, i : i + 1]
        o1, l1 = attn_chunk_ref_rows(qi, k[:, :a], v[:, :a])  # Nq = 1: row sits at position a - 1
        o2, l2 = attn_chunk_ref_rows(qi, k[:, a : p + 1], v[:, a : p + 1])
        lm = np.logaddexp(l1, l2)  # [1, Hq, 1]
        w1 = np.exp(l1 - lm)[:, :, 0][:, None, :, None]
        w2 = np.exp(l2 - lm)[:, :, 0][:, None, :, None]
        np.testing.assert_allclose(w1 * o1 + w2 * o2, out[:, i : i + 1], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lm[:, :, 0], lse[:, :, i], rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("Nq,Nk", [(1, 1), (2, 5), (4, 6), (3, 3)])
def test_brute_force_mpmath(Nq, Nk):
    mpmath.mp.dps = 50
    q, k, v = _inputs(1, Nq, Nk, 2, 1, 4, 3, seed=Nq * 10 + Nk)
    out, lse = attn_chunk_ref_rows(q, k, v)
    tau = mpmath.mpf(1) / mpmath.sqrt(4)
    for h in range(2):
        for i in range(Nq):
            p = i + Nk - Nq
            s = [tau * mpmath.fsum(mpmath.mpf(q[0, i, h, c]) * mpmath.mpf(k[0, j, 0, c]) for c in range(4))
                 for j in range(p + 1)]
            z = mpmath.fsum(mpmath.exp(x) for x in s)
            assert abs(float(mpmath.log(z)) - lse[0, h, i]) <= 1e-14 * max(1.0, abs(lse[0, h, i]))
            for c in range(3):
                o = mpmath.fsum(mpmath.exp(s[j]) * mpmath.mpf(v[0, j, 0, c]) for j in range(p + 1)) / z
                assert abs(float(o) - out[0, i, h, c]) <= 1e-14


def test_rejects_more_queries_than_keys():
    q, k, v = _inputs(1, 5, 4, 1, 1, 8, 8)
    with pytest.raises(ValueError):
        attn_chunk_ref_rows(q, k, v)


# ---- planted mistakes in a copy of the source: each must fail a pin above
def _load_mutant(old, new):
    src = open(os.path.join(ORACLE, "attention.py")).read()
    assert old in src, old
    mod = types.ModuleType("mutant")
    exec(compile(src.replace(old, new, 1), "attention.py", "exec"), mod.__dict__)
    return mod


def _pins_pass(fn):
    q, k, v = _inputs(1, 20, 57, 4, 2, 32, 32)
    tau = 1 / math.sqrt(32)
    out, lse = fn(q, k, v)
    return (np.allclose(out, _sdpa_masked(q, k, v, tau), rtol=1e-10, atol=1e-12)
            and np.allclose(lse, _lse_scipy(q, k, tau), rtol=1e-12, atol=1e-12))


CHUNK_MUTANTS = [
    ("pos = r + off  #", "pos = r  #"),  # chunk placed top-left (offset dropped)
    ("(m + np.log(l))[:, 0]", "(np.log(l))[:, 0]"),  # LSE without the max
    ("lse[b, h, s0 : s0 + r.size] = (m + np.log(l))[:, 0]", "lse[b, h, s0 : s0 + r.size] = (m + np.log(l / hi))[:, 0]"),
    ("hi = int(pos.max()) + 1  # keys", "hi = int(pos.max())  # keys"),  # last visible key dropped
]


@pytest.mark.parametrize("old,new", CHUNK_MUTANTS)
def test_chunk_mutants_are_caught(old, new):
    assert not _pins_pass(_load_mutant(old, new).attn_chunk_ref_rows)


def test_unmutated_chunk_copy_passes():
    assert _pins_pass(_load_mutant("import math", "import math").attn_chunk_ref_rows)
