"""The whole-head oracle pool (``oracle/pool.py``) against the single-process
oracle: the pool only runs the pinned functions on separate heads, so its
per-head errors must equal those computed here directly, and a planted code
mismatch must be reported."""

import numpy as np
import pytest
import torch

from bf16_causal_prefill_flashattention_amd.inputs import Workload, make_qkv
from oracle import attn_ref, dequantize_ref, quantize_ref
from oracle.pool import HeadPool, head_parity, host_cores, summarize


def _tasks(q, k, v, out, fp8=None, codes=None):
    grp = q.shape[2] // k.shape[2]
    tasks = []
    for h in range(q.shape[2]):
        g = h // grp
        t = {"key": h, "q": q[0, :, h].numpy(), "k": k[0, :, g].numpy(), "v": v[0, :, g].numpy(),
             "out": out[0, :, h], "fp8": fp8}
        if codes is not None:
            cq, ck, cv, sq, sk, sv = codes
            t["codes"] = (cq[0, :, h], ck[0, :, g], cv[0, :, g], sq[0, h], sk[0, g], sv[0, g])
        tasks.append(t)
    return tasks


def test_host_cores_is_positive_and_capped():
    assert 1 <= host_cores() <= 16


def test_pool_matches_direct_oracle_bf16_values():
    w = Workload("t", "bf16", 1, 4, 2, 150, 128, 128, seed=21)
    q, k, v = (t.to(torch.bfloat16).float() for t in make_qkv(w))
    ref = attn_ref(q, k, v)
    out = ref + np.random.default_rng(0).normal(0, 1e-3, ref.shape)
    with HeadPool(2) as pool:
        res = pool.run(_tasks(q, k, v, out))
    assert [r["key"] for r in res] == [0, 1, 2, 3]
    s = summarize(res)
    direct = np.linalg.norm(out - ref) / np.linalg.norm(ref)
    assert s["rel_fro"] == pytest.approx(direct, rel=1e-12)
    for h, r in enumerate(res):
        ph = np.linalg.norm(out[0, :, h] - ref[0, :, h]) / np.linalg.norm(ref[0, :, h])
        assert s["per_head"][h] == pytest.approx(ph, rel=1e-12)
        assert r["max_abs"] == pytest.approx(np.abs(out[0, :, h] - ref[0, :, h]).max(), rel=1e-12)
    assert s["codes_equal"] is None


@pytest.mark.parametrize("hadamard", [False, True])
def test_pool_fp8_path_quantizes_like_the_oracle(hadamard):
    w = Workload("t", "fp8", 1, 2, 1, 130, 128, 128, outliers=4, seed=22)
    q, k, v = make_qkv(w)
    (cq, sq), (ck, sk), (cv, sv) = quantize_ref(q, hadamard), quantize_ref(k, hadamard), quantize_ref(v, False)
    ref = attn_ref(dequantize_ref(cq, sq), dequantize_ref(ck, sk), dequantize_ref(cv, sv))
    codes = (cq, ck, cv, sq, sk, sv)
    res = [head_parity(t) for t in _tasks(q, k, v, ref, {"hadamard": hadamard}, codes)]
    assert summarize(res)["rel_fro"] == 0.0 and summarize(res)["codes_equal"] is True
    bad = cq.copy()
    bad[0, 7, 1, 3] ^= 1  # one code of head 1 differs
    res = [head_parity(t) for t in _tasks(q, k, v, ref, {"hadamard": hadamard}, (bad,) + codes[1:])]
    assert [r["codes_equal"] for r in res] == [True, False]
    sbad = sk.copy()
    sbad[0, 0] = np.nextafter(sbad[0, 0], np.float32(1))  # a scale one ulp off
    res = [head_parity(t) for t in _tasks(q, k, v, ref, {"hadamard": hadamard}, codes[:4] + (sbad, sv))]
    assert not any(r["codes_equal"] for r in res)
