"""GPU chunked prefill (``attn_fwd_chunk`` through the C ABI) against the fp64
oracle ``attn_chunk_ref_rows``.

The queries are the last Nq positions of a seeded sequence of Nk tokens (the
inputs of a chunked prefill).  Output: relative Frobenius error <= 1e-2 (BF16)
or 6e-2 (FP8), as for the plain path.  LSE (natural log), absolute error:

* BF16: the probabilities fed to the row sum are rounded to bf16 (relative
  error <= 2^-9, so |d lse| <= ln(1 + 2^-9) ~ 2e-3) and the fp32 scores carry
  accumulation error well below that: bound 5e-3.
* FP8: a probability 2^t (t = x - m + 6, log2 units, with the running
  reference m within [row max - 2.75, row max + 1/8]) becomes the e4m3 code
  round(8t + 55.66).  For t >= -5.96 (normal codes) its log error lies in
  [-0.0728, +0.0728] (the extremes of ln e4m3(round(8t + 55.66)) - t ln 2);
  below that the subnormal codes only under-represent it, down to zero.  So per
  row: lse_gpu - lse <= 0.0728, and lse_gpu - lse >= -0.0728 + ln(1 - f),
  where f is the share of the row's softmax mass on keys more than
  5.96 + 6 - 1/8 = 11.835 below the row max in log2 units (computed from the
  oracle's scores).  The scores themselves come from FP8 MFMAs, which sum the
  products of one instruction with about 12 bits of precision relative to the
  largest of them (measured: sums 2.4e-4 to 4.3e-4 low when one product
  dominates), so each log2-domain score is off by at most
  2^-10 * tau * log2(e) * sum_c |q_c k_c| (a 2-4x margin), and the LSE by at
  most ln 2 times the largest such bound over the row's visible keys -- large
  only for rows with outlier channels.  Plus 1e-3 for fp32 arithmetic and logs.

FP8 inputs are quantized by the oracle's quantizer on the CPU and the same
codes are uploaded, so the oracle's inputs never come from the GPU.
"""

import numpy as np
import pytest
import torch

import bf16_causal_prefill_flashattention_amd as miattn
from bf16_causal_prefill_flashattention_amd.inputs import Workload, make_qkv
from oracle import attn_chunk_ref_rows, dequantize_ref, quantize_ref
from parity_util import TOL, rel_fro

pytestmark = pytest.mark.gpu
LSE_TOL_BF16 = 5e-3
LEAN_LOG_ERR = 0.0728
LOG2_FLOOR = 11.835


def _fp8_lse_slack(ref_in, rows=None, softmax_scale=None):
    """Per [b, h, row]: (-ln(1 - f), score bound) as in the module docstring."""
    q, k = (np.asarray(t, np.float64) for t in ref_in[:2])
    B, Nq, Hq, dqk = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    c = (1 / np.sqrt(dqk) if softmax_scale is None else softmax_scale) * np.log2(np.e)
    rows = np.arange(Nq) if rows is None else rows
    lost_slack, score_slack = np.zeros((B, Hq, len(rows))), np.zeros((B, Hq, len(rows)))
    for b in range(B):
        for h in range(Hq):
            kh = k[b, :, h // (Hq // Hkv)]
            visible = np.arange(Nk)[None, :] <= (rows + Nk - Nq)[:, None]
            x = np.where(visible, c * (q[b, rows, h] @ kh.T), -np.inf)
            e = np.exp2(x - x.max(axis=1, keepdims=True))
            lost = np.where(e < 2.0 ** -LOG2_FLOOR, e, 0).sum(axis=1) / e.sum(axis=1)
            lost_slack[b, h] = -np.log1p(-np.minimum(lost, 1 - 1e-12))
            mag = np.where(visible, c * (np.abs(q[b, rows, h]) @ np.abs(kh).T), 0)
            score_slack[b, h] = np.log(2) * 2.0 ** -10 * mag.max(axis=1)
    return lost_slack, score_slack


def _check_lse(dtype, lse, ref_lse, ref_in, rows=None, softmax_scale=None):
    d = lse - ref_lse
    if dtype == "bf16":
        assert float(np.abs(d).max()) <= LSE_TOL_BF16, float(np.abs(d).max())
        return
    lost, score = _fp8_lse_slack(ref_in, rows, softmax_scale)
    hi = LEAN_LOG_ERR + 1e-3 + score
    lo = -(LEAN_LOG_ERR + 1e-3 + score + lost)
    assert bool((d <= hi).all()), float((d - hi).max())
    assert bool((d >= lo).all()), float((d - lo).min())


def _case(dtype, B, Nq, Nk, Hq, Hkv, dqk, seed, outliers=0):
    """Seeded chunk inputs: fp32 q (last Nq rows), k, v on the CPU."""
    w = Workload("chunk", dtype, B, Hq, Hkv, Nk, dqk, 128, outliers=outliers, seed=seed)
    q, k, v = make_qkv(w)
    return q[:, Nk - Nq:].contiguous(), k, v


def _run(dtype, q, k, v, softmax_scale=None, with_lse=True):
    """GPU call and the oracle inputs (fp64 arrays) it corresponds to."""
    if dtype == "bf16":
        qb, kb, vb = (t.to(torch.bfloat16) for t in (q, k, v))
        out, lse = miattn.attn_fwd_chunk(qb.cuda(), kb.cuda(), vb.cuda(), softmax_scale=softmax_scale,
                                         with_lse=with_lse)
        ref_in = (qb, kb, vb)
    else:
        (cq, sq), (ck, sk), (cv, sv) = quantize_ref(q), quantize_ref(k), quantize_ref(v)
        dev = [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in (cq, ck, cv, sq, sk, sv)]
        out, lse = miattn.attn_fwd_chunk(*dev, softmax_scale=softmax_scale, with_lse=with_lse)
        ref_in = (dequantize_ref(cq, sq), dequantize_ref(ck, sk), dequantize_ref(cv, sv))
    torch.cuda.synchronize()
    return out.cpu(), (None if lse is None else lse.cpu().numpy().astype(np.float64)), ref_in


CASES = [
    # (B, Nq, Nk, Hq, Hkv, d_qk)
    (1, 1, 1, 2, 2, 128),  # one token
    (1, 1, 777, 2, 1, 128),  # one query after a long prefix
    (1, 300, 1000, 4, 2, 128),  # ragged chunk, GQA
    (2, 256, 256, 2, 2, 128),  # Nq == Nk: plain causal prefill
    (1, 700, 701, 4, 4, 128),  # offset of one
    (1, 64, 2048, 8, 2, 128),  # short chunk, long prefix
    (1, 129, 513, 2, 2, 192),  # MLA shape, ragged
    (1, 1000, 1500, 2, 2, 192),
]


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("B,Nq,Nk,Hq,Hkv,dqk", CASES)
def test_chunk_matches_oracle(require_gpu, dtype, B, Nq, Nk, Hq, Hkv, dqk):
    q, k, v = _case(dtype, B, Nq, Nk, Hq, Hkv, dqk, seed=Nq + 7 * Nk + Hq)
    out, lse, ref_in = _run(dtype, q, k, v)
    ref, ref_lse = attn_chunk_ref_rows(*ref_in)
    err = rel_fro(out, ref)
    assert err <= TOL[dtype], err
    assert torch.isfinite(out.float()).all()
    _check_lse(dtype, lse, ref_lse, ref_in)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("tau", [0.02, 0.3])
def test_explicit_softmax_scale(require_gpu, dtype, tau):
    q, k, v = _case(dtype, 1, 200, 600, 2, 1, 128, seed=3, outliers=0)
    out, lse, ref_in = _run(dtype, q, k, v, softmax_scale=tau)
    ref, ref_lse = attn_chunk_ref_rows(*ref_in, softmax_scale=tau)
    assert rel_fro(out, ref) <= TOL[dtype]
    _check_lse(dtype, lse, ref_lse, ref_in, softmax_scale=tau)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_outlier_inputs_peaked_rows(require_gpu, dtype):
    # aligned outlier channels make most rows nearly one-hot
    q, k, v = _case(dtype, 1, 333, 1200, 8, 2, 128, seed=21, outliers=4)
    out, lse, ref_in = _run(dtype, q, k, v)
    ref, ref_lse = attn_chunk_ref_rows(*ref_in)
    assert rel_fro(out, ref) <= TOL[dtype]
    _check_lse(dtype, lse, ref_lse, ref_in)


def test_two_chunks_reproduce_the_whole_prefill(require_gpu):
    # chunked prefill: positions [0, c) with attn_fwd, then [c, N) against all N keys
    N, c = 1500, 600
    q, k, v = (t.to(torch.bfloat16) for t in _case("bf16", 1, N, N, 4, 2, 128, seed=5))
    first = miattn.attn_fwd(q[:, :c].contiguous().cuda(), k[:, :c].contiguous().cuda(), v[:, :c].contiguous().cuda())
    second, _ = miattn.attn_fwd_chunk(q[:, c:].contiguous().cuda(), k.cuda(), v.cuda(), with_lse=False)
    torch.cuda.synchronize()
    out = torch.cat([first.cpu(), second.cpu()], dim=1)
    ref, _ = attn_chunk_ref_rows(q, k, v)
    assert rel_fro(out, ref) <= TOL["bf16"]


def test_equal_length_chunk_is_attn_fwd_bitwise(require_gpu):
    # same kernel, same decomposition: Nq == Nk with the default scale is attn_fwd
    q, k, v = (t.to(torch.bfloat16).cuda() for t in _case("bf16", 1, 999, 999, 4, 2, 128, seed=9))
    a = miattn.attn_fwd(q, k, v)
    b, _ = miattn.attn_fwd_chunk(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_zero_queries_give_prefix_mean_and_log_count(require_gpu, dtype):
    # Q = 0: uniform weights over the p + 1 visible keys, lse = ln(p + 1)
    Nq, Nk = 100, 900
    _, k, v = _case(dtype, 1, Nq, Nk, 2, 2, 128, seed=13)
    q = torch.zeros(1, Nq, 2, 128)  # FP8: all-zero q quantizes to code 0 with scale 1
    out, lse, ref_in = _run(dtype, q, k, v)
    pos = np.arange(Nq) + Nk - Nq
    _check_lse(dtype, lse, np.broadcast_to(np.log(pos + 1.0), lse.shape), ref_in)
    ref, _ = attn_chunk_ref_rows(*ref_in)
    assert rel_fro(out, ref) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_bitwise_deterministic_20_launches(require_gpu, dtype):
    q, k, v = _case(dtype, 1, 500, 1300, 4, 2, 128, seed=17)
    out0, lse0, _ = _run(dtype, q, k, v)
    for _ in range(19):
        out, lse, _ = _run(dtype, q, k, v)
        assert torch.equal(out.view(torch.int16), out0.view(torch.int16))
        assert np.array_equal(lse, lse0)


def test_writes_stay_inside_out_and_lse(require_gpu):
    B, Nq, Nk, Hq, Hkv = 1, 77, 300, 2, 1
    q, k, v = (t.to(torch.bfloat16).cuda() for t in _case("bf16", B, Nq, Nk, Hq, Hkv, 128, seed=19))
    guard_o = torch.full((3, B * Nq * Hq * 128), 7.0, dtype=torch.bfloat16, device="cuda")
    guard_l = torch.full((3, B * Hq * Nq), 7.0, dtype=torch.float32, device="cuda")
    out = guard_o[1].view(B, Nq, Hq, 128)
    lse = guard_l[1].view(B, Hq, Nq)
    miattn.attn_fwd_chunk(q, k, v, out=out, lse=lse)
    torch.cuda.synchronize()
    for g in (guard_o, guard_l):
        assert bool((g[0] == 7.0).all()) and bool((g[2] == 7.0).all())
    assert bool(torch.isfinite(lse).all())


def test_full_size_chunk_sampled_rows(require_gpu):
    """The benchmarked chunk: the last 8192 positions of a 32768-token FP8
    sequence (B=1, 32 heads, d=128), quantized on the GPU; sampled heads are
    re-quantized by the oracle (codes and scales must match bit for bit) and
    sampled rows compared."""
    B, Nq, Nk, H = 1, 8192, 32768, 32
    q, k, v = _case("fp8", B, Nq, Nk, H, H, 128, seed=0)
    cq, sq = miattn.attn_quantize_fp8(q.cuda())
    ck, sk = miattn.attn_quantize_fp8(k.cuda())
    cv, sv = miattn.attn_quantize_fp8(v.cuda())
    out, lse = miattn.attn_fwd_chunk(cq, ck, cv, sq, sk, sv)
    torch.cuda.synchronize()
    out, lse = out.cpu(), lse.cpu().numpy().astype(np.float64)
    g = np.random.default_rng(1)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, Nq // 2, Nq - 2, Nq - 1], g.integers(0, Nq, 12)]))
    errs, lse_errs = [], []
    for h in (0, 13, 31):
        rq, rsq = quantize_ref(q[:, :, h:h + 1])
        rk, rsk = quantize_ref(k[:, :, h:h + 1])
        rv, rsv = quantize_ref(v[:, :, h:h + 1])
        assert np.array_equal(cq[:, :, h:h + 1].cpu().numpy(), rq)
        assert np.array_equal(ck[:, :, h:h + 1].cpu().numpy(), rk)
        assert np.array_equal(cv[:, :, h:h + 1].cpu().numpy(), rv)
        for dev_s, ref_s in ((sq, rsq), (sk, rsk), (sv, rsv)):
            assert dev_s[:, h].cpu().numpy().view(np.uint32)[0] == ref_s.view(np.uint32)[0, 0]
        ref, ref_lse = attn_chunk_ref_rows(dequantize_ref(rq, rsq), dequantize_ref(rk, rsk),
                                           dequantize_ref(rv, rsv), rows=rows)
        errs.append(rel_fro(out[:, rows, h:h + 1], ref))
        ref_in = (dequantize_ref(rq, rsq), dequantize_ref(rk, rsk), None)
        _check_lse("fp8", lse[:, h:h + 1, rows], ref_lse, ref_in, rows=rows)
    assert max(errs) <= TOL["fp8"], errs


@pytest.mark.parametrize("fp8,hadamard,Nq,Nk,tau,ret", [
    (False, False, 500, 500, None, False), (False, False, 300, 900, 0.1, True),
    (True, False, 700, 700, None, False), (True, True, 256, 1024, None, True), (True, False, 64, 2000, 0.05, True),
])
def test_flash_attn_func_drop_in(require_gpu, fp8, hadamard, Nq, Nk, tau, ret):
    """BF16 tensors in; with fp8=True the library quantizes (and rotates) them.
    The oracle runs on the inputs the kernel consumed: the BF16 values, or the
    oracle quantizer's codes (which the GPU quantizer matches bit for bit)."""
    q, k, v = (t.to(torch.bfloat16) for t in _case("bf16", 1, Nq, Nk, 4, 2, 128, seed=Nq + Nk))
    res = miattn.flash_attn_func(q.cuda(), k.cuda(), v.cuda(), softmax_scale=tau, return_lse=ret, fp8=fp8,
                                 hadamard=hadamard)
    torch.cuda.synchronize()
    out, lse = res if ret else (res, None)
    if fp8:
        (cq, sq), (ck, sk), (cv, sv) = quantize_ref(q, hadamard), quantize_ref(k, hadamard), quantize_ref(v, False)
        ref_in = (dequantize_ref(cq, sq), dequantize_ref(ck, sk), dequantize_ref(cv, sv))
    else:
        ref_in = (q, k, v)
    ref, ref_lse = attn_chunk_ref_rows(*ref_in, softmax_scale=tau)
    dtype = "fp8" if fp8 else "bf16"
    assert rel_fro(out.cpu(), ref) <= TOL[dtype]
    if ret:
        _check_lse(dtype, lse.cpu().numpy().astype(np.float64), ref_lse, ref_in, softmax_scale=tau)
