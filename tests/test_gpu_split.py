"""Key-split launches (``attn_fwd_ws`` through the C ABI) against the fp64 oracle.

A launch whose 256-query tiles leave compute units idle cuts every query tile
into ranges of at most L key tiles and merges the ranges of a tile through
their log-sum-exp.  The merge is exact in real arithmetic -- softmax over the
union of key ranges equals the log-sum-exp-weighted average of the per-range
softmax outputs -- so the same gates as the unsplit path apply: relative
Frobenius error <= 1e-2 (BF16) / 6e-2 (FP8) on the inputs the kernel consumed,
and the LSE bounds derived in test_gpu_chunk.py.

The plan (L, ranges per (batch, head)) is recomputed here from its rule and
checked against the byte count ``attn_fwd_ws_size`` reports, so every case
below is known to split (or, where stated, not to).
"""

import numpy as np
import pytest
import torch

import bf16_causal_prefill_flashattention_amd as miattn
from bf16_causal_prefill_flashattention_amd.inputs import WORKLOADS, Workload, make_inputs, make_qkv
from oracle import (attn_chunk_ref_rows, dequantize_block64_ref, dequantize_ref, quantize_block64_ref,
                    quantize_ref)
from parity_util import TOL, rel_fro
from test_gpu_chunk import _check_lse

pytestmark = pytest.mark.gpu
QT = 256


SHORT_KEYS = 4096  # launches with at most this many keys use 128-key tiles instead of 192


def tile_keys(fp8, dqk, block64, p_mode, Nk):
    if not fp8:
        return 128 if dqk == 128 else 64
    long_tiles = dqk == 128 and p_mode not in ("lean_block", "exact_block") and Nk > SHORT_KEYS
    return 192 if long_tiles else 128


def expected_plan(B, Hq, Nq, Nk, dqk, fp8, block64, p_mode, cus):
    """(L, units per (batch, head)) of the split rule, or None (no split): the
    smallest L that gives every key range a CU, or a doubling of it, whichever
    has the least modelled time, if that beats the unsplit launch."""
    nbh, nqt = B * Hq, (Nq + QT - 1) // QT
    if nbh * nqt > cus:
        return None
    bn = tile_keys(fp8, dqk, block64, p_mode, Nk)
    T = [(min((j + 1) * QT, Nq) + Nk - Nq - 1) // bn + 1 for j in range(nqt)]
    ranges = lambda L: [(t + L - 1) // L for t in T]  # noqa: E731
    L0 = next(L for L in range(1, T[-1] + 1) if nbh * sum(ranges(L)) <= cus)
    tile_us = bn * (dqk + 128) / (2.0 if fp8 else 1.0) / 24576.0

    def split_us(L):
        rows = sum(r * min(QT, Nq - j * QT) for j, r in enumerate(ranges(L)) if r > 1)
        return L * tile_us + nbh * rows * 129 * 4 * 0.55e-6 + 2.0

    best, best_us, L = None, T[-1] * tile_us, max(L0, 2)
    while L <= T[-1] - 2:
        t = split_us(L)
        if t < best_us:
            best, best_us = L, t
        L *= 2
    return None if best is None else (best, sum(ranges(best)))


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def _plan_checked(B, Hq, Hkv, Nq, Nk, dqk, fp8, scales="head", p_mode="lean_tile"):
    plan = expected_plan(B, Hq, Nq, Nk, dqk, fp8, scales == "block64", p_mode, _cus())
    n = miattn.attn_fwd_ws_size(B, Hq, Hkv, Nq, Nk, dqk, 128, fp8, scales, p_mode)
    assert n == (0 if plan is None else B * Hq * plan[1] * QT * 129 * 4), (plan, n)
    return plan


def _inputs(dtype, B, Nq, Nk, Hq, Hkv, dqk, seed, scales="head", outliers=0):
    w = Workload("split", dtype, B, Hq, Hkv, Nk, dqk, 128, outliers=outliers, seed=seed)
    q, k, v = make_qkv(w)
    q = q[:, Nk - Nq:].contiguous()
    if dtype == "bf16":
        qb, kb, vb = (t.to(torch.bfloat16) for t in (q, k, v))
        return [t.cuda() for t in (qb, kb, vb)], (qb, kb, vb)
    quant = quantize_block64_ref if scales == "block64" else quantize_ref
    deq = dequantize_block64_ref if scales == "block64" else dequantize_ref
    (cq, sq), (ck, sk), (cv, sv) = quant(q), quant(k), quant(v)
    dev = [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in (cq, ck, cv, sq, sk, sv)]
    return dev, (deq(cq, sq), deq(ck, sk), deq(cv, sv))


CASES = [
    # (dtype, B, Nq, Nk, Hq, Hkv, d_qk, scales, p_mode)
    ("fp8", 1, 2000, 2000, 2, 1, 128, "head", "lean_tile"),  # 128-key tiles (short), ragged last query tile
    ("fp8", 1, 1200, 5000, 2, 1, 128, "head", "lean_tile"),  # 192-key tiles, ragged, after a key prefix
    ("fp8", 1, 2000, 2000, 2, 2, 128, "head", "exact"),
    ("fp8", 2, 2500, 2500, 1, 1, 192, "head", "lean_tile"),  # MLA shape, 128-key tiles, two sequences
    ("fp8", 1, 1500, 1500, 2, 2, 128, "block64", "lean"),
    ("fp8", 1, 1500, 1500, 2, 2, 128, "block64", "lean_block"),
    ("fp8", 1, 300, 9000, 4, 1, 128, "head", "lean_tile"),  # short chunk, long prefix
    ("fp8", 1, 300, 9000, 4, 2, 128, "block64", "lean_tile"),  # block scales on 192-key tiles, split
    ("fp8", 1, 1, 5000, 2, 2, 128, "head", "exact_tile"),  # one query
    ("bf16", 1, 1800, 1800, 2, 1, 128, "head", "lean"),  # 128-key tiles
    ("bf16", 1, 1000, 1000, 2, 2, 192, "head", "lean"),  # 64-key tiles
    ("bf16", 1, 256, 6000, 8, 8, 128, "head", "lean"),
]


@pytest.mark.parametrize("dtype,B,Nq,Nk,Hq,Hkv,dqk,scales,pm", CASES)
def test_split_matches_oracle(require_gpu, dtype, B, Nq, Nk, Hq, Hkv, dqk, scales, pm):
    plan = _plan_checked(B, Hq, Hkv, Nq, Nk, dqk, dtype == "fp8", scales, pm)
    assert plan is not None, "the case is meant to split"
    dev, ref_in = _inputs(dtype, B, Nq, Nk, Hq, Hkv, dqk, seed=Nq + Nk, scales=scales)
    out, lse = miattn.attn_fwd_ws(*dev, scales=scales, p_mode=pm)
    torch.cuda.synchronize()
    ref, ref_lse = attn_chunk_ref_rows(*ref_in)
    err = rel_fro(out.cpu(), ref)
    print(f"split L={plan[0]} units={plan[1]}: rel_fro {err:.3e}")
    assert err <= TOL[dtype], err
    _check_lse(dtype, lse.cpu().numpy().astype(np.float64), ref_lse, ref_in)
    # every row and head is finite and close to the unsplit launch
    if dtype == "fp8":
        u, ul = miattn.attn_fwd_fp8(*dev, scales=scales, p_mode=pm)
    else:
        u, ul = miattn.attn_fwd_chunk(*dev)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    assert rel_fro(out.cpu(), u.cpu().double().numpy()) <= TOL[dtype]


def test_outlier_rows_split(require_gpu):
    """Peaked rows (outlier channels): ranges whose keys all sit far below the
    row max get weights near 0 in the merge."""
    dev, ref_in = _inputs("fp8", 1, 2000, 2000, 4, 4, 128, seed=9, outliers=4)
    assert _plan_checked(1, 4, 4, 2000, 2000, 128, True) is not None
    out, lse = miattn.attn_fwd_ws(*dev)
    torch.cuda.synchronize()
    ref, ref_lse = attn_chunk_ref_rows(*ref_in)
    assert rel_fro(out.cpu(), ref) <= TOL["fp8"]
    _check_lse("fp8", lse.cpu().numpy().astype(np.float64), ref_lse, ref_in)


def test_unsplit_shapes_run_the_plain_kernel(require_gpu):
    """Where the plan does not split (query tiles fill the CUs, too few key
    tiles to save, or partial rows that would cost what the split saves, as
    at 1K tokens with 32 heads or 4K with 8), attn_fwd_ws is attn_fwd_fp8 / attn_fwd_chunk
    bit for bit."""
    for (B, Nq, Nk, Hq, Hkv) in ((1, 2048, 2048, 32, 8), (1, 500, 500, 2, 2), (1, 1024, 1024, 32, 32),
                                 (1, 4096, 4096, 8, 8)):
        assert _plan_checked(B, Hq, Hkv, Nq, Nk, 128, True) is None
        dev, _ = _inputs("fp8", B, Nq, Nk, Hq, Hkv, 128, seed=3)
        a, la = miattn.attn_fwd_ws(*dev)
        b, lb = miattn.attn_fwd_fp8(*dev, p_mode=miattn.DEFAULT_P_MODE)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)) and torch.equal(la, lb)
    assert _plan_checked(1, 32, 32, 1024, 1024, 128, False) is None
    dev, _ = _inputs("bf16", 1, 1024, 1024, 32, 32, 128, seed=4)
    a, la = miattn.attn_fwd_ws(*dev)
    b, lb = miattn.attn_fwd_chunk(*dev)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)) and torch.equal(la, lb)


def _bitwise_100(fn, out):
    fn()
    torch.cuda.synchronize()
    first = out.view(torch.int16).clone()
    for i in range(100):
        out.view(torch.int16).fill_(0x7FC0)
        fn()
        assert torch.equal(out.view(torch.int16), first), f"launch {i + 1} differs from the first"


@pytest.mark.parametrize("dtype", ["fp8", "bf16"])
def test_split_bitwise_deterministic(require_gpu, dtype):
    """100 launches of a split 4K launch with 4 heads, LSE written."""
    w = WORKLOADS["fp8_mha_n4k"].with_(dtype=dtype, Hq=4, Hkv=4)
    assert _plan_checked(w.B, w.Hq, w.Hkv, w.N, w.N, w.d_qk, w.dtype == "fp8") is not None
    q, k, v = (t.to(torch.bfloat16).cuda() for t in make_inputs(w))
    out = torch.empty((w.B, w.N, w.Hq, w.d_v), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device="cuda")
    if w.dtype == "fp8":
        args = [t for pair in (miattn.attn_quantize_fp8(t) for t in (q, k, v)) for t in pair]
        args = [args[0], args[2], args[4], args[1], args[3], args[5]]
    else:
        args = [q, k, v]
    ws = torch.empty(miattn.attn_fwd_ws_size(w.B, w.Hq, w.Hkv, w.N, w.N, w.d_qk, w.d_v, w.dtype == "fp8"),
                     dtype=torch.uint8, device="cuda")
    fn = lambda: miattn.attn_fwd_ws(*args, out=out, lse=lse, workspace=ws)  # noqa: E731
    _bitwise_100(fn, out)
    lse0 = lse.clone()
    fn()
    torch.cuda.synchronize()
    assert torch.equal(lse.view(torch.int32), lse0.view(torch.int32))


def test_split_chunk_bitwise_deterministic(require_gpu):
    """A 512-query chunk against 32K keys (every query tile split many times)."""
    dev, _ = _inputs("fp8", 1, 512, 32768, 32, 32, 128, seed=21)
    plan = _plan_checked(1, 32, 32, 512, 32768, 128, True)
    assert plan is not None and plan[1] > 2
    out = torch.empty((1, 512, 32, 128), dtype=torch.bfloat16, device="cuda")
    _bitwise_100(lambda: miattn.attn_fwd_ws(*dev, out=out, with_lse=False), out)


def test_split_4k_whole_heads(require_gpu):
    """4K tokens, 4 heads (ranges of 8 FP8 / 14 BF16 key tiles), every head and row."""
    for dtype in ("fp8", "bf16"):
        w = WORKLOADS["fp8_mha_n4k"].with_(dtype=dtype, Hq=4, Hkv=4)
        assert _plan_checked(w.B, w.Hq, w.Hkv, w.N, w.N, w.d_qk, dtype == "fp8") is not None
        dev, ref_in = _inputs(w.dtype, w.B, w.N, w.N, w.Hq, w.Hkv, w.d_qk, seed=w.seed)
        out, lse = miattn.attn_fwd_ws(*dev)
        torch.cuda.synchronize()
        ref, ref_lse = attn_chunk_ref_rows(*ref_in)
        err = rel_fro(out.cpu(), ref)
        print(f"[{dtype} 4K x 4 heads] split whole heads rel_fro {err:.3e}")
        assert err <= TOL[w.dtype], err
        _check_lse(w.dtype, lse.cpu().numpy().astype(np.float64), ref_lse, ref_in)


def test_workspace_errors(require_gpu):
    """Too small, missing or misaligned workspace: an error, nothing enqueued."""
    dev, _ = _inputs("fp8", 1, 2000, 2000, 4, 2, 128, seed=2)
    need = miattn.attn_fwd_ws_size(1, 4, 2, 2000, 2000, 128, 128, True)
    assert need > 0
    out = torch.full((1, 2000, 4, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(need + 64, dtype=torch.uint8, device="cuda")
    lib = miattn.load_library()
    cq, ck, cv, sq, sk, sv = dev
    stream = torch.cuda.current_stream().cuda_stream

    def call(w, nbytes):
        return lib.attn_fwd_ws(cq.data_ptr(), ck.data_ptr(), cv.data_ptr(), out.data_ptr(), None, 1, 4, 2, 2000, 2000,
                               128, 128, 1, sq.data_ptr(), sk.data_ptr(), sv.data_ptr(), 0.0, 0, 4, w, nbytes, stream)

    assert call(ws.data_ptr(), need - 1) == -2
    assert call(None, need) == -1
    assert call(ws.data_ptr() + 4, need) == -6
    torch.cuda.synchronize()
    assert bool((out.float() == 7.0).all())  # nothing ran
    assert call(ws.data_ptr(), need) == 0
    torch.cuda.synchronize()
    assert not bool((out.float() == 7.0).all())
