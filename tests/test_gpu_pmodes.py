"""FP8 probability modes (``attn_fwd_fp8`` through the C ABI) against the fp64
oracle.

The modes differ only in how the softmax probabilities are rounded to e4m3 for
the P.V product ([P3] "ZYFA 如何工作？": lean P, a code written straight from
the score, against exp plus conversion; per-block power-of-two scaling of P
undone by the scaled MFMA): lean or exact, with no shift, a shift per 64-key
step, or a shift per 128-key tile.  Every mode must meet the FP8 gate
(relative Frobenius error <= 6e-2 on the dequantized inputs) and the LSE bound
derived in test_gpu_chunk.py (the lean-P log error bounds the exact
conversion's too, and a shift only removes lost mass).  The inputs are
quantized by the oracle's quantizer on the CPU and the same codes uploaded.

The far-key-block case: K and V rows in blocks of 64 positions scaled by 2^r,
r uniform in {-1, 0, 1}, 65536 keys.  Many keys of the low blocks score about
13 octaves below the row max, where lean P rounded against the running max
loses them (MI355X: 6.6% error with per-head scales); the shifted modes round
each step or tile against its own max and must meet the gate on it, and so
must the default FP8 path of attn_fwd.
"""

import os
import re

import numpy as np
import pytest
import torch

import bf16_causal_prefill_flashattention_amd as miattn
from bf16_causal_prefill_flashattention_amd.inputs import Workload, make_qkv
from oracle import (attn_chunk_ref_rows, dequantize_block64_ref, dequantize_ref, quantize_block64_ref,
                    quantize_ref)
from parity_util import TOL, rel_fro
from test_gpu_chunk import _check_lse

pytestmark = pytest.mark.gpu
MODES = sorted(miattn.P_MODES)
SHIFTED = [m for m in MODES if m.endswith("_block") or m.endswith("_tile")]
HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "miattn.h")


def default_mode() -> str:
    """The probability mode attn_fwd and attn_fwd_chunk use (MIATTN_P_DEFAULT)."""
    src = open(HEADER).read()
    name = re.search(r"#define\s+MIATTN_P_DEFAULT\s+MIATTN_P_(\w+)", src).group(1).lower()
    assert name in miattn.P_MODES
    return name


def _quantized(q, k, v, scales, hadamard=False):
    quant = quantize_block64_ref if scales == "block64" else quantize_ref
    deq = dequantize_block64_ref if scales == "block64" else dequantize_ref
    (cq, sq), (ck, sk), (cv, sv) = quant(q, hadamard), quant(k, hadamard), quant(v, False)
    dev = [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in (cq, ck, cv, sq, sk, sv)]
    return dev, (deq(cq, sq), deq(ck, sk), deq(cv, sv))


CASES = [
    # (B, Nq, Nk, Hq, Hkv, d_qk, outliers)
    (1, 700, 700, 4, 2, 128, 4),
    (2, 300, 1000, 4, 4, 128, 0),
    (1, 333, 333, 2, 2, 192, 0),
    (1, 129, 600, 4, 2, 192, 4),
    (1, 300, 5000, 4, 2, 128, 4),  # beyond 4096 keys: 192-key tiles where the mode has no 64-key shift
]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("scales", ["head", "block64"])
@pytest.mark.parametrize("B,Nq,Nk,Hq,Hkv,dqk,outl", CASES)
def test_mode_against_oracle(require_gpu, mode, scales, B, Nq, Nk, Hq, Hkv, dqk, outl):
    w = Workload("t", "fp8", B, Hq, Hkv, Nk, dqk, 128, outliers=outl, seed=Nq + Nk + Hq)
    q, k, v = make_qkv(w)
    q = q[:, Nk - Nq:].contiguous()
    dev, ref_in = _quantized(q, k, v, scales)
    out, lse = miattn.attn_fwd_fp8(*dev, scales=scales, p_mode=mode)
    torch.cuda.synchronize()
    ref, ref_lse = attn_chunk_ref_rows(*ref_in)
    err = rel_fro(out.cpu(), ref)
    assert err <= TOL["fp8"], (mode, err)
    _check_lse("fp8", lse.cpu().numpy().astype(np.float64), ref_lse, ref_in)


def test_default_mode_is_what_attn_fwd_runs(require_gpu):
    """attn_fwd_fp8 with MIATTN_SCALES_HEAD and the default mode reproduces
    attn_fwd_chunk bit for bit, and with block64 scales and the lean /
    lean-block modes, attn_fwd_block64 with p_block_scale 0 / 1."""
    w = Workload("t", "fp8", 1, 4, 2, 1500, 128, 128, outliers=4, seed=31)
    q, k, v = make_qkv(w)
    dev, _ = _quantized(q, k, v, "head")
    a, la = miattn.attn_fwd_chunk(*dev)
    b, lb = miattn.attn_fwd_fp8(*dev, scales="head", p_mode=default_mode())
    c = miattn.attn_fwd(*dev)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)) and torch.equal(la, lb)
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))
    dev, _ = _quantized(q, k, v, "block64")
    for pbs, mode in ((False, "lean"), (True, "lean_block")):
        a, la = miattn.attn_fwd_block64(*dev, p_block_scale=pbs)
        b, lb = miattn.attn_fwd_fp8(*dev, scales="block64", p_mode=mode)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)) and torch.equal(la, lb)


def _far_blocks(Nq=256, Nk=65536, Hq=2, seed=5):
    """Q N(0, 1); K, V N(0, 1) with every block of 64 positions scaled by 2^r,
    r uniform in {-1, 0, 1} (independently for K and V); fp32."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, Nq, Hq, 128)).astype(np.float32)

    def kv():
        r = np.repeat(rng.integers(-1, 2, size=Nk // 64), 64)
        return (rng.standard_normal((1, Nk, 1, 128)) * 2.0 ** r[None, :, None, None]).astype(np.float32)

    return q, kv(), kv()


@pytest.mark.parametrize("scales", ["head", "block64"])
def test_shifted_modes_keep_far_key_blocks(require_gpu, scales):
    q, k, v = _far_blocks()
    dev, ref_in = _quantized(q, k, v, scales)
    ref, ref_lse = attn_chunk_ref_rows(*ref_in)
    errs = {}
    for mode in MODES:
        out, lse = miattn.attn_fwd_fp8(*dev, scales=scales, p_mode=mode)
        torch.cuda.synchronize()
        errs[mode] = rel_fro(out.cpu(), ref)
        if mode in SHIFTED:
            _check_lse("fp8", lse.cpu().numpy().astype(np.float64), ref_lse, ref_in)
    print(f"far key blocks ({scales} scales): " + ", ".join(f"{m} {e:.4f}" for m, e in errs.items()))
    for mode in SHIFTED:
        assert errs[mode] <= TOL["fp8"], errs
    # the input reaches lean P's floor (its linear code map loses a probability
    # about 13 octaves below the running max; the exact conversion's subnormals
    # reach about 2.5 octaves further): without a shift lean P loses mass here
    assert errs["lean"] > 1.5 * max(errs["lean_block"], errs["lean_tile"]), errs


def test_default_fp8_path_keeps_far_key_blocks(require_gpu):
    """The default FP8 path -- the library's per-head quantizer and attn_fwd_chunk
    (attn_fwd's kernel) -- meets the gate on the far-key-block input, asserted
    absolutely."""
    q, k, v = _far_blocks()
    cq, sq = miattn.attn_quantize_fp8(torch.from_numpy(q).cuda())
    ck, sk = miattn.attn_quantize_fp8(torch.from_numpy(k).cuda())
    cv, sv = miattn.attn_quantize_fp8(torch.from_numpy(v).cuda())
    out, lse = miattn.attn_fwd_chunk(cq, ck, cv, sq, sk, sv)
    torch.cuda.synchronize()
    (rq, rsq), (rk, rsk), (rv, rsv) = quantize_ref(q), quantize_ref(k), quantize_ref(v)
    assert np.array_equal(ck.cpu().numpy(), rk) and np.array_equal(cv.cpu().numpy(), rv)
    ref_in = (dequantize_ref(rq, rsq), dequantize_ref(rk, rsk), dequantize_ref(rv, rsv))
    ref, ref_lse = attn_chunk_ref_rows(*ref_in)
    err = rel_fro(out.cpu(), ref)
    assert err <= TOL["fp8"], err
    _check_lse("fp8", lse.cpu().numpy().astype(np.float64), ref_lse, ref_in)


@pytest.mark.parametrize("N", [1700, 1280])
@pytest.mark.parametrize("mode", ["lean_tile", "exact", "exact_tile"])
def test_modes_bitwise_deterministic_in_paired_mode(require_gpu, mode, N):
    """100 launches of persistent-mode shapes (more 256-query tiles than CUs):
    at 1700 tokens 64 heads make 256 heavy/light pairs, at 1280 tokens 192,
    which a 256-CU device deals as single tiles in snake order instead."""
    w = Workload("t", "fp8", 1, 64, 8, N, 128, 128, outliers=4, seed=41)
    q, k, v = make_qkv(w)
    dev, _ = _quantized(q, k, v, "head")
    out = torch.empty((1, N, 64, 128), dtype=torch.bfloat16, device="cuda")
    miattn.attn_fwd_fp8(*dev, out=out, with_lse=False, p_mode=mode)
    torch.cuda.synchronize()
    first = out.view(torch.int16).clone()
    for i in range(100):
        out.view(torch.int16).fill_(0x7FC0)
        miattn.attn_fwd_fp8(*dev, out=out, with_lse=False, p_mode=mode)
        assert torch.equal(out.view(torch.int16), first), i


@pytest.mark.parametrize("scales,Nk", [("block64", 1 << 20), ("head", 1 << 18)])
def test_uniform_e4m3_bytes_at_the_key_limit(require_gpu, scales, Nk):
    """K and V: uniform random finite e4m3 bytes (every exponent equally
    likely), with random power-of-two scales per 64 positions in [2^-12, 2^-5]
    (block64, at the block-scaled key limit of 2^20) or one scale of 2^-6 per
    head; Q: Gaussian, quantized by the oracle; a ragged chunk of 100 queries
    at the end.  Rows are peaked and key blocks differ in magnitude by up to
    2^7.  Every shifted mode -- the FP8 default among them -- meets the 6e-2
    gate and the LSE bound, asserted absolutely.  Lean P without a shift loses
    the low blocks' mass below its floor here (MI355X: 7.3% with block scales),
    the limit include/miattn.h states for that mode."""
    B, Nq, Hq, Hkv, d = 1, 100, 2, 1, 128
    rng = np.random.default_rng(77)
    quant = quantize_block64_ref if scales == "block64" else quantize_ref
    deq = dequantize_block64_ref if scales == "block64" else dequantize_ref
    cq, sq = quant(rng.standard_normal((B, Nq, Hq, d)).astype(np.float32))

    def codes_and_scales():
        c = rng.integers(0, 256, size=(B, Nk, Hkv, d), dtype=np.uint8)
        c[(c & 0x7F) == 0x7F] = 0x7E  # no NaN codes
        if scales == "block64":
            s = (np.float32(2.0) ** rng.integers(-12, -4, size=(B, Hkv, Nk // 64))).astype(np.float32)
        else:
            s = np.full((B, Hkv), 2.0 ** -6, dtype=np.float32)
        return c, s

    (ck, sk), (cv, sv) = codes_and_scales(), codes_and_scales()
    dev = [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in (cq, ck, cv, sq, sk, sv)]
    ref_in = (deq(cq, sq), deq(ck, sk), deq(cv, sv))
    ref, ref_lse = attn_chunk_ref_rows(*ref_in)
    errs = {}
    for mode in MODES:
        out, lse = miattn.attn_fwd_fp8(*dev, scales=scales, p_mode=mode)
        torch.cuda.synchronize()
        errs[mode] = rel_fro(out.cpu(), ref)
        if mode in SHIFTED:
            _check_lse("fp8", lse.cpu().numpy().astype(np.float64), ref_lse, ref_in)
    print(f"uniform e4m3 bytes ({scales} scales, {Nk} keys): " + ", ".join(f"{m} {e:.4f}" for m, e in errs.items()))
    for mode in SHIFTED:
        assert errs[mode] <= TOL["fp8"], errs
    assert errs[default_mode()] <= TOL["fp8"], errs
