"""attn_fwd_noalloc (through the C ABI) against attn_fwd_ws.

attn_fwd_noalloc runs attn_fwd_ws's kernels with the library's static scratch
in place of the caller's workspace, so its results must equal attn_fwd_ws's
bit for bit.  Two calls in a row on split launches, the second smaller (the
scratch keeps the first call's contents), then an unsplit launch; and every
plan of the shapes the library is specified on fits the scratch.
"""

import ctypes
import re
import os

import numpy as np
import pytest
import torch

import bf16_causal_prefill_flashattention_amd as miattn
from bf16_causal_prefill_flashattention_amd.inputs import Workload, make_qkv
from oracle import quantize_ref

pytestmark = pytest.mark.gpu
HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "miattn.h")


def scratch_bytes():
    return int(re.search(r"#define\s+MIATTN_NOALLOC_SCRATCH_BYTES\s+(\d+)", open(HEADER).read()).group(1))


def _fp8_inputs(B, Nq, Nk, H, seed):
    w = Workload("noalloc", "fp8", B, H, H, Nk, 128, 128, seed=seed)
    q, k, v = make_qkv(w)
    q = q[:, Nk - Nq:].contiguous()
    (cq, sq), (ck, sk), (cv, sv) = quantize_ref(q), quantize_ref(k), quantize_ref(v)
    return [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in (cq, ck, cv, sq, sk, sv)]


def _noalloc(dev, B, Nq, Nk, H):
    cq, ck, cv, sq, sk, sv = dev
    out = torch.full((B, Nq, H, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, H, Nq), float("nan"), dtype=torch.float32, device="cuda")
    st = miattn.load_library().attn_fwd_noalloc(
        cq.data_ptr(), ck.data_ptr(), cv.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, H, Nq, Nk, 128, 128,
        miattn.DTYPE_FP8_E4M3, sq.data_ptr(), sk.data_ptr(), sv.data_ptr(), 0.0, 0, 4,
        torch.cuda.current_stream().cuda_stream)
    assert st == 0, miattn.attn_status_string(st)
    return out, lse


# (B, Nq, Nk, H): a 512-query chunk against 32K keys, then a smaller split
# launch, then one that does not split
SHAPES = [(1, 512, 32768, 32, True), (1, 2000, 2000, 2, True), (1, 4096, 4096, 32, False)]


def test_noalloc_matches_attn_fwd_ws(require_gpu):
    for i, (B, Nq, Nk, H, splits) in enumerate(SHAPES):
        need = miattn.attn_fwd_ws_size(B, H, H, Nq, Nk, 128, 128, True)
        assert (need > 0) == splits and need <= scratch_bytes()
        dev = _fp8_inputs(B, Nq, Nk, H, seed=11 + i)
        got, got_lse = _noalloc(dev, B, Nq, Nk, H)
        ref, ref_lse = miattn.attn_fwd_ws(*dev)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), (B, Nq, Nk, H)
        assert torch.equal(got_lse.view(torch.int32), ref_lse.view(torch.int32)), (B, Nq, Nk, H)


def test_every_plan_fits_the_scratch(require_gpu):
    """The largest plans: one range per compute unit, at both tile sizes."""
    cap = scratch_bytes()
    for fp8 in (True, False):
        for (B, H, Nq, Nk) in ((1, 1, 256, 1 << 20), (1, 2, 512, 1 << 18), (4, 8, 256, 65536), (1, 1, 1, 4096)):
            assert miattn.attn_fwd_ws_size(B, H, H, Nq, Nk, 128, 128, fp8) <= cap
