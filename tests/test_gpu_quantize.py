"""GPU FP8 front end against the oracle quantizer: codes and scales must be
bit-identical (the decision is taken in fp32 with the same steps on both
sides), for fp32 and bf16 sources, with and without the Hadamard rotation,
on ragged sizes and edge cases."""

import numpy as np
import pytest
import torch

import bf16_causal_prefill_flashattention_amd as miattn
from bf16_causal_prefill_flashattention_amd.inputs import WORKLOADS, make_qkv
from oracle import quantize_ref

pytestmark = pytest.mark.gpu


def _x(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(*shape, generator=g) * scale


def _check(x_cpu, hadamard):
    codes, scales = miattn.attn_quantize_fp8(x_cpu.cuda(), hadamard=hadamard)
    torch.cuda.synchronize()
    rc, rs = quantize_ref(x_cpu, hadamard)
    gc = codes.cpu().numpy()
    gs = scales.cpu().numpy()
    assert np.array_equal(gs.view(np.uint32), rs.view(np.uint32)), (gs, rs)
    mism = np.count_nonzero(gc != rc)
    assert mism == 0, f"{mism} codes differ of {gc.size}"


@pytest.mark.parametrize("hadamard", [False, True])
@pytest.mark.parametrize("src", ["fp32", "bf16"])
@pytest.mark.parametrize("N", [1, 17, 255, 256, 257, 1000])
def test_quantize_bit_exact_d128(require_gpu, hadamard, src, N):
    x = _x((2, N, 3, 128), N * 7 + hadamard, 3.0)
    if src == "bf16":
        x = x.to(torch.bfloat16)
    _check(x, hadamard)


@pytest.mark.parametrize("src", ["fp32", "bf16"])
def test_quantize_bit_exact_d192(require_gpu, src):
    x = _x((1, 333, 4, 192), 5, 0.01)
    if src == "bf16":
        x = x.to(torch.bfloat16)
    _check(x, False)


def test_quantize_outlier_workload(require_gpu):
    w = WORKLOADS["fp8_gqa_n16k"].with_(N=2048)
    q, k, v = make_qkv(w)
    for t in (q, k):
        _check(t, False)
        _check(t, True)
    _check(v, False)


def test_quantize_zero_head_and_wide_range(require_gpu):
    x = _x((1, 300, 3, 128), 9)
    x[:, :, 1] = 0
    x[:, :, 2] *= 1e-6
    x[0, 5, 2, 7] = 3e4  # one huge value: most codes land in the subnormal range
    _check(x, False)
    _check(x, True)


def test_quantize_empty_sequence_writes_unit_scales(require_gpu):
    x = torch.empty(2, 0, 3, 128, device="cuda")
    codes, scales = miattn.attn_quantize_fp8(x)
    codes_h, scales_h = miattn.attn_quantize_fp8(x, hadamard=True)
    torch.cuda.synchronize()
    assert codes.numel() == 0
    assert torch.all(scales.cpu() == 1.0)
    assert torch.all(scales_h.cpu() == torch.tensor(np.float32(2 ** -3.5)))
