"""GPU attention (through the C ABI) against the fp64 oracle.

Small cases compare every output element; the full-size workloads run in the
same launch configuration the benchmark times and compare sampled rows of
sampled heads, which the oracle computes one by one.  BF16: relative Frobenius
error <= 1e-2 against the oracle on the BF16 inputs.  FP8: the GPU quantizer's
codes and scales must equal the oracle quantizer's bit for bit, and the
attention output must be within 6e-2 of the oracle on the dequantized inputs.
"""

import numpy as np
import pytest
import torch

import bf16_causal_prefill_flashattention_amd as miattn
from bf16_causal_prefill_flashattention_amd.inputs import Workload, make_inputs, make_qkv
from oracle import attn_ref, dequantize_ref, quantize_ref
from parity_util import TOL, per_head_rel_fro, rel_fro

pytestmark = pytest.mark.gpu


def _bf16_case(w: Workload):
    q, k, v = make_inputs(w)
    out = miattn.attn_fwd(q.cuda(), k.cuda(), v.cuda())
    torch.cuda.synchronize()
    return out.cpu(), (q, k, v)


def _fp8_gpu(q, k, v, hadamard):
    cq, sq = miattn.attn_quantize_fp8(q.cuda(), hadamard=hadamard)
    ck, sk = miattn.attn_quantize_fp8(k.cuda(), hadamard=hadamard)
    cv, sv = miattn.attn_quantize_fp8(v.cuda(), hadamard=False)
    out = miattn.attn_fwd(cq, ck, cv, sq, sk, sv)
    torch.cuda.synchronize()
    return out.cpu(), (cq.cpu().numpy(), sq.cpu().numpy(), ck.cpu().numpy(), sk.cpu().numpy(),
                       cv.cpu().numpy(), sv.cpu().numpy())


def _fp8_oracle_inputs(q, k, v, hadamard):
    cq, sq = quantize_ref(q, hadamard)
    ck, sk = quantize_ref(k, hadamard)
    cv, sv = quantize_ref(v, False)
    return (cq, sq, ck, sk, cv, sv)


def _assert_same_codes(gpu, ref):
    names = ["q codes", "q scale", "k codes", "k scale", "v codes", "v scale"]
    for name, a, b in zip(names, gpu, ref):
        if a.dtype == np.float32:
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), name
        else:
            assert np.array_equal(a, b), f"{name}: {np.count_nonzero(a != b)} differ"


SMALL = [
    # (B, N, Hq, Hkv, d_qk, outliers)
    (1, 512, 2, 2, 128, 0),  # the small exact-check workload
    (2, 1, 2, 1, 128, 0),
    (1, 17, 4, 2, 128, 0),
    (1, 127, 2, 2, 128, 0),
    (1, 129, 2, 2, 128, 0),
    (1, 300, 8, 2, 128, 0),
    (2, 700, 4, 4, 128, 0),
    (1, 1024, 8, 2, 128, 4),  # GQA with activation-like outlier channels
    (1, 333, 2, 2, 192, 0),  # MLA shape, ragged
    (1, 1000, 4, 4, 192, 0),
]


@pytest.mark.parametrize("B,N,Hq,Hkv,dqk,outl", SMALL)
def test_bf16_small_full_compare(require_gpu, B, N, Hq, Hkv, dqk, outl):
    w = Workload("t", "bf16", B, Hq, Hkv, N, dqk, 128, outliers=outl, seed=N + Hq)
    out, (q, k, v) = _bf16_case(w)
    ref = attn_ref(q, k, v)
    err = rel_fro(out, ref)
    assert err <= TOL["bf16"], (err, per_head_rel_fro(out, ref))
    assert torch.isfinite(out.float()).all()


@pytest.mark.parametrize("B,N,Hq,Hkv,dqk,outl", SMALL)
@pytest.mark.parametrize("hadamard", [False, True])
def test_fp8_small_full_compare(require_gpu, B, N, Hq, Hkv, dqk, outl, hadamard):
    w = Workload("t", "fp8", B, Hq, Hkv, N, dqk, 128, outliers=outl, seed=N + Hq + 1)
    q, k, v = make_qkv(w)
    out, gpu_codes = _fp8_gpu(q, k, v, hadamard)
    ref_codes = _fp8_oracle_inputs(q, k, v, hadamard)
    _assert_same_codes(gpu_codes, ref_codes)
    cq, sq, ck, sk, cv, sv = ref_codes
    ref = attn_ref(dequantize_ref(cq, sq), dequantize_ref(ck, sk), dequantize_ref(cv, sv))
    err = rel_fro(out, ref)
    assert err <= TOL["fp8"], (err, per_head_rel_fro(out, ref))


PAIRED = [
    # (dtype, B, N, Hkv, d_qk): more 256-query tiles than CUs, in pairs that
    # split evenly over the CUs (the heads are chosen for that), so every
    # persistent workgroup runs heavy/light pairs of tiles, the lighter tile of
    # a pair with its keys walked downward; an odd tile count leaves a middle
    # tile unpaired
    ("bf16", 1, 1700, 8, 128),
    ("fp8", 1, 1700, 8, 128),
    ("fp8", 1, 1800, 16, 192),
    ("bf16", 2, 1800, 32, 192),
]


@pytest.mark.parametrize("dtype,B,N,Hkv,dqk", PAIRED)
def test_paired_persistent_full_compare(require_gpu, dtype, B, N, Hkv, dqk):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    nqt = (N + 255) // 256
    pairs = (nqt + 1) // 2
    if cus % (B * pairs) or (cus // (B * pairs)) % Hkv:
        pytest.skip("no head count splits these pairs evenly over this device's CUs")
    Hq = cus // (B * pairs)
    assert B * Hq * nqt > cus and (B * Hq * pairs) % cus == 0, "the case must launch in paired mode"
    w = Workload("t", dtype, B, Hq, Hkv, N, dqk, 128, outliers=4, seed=N + Hq + B)
    if dtype == "bf16":
        out, (q, k, v) = _bf16_case(w)
        ref = attn_ref(q, k, v)
    else:
        q, k, v = make_qkv(w)
        out, gpu_codes = _fp8_gpu(q, k, v, False)
        ref_codes = _fp8_oracle_inputs(q, k, v, False)
        _assert_same_codes(gpu_codes, ref_codes)
        cq, sq, ck, sk, cv, sv = ref_codes
        ref = attn_ref(dequantize_ref(cq, sq), dequantize_ref(ck, sk), dequantize_ref(cv, sv))
    err = per_head_rel_fro(out, ref)
    assert rel_fro(out, ref) <= TOL[dtype] and err.max() <= TOL[dtype], err


def _snake_heads(cus, N, G):
    """The fewest heads (a multiple of G) whose heavy/light pairs of 256-query
    tiles outnumber the CUs without splitting evenly over them, the launches
    dealt in snake order of cost."""
    pairs = ((N + 255) // 256 + 1) // 2
    H = G
    while not (H * pairs > cus and (H * pairs) % cus != 0):
        H += G
    return H


SNAKE = [
    # (dtype, N, Hkv, d_qk)
    ("bf16", 1280, 8, 128),
    ("fp8", 1280, 8, 128),
    ("fp8", 1100, 8, 192),
    ("bf16", 1100, 8, 192),
]


@pytest.mark.parametrize("dtype,N,Hkv,dqk", SNAKE)
def test_snake_order_full_compare(require_gpu, dtype, N, Hkv, dqk):
    """Launches whose tile pairs do not split evenly over the CUs deal single
    tiles in snake order of cost (every odd round walking its keys downward):
    the whole output against the oracle, and repeated launches bit for bit."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    Hq = _snake_heads(cus, N, Hkv)
    w = Workload("t", dtype, 1, Hq, Hkv, N, dqk, 128, outliers=4, seed=N + Hq)
    if dtype == "bf16":
        q, k, v = make_inputs(w)
        dev = [t.cuda() for t in (q, k, v)]
        ref = attn_ref(q, k, v)
    else:
        q, k, v = make_qkv(w)
        cq, sq, ck, sk, cv, sv = _fp8_oracle_inputs(q, k, v, False)
        dev = [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in (cq, ck, cv, sq, sk, sv)]
        ref = attn_ref(dequantize_ref(cq, sq), dequantize_ref(ck, sk), dequantize_ref(cv, sv))
    out = miattn.attn_fwd(*dev)
    torch.cuda.synchronize()
    first = out.view(torch.int16).clone()
    err = per_head_rel_fro(out.cpu(), ref)
    assert rel_fro(out.cpu(), ref) <= TOL[dtype] and err.max() <= TOL[dtype], err
    for _ in range(10):
        miattn.attn_fwd(*dev, out=out)
        assert torch.equal(out.view(torch.int16), first)


# ---------------------------------------------------------------- special cases


def test_bf16_row_zero_is_v0_exactly(require_gpu):
    w = Workload("t", "bf16", 2, 4, 2, 200, 128, 128, seed=3)
    out, (q, k, v) = _bf16_case(w)
    for h in range(4):
        assert torch.equal(out[:, 0, h], v[:, 0, h // 2])


def test_fp8_row_zero_is_dequantized_v0(require_gpu):
    w = Workload("t", "fp8", 1, 4, 2, 300, 128, 128, seed=4)
    q, k, v = make_qkv(w)
    out, codes = _fp8_gpu(q, k, v, False)
    cv, sv = codes[4], codes[5]
    expect = torch.from_numpy(dequantize_ref(cv, sv)[:, 0]).to(torch.bfloat16)
    for h in range(4):
        a = out[:, 0, h].float()
        b = expect[:, h // 2].float()
        assert torch.all((a - b).abs() <= b.abs() * 2.0 ** -7 + 1e-30)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_zero_queries_give_prefix_mean(require_gpu, dtype):
    N = 600
    w = Workload("t", dtype, 1, 2, 1, N, 128, 128, seed=5)
    q, k, v = make_qkv(w)
    q.zero_()
    if dtype == "bf16":
        out = miattn.attn_fwd(q.bfloat16().cuda(), k.bfloat16().cuda(), v.bfloat16().cuda()).cpu()
        vv = v.bfloat16().double().numpy()
    else:
        out, codes = _fp8_gpu(q, k, v, False)
        vv = dequantize_ref(codes[4], codes[5])
    prefix = np.cumsum(vv[0, :, 0], axis=0) / np.arange(1, N + 1)[:, None]
    for h in range(2):
        err = rel_fro(out[0, :, h], prefix)
        assert err <= 4e-3, err  # equal scores: every weight is exact, only the output rounding remains


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_key_permutation_inside_window(require_gpu, dtype):
    N, kk = 400, 150
    w = Workload("t", dtype, 1, 2, 2, N, 128, 128, seed=6)
    q, k, v = make_qkv(w)
    perm = torch.from_numpy(np.random.default_rng(7).permutation(kk + 1))
    k2, v2 = k.clone(), v.clone()
    k2[:, : kk + 1] = k[:, perm]
    v2[:, : kk + 1] = v[:, perm]
    if dtype == "bf16":
        a = miattn.attn_fwd(q.bfloat16().cuda(), k.bfloat16().cuda(), v.bfloat16().cuda()).cpu()
        b = miattn.attn_fwd(q.bfloat16().cuda(), k2.bfloat16().cuda(), v2.bfloat16().cuda()).cpu()
        tol = 2 * TOL["bf16"]
    else:
        a, _ = _fp8_gpu(q, k, v, False)
        b, _ = _fp8_gpu(q, k2, v2, False)  # permuting rows leaves the per-head amax unchanged
        tol = 2 * TOL["fp8"]
    assert rel_fro(b[:, kk:], a[:, kk:].double().numpy()) <= tol


@pytest.mark.parametrize("dtype,dqk", [("bf16", 128), ("fp8", 128), ("fp8", 192)])
def test_bitwise_deterministic_100_launches(require_gpu, dtype, dqk):
    w = Workload("t", dtype, 1, 8, 2, 2048, dqk, 128, outliers=0, seed=8)
    q, k, v = make_inputs(w)
    if dtype == "bf16":
        args = (q.cuda(), k.cuda(), v.cuda())
    else:
        cq, sq = miattn.attn_quantize_fp8(q.cuda())
        ck, sk = miattn.attn_quantize_fp8(k.cuda())
        cv, sv = miattn.attn_quantize_fp8(v.cuda())
        args = (cq, ck, cv, sq, sk, sv)
    first = miattn.attn_fwd(*args).view(torch.int16).clone()
    out = torch.empty_like(first).view(torch.bfloat16)
    for _ in range(100):
        miattn.attn_fwd(*args, out=out)
        assert torch.equal(out.view(torch.int16), first)


def test_output_written_only_inside_bounds(require_gpu):
    w = Workload("t", "bf16", 1, 2, 2, 77, 128, 128, seed=9)
    q, k, v = make_inputs(w)
    n = 77 * 2 * 128
    buf = torch.full((n + 4096,), 7.0, dtype=torch.bfloat16, device="cuda")
    out = buf[2048: 2048 + n].view(1, 77, 2, 128)
    miattn.attn_fwd(q.cuda(), k.cuda(), v.cuda(), out=out)
    torch.cuda.synchronize()
    assert torch.all(buf[:2048] == 7.0) and torch.all(buf[2048 + n:] == 7.0)


def test_empty_sequence_is_a_no_op(require_gpu):
    q = torch.empty(1, 0, 2, 128, dtype=torch.bfloat16, device="cuda")
    out = miattn.attn_fwd(q, q, q)
    assert out.shape == (1, 0, 2, 128)


def test_misaligned_pointer_is_rejected(require_gpu):
    base = torch.zeros(1 * 16 * 2 * 128 + 1, dtype=torch.bfloat16, device="cuda")
    q = base[1:].view(1, 16, 2, 128)
    with pytest.raises(miattn.MiattnError) as ei:
        miattn.attn_fwd(q, q, q)
    assert ei.value.status == -6
