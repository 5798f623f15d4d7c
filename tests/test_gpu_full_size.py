"""Full-size workloads on the GPU against the fp64 oracle, whole heads, every row.

Each configured workload runs in the launch configuration the benchmark times
(the persistent, paired work decomposition at 16K and 32K).  The oracle
computes whole heads, every query row, in a pool of worker processes, and the
gate is the relative Frobenius error over everything compared: <= 1e-2 for
BF16, <= 6e-2 for FP8 on the dequantized inputs.  Every head is compared when
the pool finishes them in one or two waves; at 32K tokens as many heads as the
pool has workers (all 32 on a host with 32 cores or more).  For FP8 the GPU
quantizer's codes and scales of every compared head must equal the oracle
quantizer's bit for bit.

Bitwise determinism is checked where the workloads run: 100 launches of each
32K workload (paired persistent mode, the lighter tile of each pair walking its
keys downward) must give the same bits.
"""

import numpy as np
import pytest
import torch

import bf16_causal_prefill_flashattention_amd as miattn
from bf16_causal_prefill_flashattention_amd.inputs import WORKLOADS, make_inputs
from oracle.pool import HeadPool, summarize
from parity_util import TOL

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pool():
    p = HeadPool()
    yield p
    p.close()


def _heads(w, workers):
    """Heads to compare: all of them when the pool covers them in two waves at
    N <= 16K (or one wave at 32K), else an evenly spread selection that always
    includes the first and last head and the first head of the second KV group."""
    limit = 2 * workers if w.N <= 16384 else workers
    if w.Hq <= limit:
        return list(range(w.Hq))
    grp = w.Hq // w.Hkv
    hs = {0, w.Hq - 1, min(grp, w.Hq - 1)}
    for h in np.linspace(0, w.Hq - 1, limit).round().astype(int):
        if len(hs) >= limit:
            break
        hs.add(int(h))
    return sorted(hs)[:limit]


def _tasks(w, q, k, v, out, heads, codes=None):
    grp = w.Hq // w.Hkv
    f32 = lambda t: np.ascontiguousarray(t.float().numpy())  # noqa: E731
    tasks = []
    for h in heads:
        g = h // grp
        t = {"key": h, "q": f32(q[0, :, h]), "k": f32(k[0, :, g]), "v": f32(v[0, :, g]),
             "out": f32(out[0, :, h]), "fp8": None if w.dtype == "bf16" else {"hadamard": w.hadamard}}
        if codes is not None:
            cq, ck, cv, sq, sk, sv = codes
            t["codes"] = (cq[0, :, h].numpy(), ck[0, :, g].numpy(), cv[0, :, g].numpy(),
                          float(sq[0, h]), float(sk[0, g]), float(sv[0, g]))
        tasks.append(t)
    return tasks


def _run(w, src="fp32"):
    """GPU output of workload w (B = 1) and the inputs the oracle reads.
    src: element type of the activations the FP8 front end reads (the
    benchmark's resident FP8 inputs come from BF16 activations)."""
    assert w.B == 1
    q, k, v = make_inputs(w)
    if w.dtype == "fp8" and src == "bf16":
        q, k, v = (t.to(torch.bfloat16) for t in (q, k, v))
    if w.dtype == "bf16":
        out = miattn.attn_fwd(q.cuda(), k.cuda(), v.cuda())
        torch.cuda.synchronize()
        return out.cpu(), (q, k, v), None
    (cq, sq), (ck, sk) = (miattn.attn_quantize_fp8(t.cuda(), hadamard=w.hadamard) for t in (q, k))
    cv, sv = miattn.attn_quantize_fp8(v.cuda())
    out = miattn.attn_fwd(cq, ck, cv, sq, sk, sv)
    torch.cuda.synchronize()
    codes = tuple(t.cpu() for t in (cq, ck, cv, sq, sk, sv))
    return out.cpu(), (q, k, v), codes


FULL = [
    ("bf16_gqa_n16k", "fp32"),  # C2
    ("fp8_mha_n1k", "fp32"),  # C3
    ("fp8_mha_n4k", "fp32"),
    ("fp8_mha_n16k", "fp32"),
    ("fp8_mha_n32k", "bf16"),  # C3 at 32K from the benchmark's BF16 activations
    ("bf16_mha_n32k", "fp32"),  # C3b
    ("fp8_gqa_n16k", "fp32"),  # C4 without and with the rotation
    ("fp8_gqa_n16k_had", "fp32"),
    ("fp8_mla_n32k", "fp32"),  # C5
]


@pytest.mark.parametrize("name,src", FULL)
def test_full_size_whole_heads(require_gpu, pool, name, src):
    w = WORKLOADS[name]
    out, (q, k, v), codes = _run(w, src)
    assert torch.isfinite(out.float()).all()
    heads = _heads(w, pool.workers)
    res = pool.run(_tasks(w, q, k, v, out, heads, codes))
    s = summarize(res)
    print(f"[{name}] heads {heads} rel_fro {s['rel_fro']:.3e} per-head max {s['per_head_max']:.3e}")
    if codes is not None:
        assert s["codes_equal"], "GPU FP8 codes or scales differ from the oracle quantizer"
    assert all(r["rows"] == w.N for r in res)
    assert s["rel_fro"] <= TOL[w.dtype], s
    assert s["per_head_max"] <= TOL[w.dtype], s


def _bitwise_100(fn, out):
    """100 launches of fn (which writes `out`), each into a buffer first filled
    with a NaN pattern, must all give the first launch's bits."""
    fn()
    torch.cuda.synchronize()
    first = out.view(torch.int16).clone()
    for i in range(100):
        out.view(torch.int16).fill_(0x7FC0)
        fn()
        assert torch.equal(out.view(torch.int16), first), f"launch {i + 1} differs from the first"


DETERMINISM = ["fp8_mha_n32k", "bf16_mha_n32k", "fp8_mla_n32k", "bf16_gqa_n16k", "fp8_gqa_n16k_had"]


@pytest.mark.parametrize("name", DETERMINISM)
def test_bitwise_deterministic_at_full_size(require_gpu, name):
    w = WORKLOADS[name]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert w.B * w.Hq * ((w.N + 255) // 256) > cus, "the workload launches in paired mode"
    q, k, v = (t.to(torch.bfloat16).cuda() for t in make_inputs(w))
    out = torch.empty((w.B, w.N, w.Hq, w.d_v), dtype=torch.bfloat16, device="cuda")
    if w.dtype == "bf16":
        fn = lambda: miattn.attn_fwd(q, k, v, out=out)  # noqa: E731
    else:
        (cq, sq), (ck, sk) = (miattn.attn_quantize_fp8(t, hadamard=w.hadamard) for t in (q, k))
        cv, sv = miattn.attn_quantize_fp8(v)
        fn = lambda: miattn.attn_fwd(cq, ck, cv, sq, sk, sv, out=out)  # noqa: E731
    _bitwise_100(fn, out)


def test_bitwise_deterministic_chunk_and_block64_at_full_size(require_gpu):
    """attn_fwd_chunk (last 8192 of 32768 positions, LSE written) and
    attn_fwd_block64 (with and without probability block scaling) at 32K, in
    the benchmark's launch configuration: 100 launches each, same bits."""
    w = WORKLOADS["fp8_mha_n32k"]
    q, k, v = (t.to(torch.bfloat16).cuda() for t in make_inputs(w))
    Nq = 8192
    (cq, sq), (ck, sk), (cv, sv) = (miattn.attn_quantize_fp8(t) for t in (q[:, w.N - Nq:].contiguous(), k, v))
    out = torch.empty((1, Nq, w.Hq, w.d_v), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((1, w.Hq, Nq), dtype=torch.float32, device="cuda")
    miattn.attn_fwd_chunk(cq, ck, cv, sq, sk, sv, out=out, lse=lse)
    torch.cuda.synchronize()
    lse0 = lse.clone()
    _bitwise_100(lambda: miattn.attn_fwd_chunk(cq, ck, cv, sq, sk, sv, out=out, lse=lse), out)
    assert torch.equal(lse.view(torch.int32), lse0.view(torch.int32))
    del cq, ck, cv, sq, sk, sv, out, lse
    (bq, bsq), (bk, bsk), (bv, bsv) = (miattn.attn_quantize_fp8_block64(t) for t in (q, k, v))
    out = torch.empty((1, w.N, w.Hq, w.d_v), dtype=torch.bfloat16, device="cuda")
    for ps in (False, True):
        _bitwise_100(lambda: miattn.attn_fwd_block64(bq, bk, bv, bsq, bsk, bsv, out=out, with_lse=False,
                                                     p_block_scale=ps), out)
