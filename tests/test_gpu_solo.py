"""The 4-wave mode (128-query work items, one wave per SIMD) against the 8-wave
ping-pong mode, bit for bit.

A launch of at most 1536 keys whose 256-query tiles leave CUs idle while its
128-query items fit one per CU runs 4-wave workgroups; twice as many heads
fill the CUs with 256-query tiles and run the 8-wave kernel.  Each wave owns
32 query rows in both modes and walks the same key tiles in the same order
with the same instruction sequence per row, so the first half of the heads of
the larger launch must equal the smaller launch exactly (output and LSE).
Parity of small launches with the oracle is covered by the other GPU tests,
whose small shapes take this mode.
"""

import pytest
import torch

import bf16_causal_prefill_flashattention_amd as miattn

pytestmark = pytest.mark.gpu

SOLO_MAX_KEYS = 1536


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def _run(kind, mode, q, k, v, scales):
    if kind == "bf16":
        return miattn.attn_fwd_chunk(q, k, v)
    qs, ks, vs = scales
    return miattn.attn_fwd_fp8(q, k, v, qs, ks, vs, scales=kind, p_mode=mode)


def _inputs(kind, B, H, G, Nq, Nk, dqk, seed):
    g = torch.Generator().manual_seed(seed)
    dev = torch.device("cuda:0")
    q = torch.randn(B, Nq, H, dqk, generator=g).to(torch.bfloat16).to(dev)
    k = torch.randn(B, Nk, H // G, dqk, generator=g).to(torch.bfloat16).to(dev)
    v = torch.randn(B, Nk, H // G, 128, generator=g).to(torch.bfloat16).to(dev)
    if kind == "bf16":
        return (q, k, v), None
    quant = miattn.attn_quantize_fp8_block64 if kind == "block64" else miattn.attn_quantize_fp8
    (cq, sq), (ck, sk), (cv, sv) = (quant(t) for t in (q, k, v))
    return (cq, ck, cv), (sq, sk, sv)


CASES = [
    ("head", "lean_tile", 128, 1, 1024, 1024),
    ("head", "lean", 128, 1, 1024, 1024),
    ("head", "exact", 128, 1, 1024, 1024),
    ("head", "lean_block", 128, 4, 1024, 1024),
    ("head", "exact_tile", 128, 1, 700, 1536),
    ("block64", "lean_block", 128, 1, 1024, 1024),
    ("block64", "lean", 128, 2, 1000, 1500),
    ("head", "lean_tile", 192, 1, 1024, 1024),
    ("bf16", "lean", 128, 1, 1024, 1024),
    ("bf16", "lean", 128, 4, 777, 1400),
    ("bf16", "lean", 192, 1, 1024, 1024),
]


@pytest.mark.parametrize("kind,mode,dqk,G,Nq,Nk", CASES)
def test_four_wave_items_match_eight_wave_tiles(kind, mode, dqk, G, Nq, Nk):
    assert Nk <= SOLO_MAX_KEYS
    cus = _cus()
    items128 = (Nq + 127) // 128
    tiles256 = (Nq + 255) // 256
    # heads (a multiple of G): the small launch's 256-query tiles leave CUs
    # idle and its 128-query items fit one per CU (4-wave mode); the doubled
    # launch's 128-query items do not fit, while its 256-query tiles still
    # get a workgroup each (8-wave mode, one tile per workgroup, every walk
    # upward as in the 4-wave mode)
    H = min(cus // items128, cus // (2 * tiles256)) // G * G
    assert H >= G
    assert H * tiles256 < cus and H * items128 <= cus
    assert 2 * H * items128 > cus and 2 * H * tiles256 <= cus
    (q2, k2, v2), sc2 = _inputs(kind, 1, 2 * H, G, Nq, Nk, dqk, seed=Nq + 7 * G)
    hk = H // G
    q1, k1, v1 = q2[:, :, :H].contiguous(), k2[:, :, :hk].contiguous(), v2[:, :, :hk].contiguous()
    sc1 = None
    if sc2 is not None:
        sc1 = (sc2[0][:, :H].contiguous(), sc2[1][:, :hk].contiguous(), sc2[2][:, :hk].contiguous())
    o1, l1 = _run(kind, mode, q1, k1, v1, sc1)
    o2, l2 = _run(kind, mode, q2, k2, v2, sc2)
    torch.cuda.synchronize()
    assert torch.isfinite(o1.float()).all()
    a, b = o1.view(torch.int16), o2[:, :, :H].contiguous().view(torch.int16)
    assert torch.equal(a, b), f"{int((a != b).sum())} of {a.numel()} output elements differ"
    assert torch.equal(l1.view(torch.int32), l2[:, :H].contiguous().view(torch.int32))
