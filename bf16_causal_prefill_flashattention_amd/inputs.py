"""Seeded synthetic workloads for causal prefill attention.

This module draws random inputs and nothing else: it holds none of the
attention, quantization or rotation arithmetic, and both the GPU path's callers
(tests, benchmark) and the CPU oracle's tests take their inputs from it.

Shapes and value structure follow the workloads of the pages (page legend: [P2]
"Zyphra Says Its AMD MI355X Attention Kernel Is 1.76x Faster", [P3] "Zyphra 开源
ZYFA：面向 AMD MI355X 的 FP8 FlashAttention，最高提速 1.76 倍"): head dim 128 with
grouped-query attention at 16K tokens as in Mistral-7B / Qwen3-8B, the
multi-head-latent shape 192/128 as in DeepSeek-V2, and Gaussian inputs up to 32K
tokens ([P2] "What Zyphra Reported", [P3] "ZYFA 有多快？").  Captured model
activations are not available, so heavy-tailed "activation-like" inputs are
stood in for by Gaussian Q/K with a few large channels.

Recipe (one torch CPU generator per tensor, fp32 N(0, 1)):
  Q <- seed, K <- seed + 1, V <- seed + 2, outlier channels <- seed + 3.
  With ``outliers = c``: for every (batch, kv head g) draw c distinct channels
  (a random permutation's first c entries), multiply those channels by
  ``outlier_gain`` in K[:, :, g] and in Q[:, :, h] for every query head h of g's
  group (aligned channels).  V stays N(0, 1).
  With ``kv_decades = D > 0``: every position n of every batch b gets a gain
  10^(-D * u[b, n]), u ~ Uniform[0, 1) from seed + 4, applied to its K and V
  rows of all heads (magnitudes that drift along the sequence, the case finer
  FP8 scale granularity is for).
  ``scales`` names the FP8 scale granularity a workload is quantized with:
  "head" (one scale per batch and head) or "block64" (one per 64 positions);
  ``p_block_scale`` asks the block-scaled attention to scale its probabilities
  per block by powers of two as well.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str  # "bf16" or "fp8"
    B: int
    Hq: int
    Hkv: int
    N: int
    d_qk: int
    d_v: int
    outliers: int = 0
    outlier_gain: float = 20.0
    hadamard: bool = False
    seed: int = 0
    kv_decades: float = 0.0
    scales: str = "head"
    p_block_scale: bool = False
    note: str = field(default="", compare=False)

    @property
    def causal_flops(self) -> float:
        """B * Hq * N^2 * (d_qk + d_v): the causal half of the dense
        2 * N^2 * (d_qk + d_v) multiply-add count per head."""
        return float(self.B) * self.Hq * float(self.N) ** 2 * (self.d_qk + self.d_v)

    def with_(self, **kw) -> "Workload":
        d = {k: getattr(self, k) for k in self.__dataclass_fields__}
        d.update(kw)
        return Workload(**d)


def _w(*a, **k):
    return Workload(*a, **k)


# Named workloads: the five shapes/structures the path is specified on.
WORKLOADS = {
    "bf16_mha_n512": _w("bf16_mha_n512", "bf16", 1, 2, 2, 512, 128, 128,
                        note="small exact-check case"),
    "bf16_gqa_n16k": _w("bf16_gqa_n16k", "bf16", 1, 32, 8, 16384, 128, 128, outliers=4,
                        note="GQA, activation-like outlier channels"),
    "fp8_mha_n1k": _w("fp8_mha_n1k", "fp8", 1, 32, 32, 1024, 128, 128),
    "bf16_mha_n1k": _w("bf16_mha_n1k", "bf16", 1, 32, 32, 1024, 128, 128,
                       note="BF16 point of the short-sequence case"),
    "fp8_mha_n4k": _w("fp8_mha_n4k", "fp8", 1, 32, 32, 4096, 128, 128),
    "fp8_mha_n16k": _w("fp8_mha_n16k", "fp8", 1, 32, 32, 16384, 128, 128),
    "fp8_mha_n32k": _w("fp8_mha_n32k", "fp8", 1, 32, 32, 32768, 128, 128),
    "bf16_mha_n32k": _w("bf16_mha_n32k", "bf16", 1, 32, 32, 32768, 128, 128,
                        note="BF16 point of the d=128, N=32K metric"),
    "fp8_gqa_n16k": _w("fp8_gqa_n16k", "fp8", 1, 32, 8, 16384, 128, 128, outliers=4),
    "fp8_gqa_n16k_had": _w("fp8_gqa_n16k_had", "fp8", 1, 32, 8, 16384, 128, 128,
                           outliers=4, hadamard=True),
    "fp8_mla_n32k": _w("fp8_mla_n32k", "fp8", 1, 16, 16, 32768, 192, 128),
    "fp8_mha_n32k_block64": _w("fp8_mha_n32k_block64", "fp8", 1, 32, 32, 32768, 128, 128, scales="block64",
                               note="the FP8 headline shape with per-64-position scales"),
    "fp8_mha_n32k_block64_pscale": _w("fp8_mha_n32k_block64_pscale", "fp8", 1, 32, 32, 32768, 128, 128,
                                      scales="block64", p_block_scale=True,
                                      note="as fp8_mha_n32k_block64, probabilities scaled per block too"),
}


def _randn(shape, seed: int) -> torch.Tensor:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return torch.randn(*shape, generator=g, dtype=torch.float32)


def outlier_channels(w: Workload) -> torch.Tensor:
    """[B, Hkv, outliers] int64 channel indices (empty if no outliers)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(w.seed) + 3)
    idx = torch.empty((w.B, w.Hkv, w.outliers), dtype=torch.int64)
    for b in range(w.B):
        for h in range(w.Hkv):
            idx[b, h] = torch.randperm(w.d_qk, generator=g)[: w.outliers]
    return idx


def make_qkv(w: Workload):
    """fp32 CPU tensors q [B,N,Hq,d_qk], k [B,N,Hkv,d_qk], v [B,N,Hkv,d_v]."""
    if w.Hkv <= 0 or w.Hq % w.Hkv:
        raise ValueError("Hq must be a positive multiple of Hkv")
    q = _randn((w.B, w.N, w.Hq, w.d_qk), w.seed)
    k = _randn((w.B, w.N, w.Hkv, w.d_qk), w.seed + 1)
    v = _randn((w.B, w.N, w.Hkv, w.d_v), w.seed + 2)
    if w.outliers:
        grp = w.Hq // w.Hkv
        ch = outlier_channels(w)
        for b in range(w.B):
            for g in range(w.Hkv):
                c = ch[b, g]
                k[b, :, g, c] *= w.outlier_gain
                for h in range(g * grp, (g + 1) * grp):
                    q[b, :, h, c] *= w.outlier_gain
    if w.kv_decades:
        g = torch.Generator(device="cpu")
        g.manual_seed(int(w.seed) + 4)
        u = torch.rand((w.B, w.N), generator=g, dtype=torch.float32)
        gain = torch.pow(torch.tensor(10.0), -w.kv_decades * u)[:, :, None, None]
        k *= gain
        v *= gain
    return q, k, v


def make_inputs(w: Workload):
    """Inputs in the form the attention entry point's callers hold them: bf16
    for the BF16 workloads (RNE from the fp32 draws), fp32 activations for the
    FP8 workloads (quantized by the FP8 front end)."""
    q, k, v = make_qkv(w)
    if w.dtype == "bf16":
        return q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)
    return q, k, v
