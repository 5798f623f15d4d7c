"""Exact causal softmax attention in fp64 -- test infrastructure only.

Definition followed (page legend in ``oracle/__init__.py``): the method is a
forward, causal (prefill) attention pass ([P2] "What Zyphra Reported", [P3]
"TL;DR"); FlashAttention tiling plus online softmax reaches exactly the plain
softmax-attention result without materialising the score matrix ([P1] "Why
prefill attention deserves dedicated optimization"), so the oracle is that plain
result.  The pages measure error against fp64 attention ([P3] "ZYFA 的 FP8
注意力有多准确？"), so everything here runs in fp64.

Readings taken where the pages are silent:

* causal alignment: equal query and key lengths; key j is visible to query i
  iff j <= i;
* softmax scale tau = 1/sqrt(d_qk);
* grouped-query mapping: query head h reads key/value head h // (Hq // Hkv);
* layout: [B, N, H, d] (batch, sequence, head, channel).

The query-row loop below processes rows in slabs only to bound memory; each
output row is computed with exactly the same operations whatever the slab size.

``attn_chunk_ref_rows`` is the same definition for a chunk of queries placed
after a prefix of keys (chunked prefill, the step beside the pages' plain causal
prefill): with Nq queries and Nk >= Nq keys, query row i sits at position
i + Nk - Nq and sees keys j <= i + Nk - Nq.  It also returns the natural-log
sum of exp of each row's scaled scores (LSE), the quantity with which results
over separate key ranges combine.  Reading where the pages are silent: the
queries are the *last* Nq positions (bottom-right alignment), the only
placement under which every query of a causal chunk sees at least one key.
"""

from __future__ import annotations

import math

import numpy as np


def _as_f64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # a torch tensor: upcast exactly
        x = x.detach().to("cpu")
        import torch

        x = x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _check_shapes(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, N, H, d]")
    B, N, Hq, dqk = q.shape
    if k.shape[0] != B or k.shape[1] != N or k.shape[3] != dqk:
        raise ValueError(f"k shape {k.shape} does not match q {q.shape}")
    Hkv = k.shape[2]
    if v.shape[:3] != (B, N, Hkv):
        raise ValueError(f"v shape {v.shape} does not match k {k.shape}")
    if Hkv == 0 or Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    return B, N, Hq, Hkv, dqk, v.shape[3]


def attn_ref_rows(q, k, v, rows=None, softmax_scale=None, slab=256):
    """Causal attention output for the selected query rows, fp64.

    q: [B, N, Hq, d_qk]; k: [B, N, Hkv, d_qk]; v: [B, N, Hkv, d_v]; any real
    dtype (upcast exactly to fp64).  ``rows``: 1-D int array of query indices
    (default: all).  Returns fp64 [B, len(rows), Hq, d_v].

    For query i of head h (kv head g = h // (Hq // Hkv)):
        s_j = tau * <q_i, k_j>            for j <= i
        w_j = exp(s_j - max s) / sum_j' exp(s_j' - max s)
        o_i = sum_j w_j v_j
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, N, Hq, Hkv, dqk, dv = _check_shapes(q, k, v)
    tau = (1.0 / math.sqrt(dqk)) if softmax_scale is None else float(softmax_scale)
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    if rows.size and (rows.min() < 0 or rows.max() >= N):
        raise ValueError("row index out of range")
    group = Hq // Hkv
    out = np.zeros((B, rows.size, Hq, dv), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            g = h // group
            kh = k[b, :, g, :]  # [N, dqk]
            vh = v[b, :, g, :]  # [N, dv]
            for s0 in range(0, rows.size, slab):
                r = rows[s0 : s0 + slab]
                hi = int(r.max()) + 1  # keys beyond the last row are never visible
                s = tau * (q[b, r, h, :] @ kh[:hi].T)  # [len(r), hi]
                visible = np.arange(hi)[None, :] <= r[:, None]
                s = np.where(visible, s, -np.inf)
                m = s.max(axis=1, keepdims=True)
                e = np.exp(s - m)  # masked entries give exp(-inf) = 0 exactly
                w = e / e.sum(axis=1, keepdims=True)
                out[b, s0 : s0 + r.size, h, :] = w @ vh[:hi]
    return out


def attn_chunk_ref_rows(q, k, v, rows=None, softmax_scale=None, slab=256):
    """Chunked-prefill causal attention and its LSE, fp64.

    q: [B, Nq, Hq, d_qk]; k: [B, Nk, Hkv, d_qk]; v: [B, Nk, Hkv, d_v] with
    Nq <= Nk.  ``rows``: query-row indices in [0, Nq) (default: all).
    Returns (out fp64 [B, len(rows), Hq, d_v], lse fp64 [B, Hq, len(rows)]).

    For query row i of head h (kv head g = h // (Hq // Hkv)), p = i + Nk - Nq:
        s_j = tau * <q_i, k_j>             for j <= p
        m = max_j s_j
        lse_i = m + log sum_j exp(s_j - m)
        o_i = sum_j exp(s_j - lse_i) v_j
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, N, H, d]")
    B, Nq, Hq, dqk = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    if k.shape[0] != B or k.shape[3] != dqk or v.shape[:3] != (B, Nk, Hkv):
        raise ValueError(f"shapes q {q.shape} k {k.shape} v {v.shape} do not match")
    if Nq > Nk:
        raise ValueError("a chunk has at most as many queries as keys")
    if Hkv == 0 or Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    dv = v.shape[3]
    off = Nk - Nq
    tau = (1.0 / math.sqrt(dqk)) if softmax_scale is None else float(softmax_scale)
    rows = np.arange(Nq) if rows is None else np.asarray(rows, dtype=np.int64)
    if rows.size and (rows.min() < 0 or rows.max() >= Nq):
        raise ValueError("row index out of range")
    group = Hq // Hkv
    out = np.zeros((B, rows.size, Hq, dv), dtype=np.float64)
    lse = np.zeros((B, Hq, rows.size), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            g = h // group
            for s0 in range(0, rows.size, slab):
                r = rows[s0 : s0 + slab]
                pos = r + off  # sequence position of each query row
                hi = int(pos.max()) + 1  # keys beyond the last position are never visible
                s = tau * (q[b, r, h, :] @ k[b, :hi, g, :].T)  # [len(r), hi]
                s = np.where(np.arange(hi)[None, :] <= pos[:, None], s, -np.inf)
                m = s.max(axis=1, keepdims=True)
                e = np.exp(s - m)
                l = e.sum(axis=1, keepdims=True)
                out[b, s0 : s0 + r.size, h, :] = (e / l) @ v[b, :hi, g, :]
                lse[b, h, s0 : s0 + r.size] = (m + np.log(l))[:, 0]
    return out, lse


def attn_ref(q, k, v, softmax_scale=None):
    """Causal attention for every query row: fp64 [B, N, Hq, d_v]."""
    return attn_ref_rows(q, k, v, None, softmax_scale)


def causal_weights_ref(q, k, b=0, h=0, softmax_scale=None):
    """The full causal softmax weight matrix W[i, j] of one (batch, head), fp64.

    Exposed so that tests can check the weights themselves (rows sum to one,
    zeros above the diagonal).  Same arithmetic as ``attn_ref_rows``.
    """
    q, k = _as_f64(q), _as_f64(k)
    Hq, Hkv, dqk = q.shape[2], k.shape[2], q.shape[3]
    tau = (1.0 / math.sqrt(dqk)) if softmax_scale is None else float(softmax_scale)
    g = h // (Hq // Hkv)
    N = q.shape[1]
    s = tau * (q[b, :, h, :] @ k[b, :, g, :].T)
    s = np.where(np.tril(np.ones((N, N), dtype=bool)), s, -np.inf)
    e = np.exp(s - s.max(axis=1, keepdims=True))
    return e / e.sum(axis=1, keepdims=True)
