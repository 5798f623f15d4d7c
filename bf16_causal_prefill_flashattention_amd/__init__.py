"""Causal forward (prefill) attention for AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI of ``libmiattn.so`` (declared in
``include/miattn.h``).  It only marshals arguments: every step of the
computation runs in the library's HIP kernels.  PyTorch supplies device memory
and the current stream.  There is no fallback: if the library is not built, or
a tensor is not on a GPU, the call raises.

Entry points (same names as the C ABI):

* ``attn_fwd(q, k, v, q_scale=None, k_scale=None, v_scale=None, out=None)``
* ``attn_fwd_chunk(q, k, v, q_scale=None, k_scale=None, v_scale=None, out=None,
  lse=None, with_lse=True, softmax_scale=None)``
* ``attn_quantize_fp8(x, hadamard=False, out=None, scale=None)``
* ``attn_fwd_block64(q, k, v, q_scale, k_scale, v_scale, out=None, lse=None,
  with_lse=True, softmax_scale=None, p_block_scale=False)`` (FP8 with
  per-64-position scales, optionally power-of-two scaled probabilities)
* ``attn_quantize_fp8_block64(x, hadamard=False, out=None, scale=None)``
* ``attn_fwd_fp8(q, k, v, q_scale, k_scale, v_scale, out=None, lse=None,
  with_lse=True, softmax_scale=None, scales="head", p_mode="lean")`` (FP8
  with a chosen scale granularity and probability mode, ``P_MODES``)
* ``attn_fwd_ws_size(B, Hq, Hkv, Nq, Nk, d_qk, d_v, fp8, scales="head",
  p_mode=DEFAULT_P_MODE, device=None)`` and ``attn_fwd_ws(q, k, v, q_scale=None,
  k_scale=None, v_scale=None, out=None, lse=None, with_lse=True,
  softmax_scale=None, scales="head", p_mode=DEFAULT_P_MODE, workspace=None)``
  (BF16 or FP8 with a workspace, which lets launches that leave compute units
  idle split their keys; the workspace is allocated here when not given), and
  ``attn_fwd_ws_bind(...)``, which checks and marshals such a call once and
  returns a callable that enqueues it again
* ``attn_status_string(status)``, ``attn_version()``

and ``flash_attn_func``, a ``flash_attn_func``-style drop-in over them (BSHD
torch tensors in, causal, optional FP8 with automatic per-head or
per-64-position quantization).
"""

from __future__ import annotations

import ctypes
import os

__all__ = [
    "attn_fwd",
    "attn_fwd_block64",
    "attn_fwd_chunk",
    "attn_fwd_fp8",
    "attn_fwd_ws",
    "attn_fwd_ws_bind",
    "attn_fwd_ws_size",
    "attn_quantize_fp8",
    "attn_quantize_fp8_block64",
    "attn_status_string",
    "attn_version",
    "flash_attn_func",
    "library_path",
    "load_library",
    "MiattnError",
    "DTYPE_BF16",
    "DTYPE_FP8_E4M3",
    "P_MODES",
    "DEFAULT_P_MODE",
]

DTYPE_BF16 = 0
DTYPE_FP8_E4M3 = 1
SRC_FP32 = 0
SRC_BF16 = 1
SCALES = {"head": 0, "block64": 1}
# probability modes of the FP8 kernels (include/miattn.h, MIATTN_P_*)
P_MODES = {"lean": 0, "lean_block": 1, "exact": 2, "exact_block": 3, "lean_tile": 4, "exact_tile": 5}
DEFAULT_P_MODE = "lean_tile"  # MIATTN_P_DEFAULT: what attn_fwd and attn_fwd_chunk use on FP8 inputs

_LIB = None
_HERE = os.path.dirname(os.path.abspath(__file__))


class MiattnError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed with status {status}: {attn_status_string(status)}")
        self.status = status


def library_path() -> str:
    return os.path.join(_HERE, "libmiattn.so")


def load_library() -> ctypes.CDLL:
    """Load libmiattn.so (built in-tree by ``build.py``); raise if missing."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built; run `python -m bf16_causal_prefill_flashattention_amd.build`"
        )
    lib = ctypes.CDLL(path)
    vp, ci, fp = ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, fp, fp, fp, vp]
    lib.attn_fwd.restype = ci
    lib.attn_fwd_chunk.argtypes = [vp, vp, vp, vp, fp, ci, ci, ci, ci, ci, ci, ci, ci, fp, fp, fp,
                                   ctypes.c_float, vp]
    lib.attn_fwd_chunk.restype = ci
    lib.attn_quantize_fp8.argtypes = [vp, ci, vp, fp, ci, ci, ci, ci, ci, vp]
    lib.attn_quantize_fp8.restype = ci
    lib.attn_fwd_block64.argtypes = [vp, vp, vp, vp, fp, ci, ci, ci, ci, ci, ci, ci, fp, fp, fp, ctypes.c_float, ci,
                                     vp]
    lib.attn_fwd_block64.restype = ci
    lib.attn_fwd_fp8.argtypes = [vp, vp, vp, vp, fp, ci, ci, ci, ci, ci, ci, ci, fp, fp, fp, ctypes.c_float, ci, ci,
                                 vp]
    lib.attn_fwd_fp8.restype = ci
    lib.attn_quantize_fp8_block64.argtypes = [vp, ci, vp, fp, ci, ci, ci, ci, ci, vp]
    lib.attn_quantize_fp8_block64.restype = ci
    sz = ctypes.c_size_t
    lib.attn_fwd_ws_size.argtypes = [ci, ci, ci, ci, ci, ci, ci, ci, ci, ci, ctypes.POINTER(sz)]
    lib.attn_fwd_ws_size.restype = ci
    lib.attn_fwd_ws.argtypes = [vp, vp, vp, vp, fp, ci, ci, ci, ci, ci, ci, ci, ci, fp, fp, fp, ctypes.c_float, ci,
                                ci, vp, sz, vp]
    lib.attn_fwd_ws.restype = ci
    lib.attn_fwd_noalloc.argtypes = [vp, vp, vp, vp, fp, ci, ci, ci, ci, ci, ci, ci, ci, fp, fp, fp, ctypes.c_float,
                                     ci, ci, vp]
    lib.attn_fwd_noalloc.restype = ci
    lib.attn_status_string.argtypes = [ci]
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_version.argtypes = []
    lib.attn_version.restype = ci
    _LIB = lib
    return lib


def attn_status_string(status: int) -> str:
    return load_library().attn_status_string(int(status)).decode()


def attn_version() -> int:
    return int(load_library().attn_version())


def _torch():
    import torch

    return torch


def _stream_handle(device) -> int:
    torch = _torch()
    return int(torch.cuda.current_stream(device).cuda_stream)


def _check_gpu_contig(name, t):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _as_codes(name, t):
    torch = _torch()
    if t.dtype == torch.uint8:
        return t
    if t.dtype == getattr(torch, "float8_e4m3fn", None):
        return t.view(torch.uint8)
    raise TypeError(f"{name} must be uint8 or float8_e4m3fn codes for the FP8 path")


def _attn_args(q, k, v, q_scale, k_scale, v_scale, block64=False):
    """Check q [B,Nq,Hq,d_qk], k [B,Nk,Hkv,d_qk], v [B,Nk,Hkv,d_v] and the FP8
    scales (per head, or per 64 positions with ``block64``); returns (q, k, v,
    dtype code, scale pointers, sizes)."""
    torch = _torch()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_gpu_contig(name, t)
        if t.dim() != 4:
            raise ValueError(f"{name} must be [B, N, H, d]")
    B, Nq, Hq, dqk = q.shape
    Nk, Hkv, dv = k.shape[1], k.shape[2], v.shape[3]
    if tuple(k.shape) != (B, Nk, Hkv, dqk) or tuple(v.shape[:3]) != (B, Nk, Hkv):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    if q.dtype == torch.bfloat16 and not block64:
        if k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
            raise TypeError("q, k, v must share one dtype")
        dtype = DTYPE_BF16
        ptr_s = [None, None, None]
    else:
        q, k, v = _as_codes("q", q), _as_codes("k", k), _as_codes("v", v)
        dtype = DTYPE_FP8_E4M3
        scales = []
        nbq, nbk = (Nq + 63) // 64, (Nk + 63) // 64
        shapes = ((B, Hq, nbq), (B, Hkv, nbk), (B, Hkv, nbk)) if block64 else ((B, Hq), (B, Hkv), (B, Hkv))
        for name, s, shape in zip(("q_scale", "k_scale", "v_scale"), (q_scale, k_scale, v_scale), shapes):
            if s is None:
                raise ValueError(f"{name} is required for the FP8 path")
            _check_gpu_contig(name, s)
            if s.dtype != torch.float32 or tuple(s.shape) != shape:
                raise ValueError(f"{name} must be float32 {shape}")
            scales.append(s)
        ptr_s = [s.data_ptr() for s in scales]
    return q, k, v, dtype, ptr_s, (B, Nq, Nk, Hq, Hkv, dqk, dv)


def _out_tensor(out, q, B, Nq, Hq, dv):
    torch = _torch()
    if out is None:
        return torch.empty((B, Nq, Hq, dv), dtype=torch.bfloat16, device=q.device)
    _check_gpu_contig("out", out)
    if out.dtype != torch.bfloat16 or tuple(out.shape) != (B, Nq, Hq, dv):
        raise ValueError(f"out must be bfloat16 {(B, Nq, Hq, dv)}")
    return out


def attn_fwd(q, k, v, q_scale=None, k_scale=None, v_scale=None, out=None):
    """Causal attention forward.  q [B,N,Hq,d_qk], k [B,N,Hkv,d_qk],
    v [B,N,Hkv,d_v] (contiguous BSHD, on one GPU).  BF16 tensors select the
    BF16 path; uint8 / float8_e4m3fn codes select the FP8 path, which needs
    fp32 scales q_scale [B,Hq], k_scale [B,Hkv], v_scale [B,Hkv].  Returns
    ``out`` (bf16 [B,N,Hq,d_v]), allocated if not given."""
    q, k, v, dtype, ptr_s, (B, N, Nk, Hq, Hkv, dqk, dv) = _attn_args(q, k, v, q_scale, k_scale, v_scale)
    if Nk != N:
        raise ValueError(f"q and k must have the same length (got {N} and {Nk}); see attn_fwd_chunk")
    out = _out_tensor(out, q, B, N, Hq, dv)
    st = load_library().attn_fwd(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, Hq, Hkv, N, dqk, dv, dtype,
        ptr_s[0], ptr_s[1], ptr_s[2], _stream_handle(q.device),
    )
    if st != 0:
        raise MiattnError("attn_fwd", st)
    return out


def attn_fwd_chunk(q, k, v, q_scale=None, k_scale=None, v_scale=None, out=None, lse=None, with_lse=True,
                   softmax_scale=None):
    """One chunk of a chunked causal prefill: q [B,Nq,Hq,d_qk] holds the last
    Nq positions of a sequence whose first Nk >= Nq keys and values are
    k [B,Nk,Hkv,d_qk], v [B,Nk,Hkv,d_v]; query row i sees keys
    j <= i + Nk - Nq.  Dtypes and scales as for ``attn_fwd``.
    ``softmax_scale``: tau (default 1/sqrt(d_qk)).  Returns ``(out, lse)``:
    out bf16 [B,Nq,Hq,d_v]; lse fp32 [B,Hq,Nq], the natural-log sum of
    exp(tau <q_i, k_j>) over the visible keys, or None when ``with_lse`` is
    false and no ``lse`` tensor is given."""
    q, k, v, dtype, ptr_s, (B, Nq, Nk, Hq, Hkv, dqk, dv) = _attn_args(q, k, v, q_scale, k_scale, v_scale)
    out = _out_tensor(out, q, B, Nq, Hq, dv)
    lse = _lse_tensor(lse, with_lse, q, B, Hq, Nq)
    st = load_library().attn_fwd_chunk(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), None if lse is None else lse.data_ptr(),
        B, Hq, Hkv, Nq, Nk, dqk, dv, dtype, ptr_s[0], ptr_s[1], ptr_s[2],
        0.0 if softmax_scale is None else float(softmax_scale), _stream_handle(q.device),
    )
    if st != 0:
        raise MiattnError("attn_fwd_chunk", st)
    return out, lse


def attn_quantize_fp8(x, hadamard: bool = False, out=None, scale=None):
    """Per-(batch, head) FP8 e4m3fn quantization of x [B,N,H,d] (fp32 or bf16,
    on a GPU).  Returns (codes uint8 [B,N,H,d], scale fp32 [B,H])."""
    return _quantize("attn_quantize_fp8", x, hadamard, out, scale, lambda B, N, H: (B, H))


def _lse_tensor(lse, with_lse, q, B, Hq, Nq):
    torch = _torch()
    if lse is None and with_lse:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _check_gpu_contig("lse", lse)
        if lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, Nq):
            raise ValueError(f"lse must be float32 {(B, Hq, Nq)}")
    return lse


def attn_fwd_block64(q, k, v, q_scale, k_scale, v_scale, out=None, lse=None, with_lse=True, softmax_scale=None,
                     p_block_scale=False):
    """FP8 causal attention with per-64-position scales: q [B,Nq,Hq,d_qk],
    k [B,Nk,Hkv,d_qk], v [B,Nk,Hkv,d_v] e4m3 codes (uint8 or float8_e4m3fn),
    q_scale fp32 [B,Hq,ceil(Nq/64)], k_scale and v_scale fp32
    [B,Hkv,ceil(Nk/64)] (powers of two, as ``attn_quantize_fp8_block64``
    writes them).  Query row i sees keys j <= i + Nk - Nq.  ``p_block_scale``
    shifts each query's probabilities of every 64-key step by a power of two
    of their own before rounding (undone by the scaled MFMAs), which keeps key
    blocks far below the row max at e4m3 precision.  Returns ``(out, lse)`` as
    ``attn_fwd_chunk``."""
    torch = _torch()
    if q.dtype == torch.bfloat16:
        raise TypeError("attn_fwd_block64 takes e4m3 codes (quantize with attn_quantize_fp8_block64)")
    q, k, v, _, ptr_s, (B, Nq, Nk, Hq, Hkv, dqk, dv) = _attn_args(q, k, v, q_scale, k_scale, v_scale, True)
    out = _out_tensor(out, q, B, Nq, Hq, dv)
    lse = _lse_tensor(lse, with_lse, q, B, Hq, Nq)
    st = load_library().attn_fwd_block64(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), None if lse is None else lse.data_ptr(),
        B, Hq, Hkv, Nq, Nk, dqk, dv, ptr_s[0], ptr_s[1], ptr_s[2],
        0.0 if softmax_scale is None else float(softmax_scale), 1 if p_block_scale else 0,
        _stream_handle(q.device),
    )
    if st != 0:
        raise MiattnError("attn_fwd_block64", st)
    return out, lse


def attn_fwd_fp8(q, k, v, q_scale, k_scale, v_scale, out=None, lse=None, with_lse=True, softmax_scale=None,
                 scales="head", p_mode="lean"):
    """FP8 causal attention with a chosen scale granularity (``scales``:
    "head" -- q_scale [B,Hq], k_scale and v_scale [B,Hkv], as ``attn_fwd``; or
    "block64" -- per-64-position scales, as ``attn_fwd_block64``) and
    probability mode (``p_mode``: "lean", "lean_block", "lean_tile",
    "exact", "exact_block", "exact_tile"; see ``P_MODES`` and MIATTN_P_* in
    include/miattn.h).
    q [B,Nq,Hq,d_qk], k [B,Nk,Hkv,d_qk], v [B,Nk,Hkv,d_v] e4m3 codes; query row
    i sees keys j <= i + Nk - Nq.  Returns ``(out, lse)`` as
    ``attn_fwd_chunk``."""
    torch = _torch()
    if scales not in SCALES:
        raise ValueError(f"scales must be one of {sorted(SCALES)}")
    if p_mode not in P_MODES:
        raise ValueError(f"p_mode must be one of {sorted(P_MODES)}")
    if q.dtype == torch.bfloat16:
        raise TypeError("attn_fwd_fp8 takes e4m3 codes")
    block64 = scales == "block64"
    q, k, v, _, ptr_s, (B, Nq, Nk, Hq, Hkv, dqk, dv) = _attn_args(q, k, v, q_scale, k_scale, v_scale, block64)
    out = _out_tensor(out, q, B, Nq, Hq, dv)
    lse = _lse_tensor(lse, with_lse, q, B, Hq, Nq)
    st = load_library().attn_fwd_fp8(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), None if lse is None else lse.data_ptr(),
        B, Hq, Hkv, Nq, Nk, dqk, dv, ptr_s[0], ptr_s[1], ptr_s[2],
        0.0 if softmax_scale is None else float(softmax_scale), SCALES[scales], P_MODES[p_mode],
        _stream_handle(q.device),
    )
    if st != 0:
        raise MiattnError("attn_fwd_fp8", st)
    return out, lse


_WS_SIZES = {}  # (device index, arguments) -> attn_fwd_ws_size bytes


def attn_fwd_ws_size(B, Hq, Hkv, Nq, Nk, d_qk, d_v, fp8, scales="head", p_mode=DEFAULT_P_MODE, device=None) -> int:
    """Workspace bytes ``attn_fwd_ws`` needs for these sizes on ``device`` (the
    current GPU by default); 0 when the launch does not split its keys."""
    torch = _torch()
    if scales not in SCALES:
        raise ValueError(f"scales must be one of {sorted(SCALES)}")
    if p_mode not in P_MODES:
        raise ValueError(f"p_mode must be one of {sorted(P_MODES)}")
    idx = torch.cuda.current_device() if device is None else torch.device(device).index
    idx = torch.cuda.current_device() if idx is None else idx
    key = (idx, B, Hq, Hkv, Nq, Nk, d_qk, d_v, bool(fp8), scales, p_mode)
    n = _WS_SIZES.get(key)
    if n is None:
        c = ctypes.c_size_t(0)
        with torch.cuda.device(idx):  # the figure depends on the device's compute units
            st = load_library().attn_fwd_ws_size(B, Hq, Hkv, Nq, Nk, d_qk, d_v,
                                                 DTYPE_FP8_E4M3 if fp8 else DTYPE_BF16, SCALES[scales],
                                                 P_MODES[p_mode], ctypes.byref(c))
        if st != 0:
            raise MiattnError("attn_fwd_ws_size", st)
        n = _WS_SIZES[key] = int(c.value)
    return n


def attn_fwd_ws_bind(q, k, v, q_scale=None, k_scale=None, v_scale=None, out=None, lse=None, with_lse=True,
                     softmax_scale=None, scales="head", p_mode=DEFAULT_P_MODE, workspace=None):
    """Check and marshal an ``attn_fwd_ws`` call once.  Returns ``(call, out,
    lse)``: ``call()`` enqueues the call on the stream that was current here,
    with these tensors (for loops over fixed buffers; the tensors must stay
    alive).  Arguments as ``attn_fwd_ws``."""
    torch = _torch()
    if scales not in SCALES:
        raise ValueError(f"scales must be one of {sorted(SCALES)}")
    if p_mode not in P_MODES:
        raise ValueError(f"p_mode must be one of {sorted(P_MODES)}")
    block64 = scales == "block64" and q.dtype != torch.bfloat16
    q, k, v, dtype, ptr_s, (B, Nq, Nk, Hq, Hkv, dqk, dv) = _attn_args(q, k, v, q_scale, k_scale, v_scale, block64)
    out = _out_tensor(out, q, B, Nq, Hq, dv)
    lse = _lse_tensor(lse, with_lse, q, B, Hq, Nq)
    need = attn_fwd_ws_size(B, Hq, Hkv, Nq, Nk, dqk, dv, dtype == DTYPE_FP8_E4M3, scales, p_mode, q.device)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        _check_gpu_contig("workspace", workspace)
        if workspace.device != q.device:
            raise ValueError("workspace must be on the device of q")
    argv = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), None if lse is None else lse.data_ptr(),
            B, Hq, Hkv, Nq, Nk, dqk, dv, dtype, ptr_s[0], ptr_s[1], ptr_s[2],
            0.0 if softmax_scale is None else float(softmax_scale), SCALES[scales], P_MODES[p_mode],
            None if workspace is None else workspace.data_ptr(),
            0 if workspace is None else workspace.numel() * workspace.element_size(), _stream_handle(q.device))
    fn = load_library().attn_fwd_ws
    keep = (q, k, v, out, lse, workspace)  # noqa: F841  (held by the closure)

    def call():
        st = fn(*argv)
        if st != 0:
            raise MiattnError("attn_fwd_ws", st)
        return keep

    return call, out, lse


def attn_fwd_ws(q, k, v, q_scale=None, k_scale=None, v_scale=None, out=None, lse=None, with_lse=True,
                softmax_scale=None, scales="head", p_mode=DEFAULT_P_MODE, workspace=None):
    """Causal attention through ``attn_fwd_ws``: BF16 tensors as
    ``attn_fwd_chunk`` (``scales`` and ``p_mode`` unused), e4m3 codes as
    ``attn_fwd_fp8``.  A launch whose query tiles leave compute units idle
    splits its keys over them, with partial results in ``workspace`` (a uint8
    GPU tensor of at least ``attn_fwd_ws_size`` bytes; allocated here when
    None).  Returns ``(out, lse)`` as ``attn_fwd_chunk``."""
    call, out, lse = attn_fwd_ws_bind(q, k, v, q_scale, k_scale, v_scale, out, lse, with_lse, softmax_scale, scales,
                                      p_mode, workspace)
    call()
    return out, lse


def _quantize(fn_name, x, hadamard, out, scale, scale_shape):
    torch = _torch()
    _check_gpu_contig("x", x)
    if x.dim() != 4:
        raise ValueError("x must be [B, N, H, d]")
    if x.dtype == torch.float32:
        src = SRC_FP32
    elif x.dtype == torch.bfloat16:
        src = SRC_BF16
    else:
        raise TypeError("x must be float32 or bfloat16")
    B, N, H, d = x.shape
    shape = scale_shape(B, N, H)
    if out is None:
        out = torch.empty((B, N, H, d), dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = torch.empty(shape, dtype=torch.float32, device=x.device)
    _check_gpu_contig("out", out)
    _check_gpu_contig("scale", scale)
    if out.dtype != torch.uint8 or tuple(out.shape) != (B, N, H, d):
        raise ValueError("out must be uint8 [B, N, H, d]")
    if scale.dtype != torch.float32 or tuple(scale.shape) != shape:
        raise ValueError(f"scale must be float32 {shape}")
    st = getattr(load_library(), fn_name)(
        x.data_ptr(), src, out.data_ptr(), scale.data_ptr(), B, H, N, d, 1 if hadamard else 0,
        _stream_handle(x.device),
    )
    if st != 0:
        raise MiattnError(fn_name, st)
    return out, scale


def attn_quantize_fp8_block64(x, hadamard: bool = False, out=None, scale=None):
    """Per-64-position FP8 e4m3fn quantization of x [B,N,H,d] (fp32 or bf16,
    on a GPU) with power-of-two scales.  Returns (codes uint8 [B,N,H,d],
    scale fp32 [B,H,ceil(N/64)])."""
    return _quantize("attn_quantize_fp8_block64", x, hadamard, out, scale, lambda B, N, H: (B, H, (N + 63) // 64))


def flash_attn_func(q, k, v, dropout_p=0.0, softmax_scale=None, causal=True, return_lse=False, fp8=False,
                    hadamard=False, fp8_scales="head", p_block_scale=False):
    """Drop-in for the ``flash_attn_func`` call convention: q [B,Nq,Hq,d_qk],
    k [B,Nk,Hkv,d_qk], v [B,Nk,Hkv,d_v] BF16 GPU tensors (BSHD), causal, with
    Nq <= Nk (the queries are the last Nq positions; Nq == Nk is a plain
    prefill).  ``fp8=True`` quantizes q, k, v to e4m3 with the library's
    quantizer -- one scale per (batch, head) (``fp8_scales="head"``) or one
    power-of-two scale per 64 positions (``fp8_scales="block64"``);
    ``hadamard=True`` rotates q and k first -- and runs the FP8 path;
    ``p_block_scale=True`` (with ``fp8_scales="block64"``) also scales the
    probabilities per block by powers of two.  Returns
    the bf16 output, or ``(out, lse)`` with ``return_lse`` (lse fp32
    [B,Hq,Nq], natural log).  Only what the kernels compute is accepted:
    causal=False and dropout raise."""
    torch = _torch()
    if not causal:
        raise NotImplementedError("only causal attention is implemented")
    if dropout_p:
        raise NotImplementedError("dropout is not implemented (forward inference only)")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{name} must be bfloat16 (fp8=True quantizes it)")
    if hadamard and not fp8:
        raise ValueError("hadamard applies to the FP8 path only")
    if fp8_scales not in ("head", "block64"):
        raise ValueError('fp8_scales must be "head" or "block64"')
    if p_block_scale and not (fp8 and fp8_scales == "block64"):
        raise ValueError('p_block_scale needs fp8=True and fp8_scales="block64"')
    p_mode = DEFAULT_P_MODE
    if fp8 and fp8_scales == "block64":
        (cq, sq) = attn_quantize_fp8_block64(q.contiguous(), hadamard=hadamard)
        (ck, sk) = attn_quantize_fp8_block64(k.contiguous(), hadamard=hadamard)
        (cv, sv) = attn_quantize_fp8_block64(v.contiguous())
        args = (cq, ck, cv, sq, sk, sv)
        p_mode = "lean_block" if p_block_scale else "lean"  # as attn_fwd_block64
    elif fp8:
        (cq, sq) = attn_quantize_fp8(q.contiguous(), hadamard=hadamard)
        (ck, sk) = attn_quantize_fp8(k.contiguous(), hadamard=hadamard)
        (cv, sv) = attn_quantize_fp8(v.contiguous())
        args = (cq, ck, cv, sq, sk, sv)
    else:
        args = (q.contiguous(), k.contiguous(), v.contiguous())
    out, lse = attn_fwd_ws(*args, with_lse=return_lse, softmax_scale=softmax_scale,
                           scales=fp8_scales if fp8 else "head", p_mode=p_mode)
    return (out, lse) if return_lse else out
