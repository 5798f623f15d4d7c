"""Benchmark: causal attention forward throughput on one MI355X.

Prints ONE JSON line.  The headline workload is FP8 e4m3 causal attention at
head dim 128 and N = 32768 (B = 1, Hq = Hkv = 32).  One step is one causal
attention launch on one batch of synthetic input already resident in HBM in
the kernel's input format: e4m3 codes plus per-head fp32 scales for FP8, BF16
for BF16.  ``value`` = causal FLOPs / step time, with causal FLOPs =
B * Hq * N^2 * (d_qk + d_v), the attention kernel alone as the metric defines
it.  The FP8 front end (per-head amax/448 quantization of the BF16 activations
Q, K, V) produces those resident inputs before the timed region and is timed
on its own under ``front_end``.  The BF16 point of the same metric (BF16,
d = 128, N = 32K) is reported in the same line under ``bf16``, and one chunk
of a chunked prefill (the last 8192 positions of the same 32K FP8 sequence
against all 32768 keys, with the LSE output) under ``chunk``, its FLOPs
counted the same way: B * Hq * (2 Nq Nk - Nq^2) * (d_qk + d_v).  The same FP8
workload quantized with one power-of-two scale per 64 positions instead of
one per head (``attn_fwd_block64``) is reported under ``block64``, and with
the probabilities scaled per block as well under ``block64.p_block_scale``.

``roofline`` describes the attention kernel (the dominant one): its algorithmic
FLOPs per launch divided by its average launch duration, measured with HIP
events on the launch stream inside the timed region, against the dense MFMA
peak of its dtype.  Before the counted warmup launches, each leg runs at least
``--prewarm`` seconds (default 1.5) of back-to-back launches so that the clock
has settled when the timed region starts.  ``sclk_mhz`` is the graphics clock
sampled (amdsmi, every 10 ms) during the timed region, ``sclk_prewarm_mhz`` the
same over the second half of the pre-warm, and ``frac_at_sclk`` the fraction of
the peak scaled from its 2.4 GHz to the timed region's clock (the random
operand data holds the clock below 2.4 GHz).  ``launch_ms_median`` and
``launch_ms_min`` come from a second pass of as many launches with an event
between consecutive ones.  ``determinism``: after each leg's timed launches,
``--determinism`` (default 100) more launches on the same inputs, each compared
bit for bit with the output (and, for the chunk, the LSE) of the timed ones.

``cpu_baseline`` times the CPU oracle (test infrastructure, untuned) on a
bounded sample of the same workload: whole heads, every row, one head per
worker process of a pool as large as the host cores this process may use (at
most 16); ``cores`` is that worker count.  The same oracle outputs are compared
with the output of the timed launches, and ``parity`` reports the relative
Frobenius error over the compared heads (and per head), the gate of the
workload's dtype (BF16 1e-2, FP8 6e-2 against the oracle on the dequantized
inputs), and whether the GPU quantizer's codes and scales of those heads equal
the oracle quantizer's.  The BF16 leg gets its own ``parity`` the same way.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--prewarm SECONDS] [--no-bf16] [--no-cpu-baseline]
                       [--no-chunk] [--no-block64] [--determinism N] [--p-mode MODE]
       python bench.py --clock-study [--study-seconds S]

``--clock-study`` measures how the input data and the FP8 probability mode
move the sustained clock and the energy per FLOP: for several input
distributions of the 32K workloads (and, on the Gaussian FP8 inputs, every
probability mode: lean or exact, with no shift, a shift per 128-key tile or
per 64-key step) it runs back-to-back launches for a few seconds while
sampling the graphics clock and reading the board's energy counter (amdsmi),
and prints one JSON line per case (time, TFLOP/s, mean SCLK, mean power,
TFLOP/J).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "causal attn fwd TFLOP/s (FP8 & BF16, d=128, N=32K) + % of MFMA peak"
PEAK_TFLOPS = {"fp8": 5000.0, "bf16": 2500.0}  # MI355X dense MFMA, published
PAGES_FP8_HD128_32K = 2672.0  # TFLOP/s, FP8 causal fwd, hd128, N=32K, Gaussian, on MI355X (the pages' figure)
# the kernel template, its helpers, the tile-size rules and the launch logic that picks the variant and grid
ATTN_KERNEL_SOURCES = ["attn_fwd_impl.hpp", "device_common.hpp", "kernels.h", "attn_fwd.hip"]


def code_tokens(text: str) -> str:
    """Source text without // comments and with whitespace collapsed: what the
    compiler sees, so editing a comment does not invalidate a profile."""
    import re

    return " ".join(re.sub(r"//[^\n]*", " ", text).split())


def kernel_source_hash(read=None) -> str:
    """Hash of the attention kernel's code (comments and layout excluded)."""
    h = hashlib.sha256()
    for s in ATTN_KERNEL_SOURCES:
        path = os.path.join(ROOT, "bf16_causal_prefill_flashattention_amd", "csrc", s)
        text = read(s) if read else open(path, encoding="utf-8").read()
        h.update(code_tokens(text).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, launches_bytes: float):
    """HBM bytes per launch of the attention kernel from the committed
    rocprofv3 counter summary, if it was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"attn_fwd_traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


_AMDSMI = []  # [handle] once amdsmi is initialised, [None] if unavailable


def amdsmi_handle():
    """The first GPU's amdsmi handle (initialised once), or None."""
    if not _AMDSMI:
        try:
            import amdsmi

            amdsmi.amdsmi_init()
            _AMDSMI.append(amdsmi.amdsmi_get_processor_handles()[0])
        except Exception:
            _AMDSMI.append(None)
    return _AMDSMI[0]


class ClockSampler:
    """Samples the graphics clock (amdsmi's current-clock reading, MHz) every
    10 ms on a thread while it runs; no-op where amdsmi is unavailable."""

    def __init__(self):
        self.handle = amdsmi_handle()
        self.samples = []  # (perf_counter seconds, MHz)
        self._stop = None
        self._th = None

    def __enter__(self):
        import threading

        if self.handle is None:
            return self
        import amdsmi

        self._stop = threading.Event()

        def sample():
            while not self._stop.wait(0.01):
                try:
                    mhz = amdsmi.amdsmi_get_clock_info(self.handle, amdsmi.AmdSmiClkType.GFX)["clk"]
                    self.samples.append((time.perf_counter(), mhz))
                except Exception:
                    pass

        self._th = threading.Thread(target=sample, daemon=True)
        self._th.start()
        return self

    def __exit__(self, *exc):
        if self._th is not None:
            self._stop.set()
            self._th.join()

    def mean(self, t0: float, t1: float):
        c = [m for t, m in self.samples if t0 <= t <= t1]
        return (round(sum(c) / len(c), 1), len(c)) if c else (None, 0)


def timed_launches(step, steps: int, warmup: int, prewarm_s: float, stream):
    """Pre-warm (back-to-back launches for at least prewarm_s seconds), then
    `warmup` untimed launches, then `steps` timed ones bracketed by device
    synchronisation and by one pair of HIP events recorded on `stream`, the
    stream the kernels are launched on (events around every launch would let
    the host's enqueue time into short launches' figures).  The clock is
    sampled throughout.  A second pass of `steps` launches, with an event
    recorded between consecutive ones, gives the median and the minimum per
    launch (reported beside the mean of the timed region, not in its place).
    Returns (wall ms per step, [event ms per step], clock dict with the median
    and minimum)."""
    import torch

    with ClockSampler() as clk:
        torch.cuda.synchronize()
        tp0 = time.perf_counter()
        while time.perf_counter() - tp0 < prewarm_s:
            for _ in range(8):
                step()
            torch.cuda.synchronize()
        tp1 = time.perf_counter()
        for _ in range(warmup):
            step()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(steps):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        evs[0].record(stream)
        for i in range(steps):
            step()
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
    per = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(steps))
    median = per[steps // 2] if steps % 2 else (per[steps // 2 - 1] + per[steps // 2]) / 2
    sclk, n = clk.mean(t0, t1)
    sclk_pre, npre = clk.mean((tp0 + tp1) / 2, tp1)
    clock = {"sclk_mhz": sclk, "sclk_samples": n, "sclk_prewarm_mhz": sclk_pre, "prewarm_s": round(tp1 - tp0, 2),
             "launch_ms_median": round(median, 4), "launch_ms_min": round(per[0], 4)}
    return (t1 - t0) * 1e3 / steps, [e0.elapsed_time(e1) / steps], clock


def determinism_pass(step, outs, launches: int):
    """`launches` more calls of `step` on the same inputs after the timed ones;
    each must reproduce the tensors in `outs` (as the timed launches left them)
    bit for bit, compared as raw integers (so -0 against +0 or a NaN payload
    would count as a difference).  None when launches is 0."""
    import torch

    if launches <= 0:
        return None
    ints = {1: torch.uint8, 2: torch.int16, 4: torch.int32}
    refs = [t.view(ints[t.element_size()]).clone() for t in outs]
    equal = 0
    for _ in range(launches):
        step()
        equal += all(torch.equal(t.view(ints[t.element_size()]), r) for t, r in zip(outs, refs))
    return {"launches": launches, "bitwise_equal": int(equal), "pass": equal == launches,
            "reference": "the output of the timed launches"}


def run_gpu(w, steps: int, warmup: int, prewarm_s: float, determinism: int = 0, p_mode=None):
    """Time `steps` attention launches of workload w on inputs resident in HBM.
    Returns a dict: wall ms per step, per-launch event ms, front-end ms (FP8),
    clock readings, and on the host the output of the timed launches, the BF16
    activations and (FP8) the codes and scales, for the parity check."""
    import torch

    import bf16_causal_prefill_flashattention_amd as miattn
    from bf16_causal_prefill_flashattention_amd.inputs import make_qkv

    dev = torch.device("cuda:0")
    hq, hk, hv = (t.to(torch.bfloat16) for t in make_qkv(w))  # BF16 activations
    q, k, v = (t.to(dev) for t in (hq, hk, hv))
    fp8 = w.dtype == "fp8"
    block64 = fp8 and w.scales == "block64"
    out = torch.empty((w.B, w.N, w.Hq, w.d_v), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)  # every kernel below is enqueued on this stream
    front_ms = None
    codes = None
    if fp8:
        cq = torch.empty(q.shape, dtype=torch.uint8, device=dev)
        ck = torch.empty(k.shape, dtype=torch.uint8, device=dev)
        cv = torch.empty(v.shape, dtype=torch.uint8, device=dev)
        nb = ((w.N + 63) // 64,) if block64 else ()
        sq = torch.empty((w.B, w.Hq) + nb, dtype=torch.float32, device=dev)
        sk = torch.empty((w.B, w.Hkv) + nb, dtype=torch.float32, device=dev)
        sv = torch.empty((w.B, w.Hkv) + nb, dtype=torch.float32, device=dev)
        quantize = miattn.attn_quantize_fp8_block64 if block64 else miattn.attn_quantize_fp8

        def front_end():
            quantize(q, hadamard=w.hadamard, out=cq, scale=sq)
            quantize(k, hadamard=w.hadamard, out=ck, scale=sk)
            quantize(v, hadamard=False, out=cv, scale=sv)

        # the FP8 front end, timed on its own (it also leaves the resident inputs)
        fe = []
        for i in range(6):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            front_end()
            e1.record(stream)
            torch.cuda.synchronize()
            if i >= 1:
                fe.append(e0.elapsed_time(e1))
        front_ms = sorted(fe)[len(fe) // 2]
        args = (cq, ck, cv, sq, sk, sv)
        if not block64:
            codes = tuple(t.cpu() for t in args)
    else:
        args = (q, k, v)

    # one call of the library's attention entry point with a workspace (launches
    # that leave compute units idle split their keys), checked and marshalled
    # once; the workspace is allocated here, outside the timed launches
    scales = "block64" if block64 else "head"
    p_mode = ("lean_block" if w.p_block_scale else "lean") if block64 else (p_mode or miattn.DEFAULT_P_MODE)
    step, _, _ = miattn.attn_fwd_ws_bind(*args, out=out, with_lse=False, scales=scales, p_mode=p_mode)

    ms, attn_ms, clock = timed_launches(step, steps, warmup, prewarm_s, stream)
    det = determinism_pass(step, [out], determinism)
    return {"ms": ms, "attn_ms": attn_ms, "front_ms": front_ms, "clock": clock, "determinism": det,
            "out": out.cpu(), "inputs": (hq, hk, hv), "codes": codes}


def parity_tasks(w, res, heads):
    """Oracle tasks for whole heads of workload w (B = 1): the BF16 activations
    the timed launches read (FP8: the activations the front end quantized, with
    its codes and scales), and the output of the timed launches."""
    import numpy as np

    q, k, v = res["inputs"]
    out, codes = res["out"], res["codes"]
    grp = w.Hq // w.Hkv
    f32 = lambda t: np.ascontiguousarray(t.float().numpy())  # noqa: E731
    tasks = []
    for h in heads:
        g = h // grp
        t = {"key": h, "q": f32(q[0, :, h]), "k": f32(k[0, :, g]), "v": f32(v[0, :, g]), "out": f32(out[0, :, h]),
             "fp8": {"hadamard": w.hadamard} if w.dtype == "fp8" else None}
        if codes is not None:
            cq, ck, cv, sq, sk, sv = codes
            t["codes"] = (cq[0, :, h].numpy(), ck[0, :, g].numpy(), cv[0, :, g].numpy(),
                          float(sq[0, h]), float(sk[0, g]), float(sv[0, g]))
        tasks.append(t)
    return tasks


def oracle_heads(pool, w, res):
    """Run the oracle on one wave of whole heads (as many as the pool has
    workers, spread over the heads) and compare them with the timed launches'
    output.  Returns (parity dict, heads, wall seconds)."""
    import numpy as np

    from oracle.pool import summarize

    n = min(w.Hq, pool.workers)
    heads = sorted({int(h) for h in np.linspace(0, w.Hq - 1, n).round()})
    tasks = parity_tasks(w, res, heads)
    t0 = time.perf_counter()
    results = pool.run(tasks)
    el = time.perf_counter() - t0
    s = summarize(results)
    tol = 6e-2 if w.dtype == "fp8" else 1e-2
    parity = {"rel_fro": float(f"{s['rel_fro']:.4e}"), "per_head_max": float(f"{s['per_head_max']:.4e}"),
              "tolerance": tol, "pass": bool(s["rel_fro"] <= tol and s["per_head_max"] <= tol),
              "heads": heads, "rows": "all", "codes_equal": s["codes_equal"],
              "reference": "fp64 oracle on the dequantized inputs" if w.dtype == "fp8" else
              "fp64 oracle on the BF16 inputs"}
    return parity, heads, el


def cpu_baseline(pool, w, res):
    """The oracle (as it stands) on a bounded sample of the workload: one wave
    of whole heads, every row, one head per worker process.  FP8: oracle
    quantization of the head's Q, K, V plus exact attention on the dequantized
    values; BF16: exact attention on the BF16 values.  Also returns the parity
    of those heads against the timed launches' output."""
    parity, heads, el = oracle_heads(pool, w, res)
    flops = float(w.B) * len(heads) * float(w.N) ** 2 * (w.d_qk + w.d_v)
    base = {
        "value": round(flops / el / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": int(pool.workers),
        "kind": "oracle",
        "sample": f"{len(heads)} of {w.Hq} query heads (all {w.N} rows each) of {w.name}, "
                  f"{'quantize + ' if w.dtype == 'fp8' else ''}fp64 attention, one head per worker process "
                  f"({pool.workers} workers, one BLAS thread each), {el:.1f} s",
        "seconds": round(el, 2),
    }
    return base, parity


def chunk_flops(B, Hq, Nq, Nk, d_qk, d_v) -> float:
    """Causal FLOPs of a chunk, in the convention of B * Hq * N^2 * (d_qk + d_v)
    (which is the Nq == Nk case): 2 * (visible query-key pairs) * (d_qk + d_v)
    with the pairs counted as Nq * Nk - Nq^2 / 2."""
    return float(B) * Hq * (2.0 * Nq * Nk - float(Nq) ** 2) * (d_qk + d_v)


def run_chunk(w, Nq: int, steps: int, warmup: int, prewarm_s: float, determinism: int = 0, p_mode=None):
    """Time attn_fwd_chunk (with LSE) for the last Nq positions of workload w's
    FP8 sequence; inputs quantized by the library and resident in HBM.
    Returns (wall ms per step, per-launch event ms, clock dict, determinism
    record of output and LSE)."""
    import torch

    import bf16_causal_prefill_flashattention_amd as miattn
    from bf16_causal_prefill_flashattention_amd.inputs import make_qkv

    dev = torch.device("cuda:0")
    q, k, v = make_qkv(w)
    q = q[:, w.N - Nq:].contiguous()
    q, k, v = (t.to(torch.bfloat16).to(dev) for t in (q, k, v))
    (cq, sq), (ck, sk), (cv, sv) = (miattn.attn_quantize_fp8(t) for t in (q, k, v))
    del q, k, v
    out = torch.empty((w.B, Nq, w.Hq, w.d_v), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.Hq, Nq), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        if p_mode is None:  # the library's default probability mode
            miattn.attn_fwd_chunk(cq, ck, cv, sq, sk, sv, out=out, lse=lse)
        else:
            miattn.attn_fwd_fp8(cq, ck, cv, sq, sk, sv, out=out, lse=lse, p_mode=p_mode)

    ms, attn_ms, clock = timed_launches(step, steps, warmup, prewarm_s, stream)
    return ms, attn_ms, clock, determinism_pass(step, [out, lse], determinism)


PEAK_SCLK_MHZ = 2400.0  # the engine clock the published MFMA peaks are quoted at


def roofline(w, attn_ms, flops=None, clock=None):
    flops = w.causal_flops if flops is None else flops
    avg_s = sum(attn_ms) / len(attn_ms) * 1e-3
    achieved = flops / avg_s / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    return {
        "kernel": f"attn_fwd_{w.dtype}{'_block64' if w.scales == 'block64' else ''}"
                  f"{'_pscale' if w.p_block_scale else ''}_kernel<{w.d_qk},{w.d_v}>",
        "bound": "mfma",
        "achieved": round(achieved, 1),
        "peak": peak,
        "unit": "TFLOP/s",
        "frac": round(achieved / peak, 4),
        "traffic": measured_traffic(w.name, None),
        "avg_launch_ms": round(avg_s * 1e3, 4),
        "flops_per_launch": flops,
        # graphics clock during the timed region (after the pre-warm), and the
        # fraction of the peak scaled to that clock (the MFMA work per cycle is fixed)
        **(clock or {}),
        "frac_at_sclk": None if not (clock or {}).get("sclk_mhz") else
        round(achieved / (peak * clock["sclk_mhz"] / PEAK_SCLK_MHZ), 4),
    }


# (instruction form, byte stride between lanes, expected bank behaviour) of the probe kernels
LDS_PROBES = [
    (0, 4, "ds_read_b32, consecutive words: conflict-free"),
    (0, 8, "ds_read_b32, every other word: 2-way conflict"),
    (0, 256, "ds_read_b32, all lanes in bank 0"),
    (1, 16, "ds_read_b128, consecutive 16-byte chunks: conflict-free"),
    (1, 256, "ds_read_b128, every chunk starting at bank 0"),
    (2, 8, "ds_read_b64_tr_b8, consecutive 8-byte pieces"),
    (2, 256, "ds_read_b64_tr_b8, every piece at bank 0"),
]


def lds_probe(blocks: int = 256, iters: int = 4096):
    """Run every LDS probe kernel once (one workgroup per CU); one JSON line."""
    import ctypes

    import torch

    from bf16_causal_prefill_flashattention_amd import build as B

    if not torch.cuda.is_available():
        print("bench.py --lds-probe needs a GPU", file=sys.stderr)
        return 1
    lib = ctypes.CDLL(B.PROBE_LIB)
    lib.lds_probe_run.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                  ctypes.c_void_p]
    lib.lds_probe_run.restype = ctypes.c_int
    out = torch.zeros(blocks * lib.lds_probe_threads(), dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    runs = []
    for kind, stride, what in LDS_PROBES:
        st = lib.lds_probe_run(kind, stride, blocks, iters, ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(stream))
        torch.cuda.synchronize()
        if st != 0:
            print(f"lds_probe_run({kind}, {stride}) failed: {st}", file=sys.stderr)
            return 1
        runs.append({"kernel": f"lds_probe_kernel<{kind}, {stride}>", "pattern": what,
                     "lds_instructions": blocks * (lib.lds_probe_threads() // 64) * iters})
    print(json.dumps({"lds_probe": runs, "blocks": blocks, "iters_per_wave": iters}), flush=True)
    return 0


def amdsmi_gpu0():
    """(amdsmi module, handle of the first GPU), or (None, None) when unavailable."""
    try:
        import amdsmi

        amdsmi.amdsmi_init()
        return amdsmi, amdsmi.amdsmi_get_processor_handles()[0]
    except Exception as e:  # the readings are optional; timing still runs
        print(f"amdsmi unavailable ({e}); clock and power are not reported", file=sys.stderr)
        return None, None


def sustained(launch, seconds: float, smi, flops: float):
    """Back-to-back launches for about `seconds` (after 20 untimed ones), timed
    with one event pair, with the GFX clock and the board energy counter
    sampled every 50 ms.  Returns a dict: launches, ms per launch, TFLOP/s
    (flops per launch), and with amdsmi the mean clock of the second half of
    the samples, board watts and TFLOP/J."""
    import threading

    import torch

    amdsmi, handle = smi

    def energy_j():
        r = amdsmi.amdsmi_get_energy_count(handle)
        return r["energy_accumulator"] * r["counter_resolution"] * 1e-6

    for _ in range(20):
        launch()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    launch()
    e1.record()
    torch.cuda.synchronize()
    n = max(10, int(seconds * 1e3 / e0.elapsed_time(e1)))
    clocks, energy, stop = [], [], threading.Event()

    def sample():
        while not stop.wait(0.05):
            try:
                clocks.append(amdsmi.amdsmi_get_clock_info(handle, amdsmi.AmdSmiClkType.GFX)["clk"])
                energy.append((time.perf_counter(), energy_j()))
            except Exception:
                pass

    th = None
    if handle is not None:
        th = threading.Thread(target=sample, daemon=True)
        ej0, t0 = energy_j(), time.perf_counter()
        th.start()
    e0.record()
    for _ in range(n):
        launch()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    rec = {"launches": n, "ms_per_launch": round(ms, 4), "tflops": round(flops / (ms * 1e-3) / 1e12, 1)}
    if th is not None:
        t1, ej1 = time.perf_counter(), energy_j()
        stop.set()
        th.join()
        # The energy counter advances in coarse steps (about once a second on
        # MI355X boards): the rate between its first and last change inside
        # the window is the board power; the clock reading lags the load, so
        # only its second half is kept.
        watts = (ej1 - ej0) / (t1 - t0)
        steps = [energy[i] for i in range(1, len(energy)) if energy[i][1] != energy[i - 1][1]]
        rec["energy_steps"] = len(steps)
        if len(steps) >= 2 and steps[-1][0] > steps[0][0]:
            watts = (steps[-1][1] - steps[0][1]) / (steps[-1][0] - steps[0][0])
        clocks = clocks[len(clocks) // 2:]
        rec["sclk_mhz_mean"] = round(sum(clocks) / len(clocks), 1) if clocks else None
        rec["sclk_samples"] = len(clocks)
        rec["board_watts_mean"] = round(watts, 1)
        rec["tflop_per_joule"] = round(rec["tflops"] / watts, 3) if watts > 0 else None
    return rec


def mfma_probe(seconds: float):
    """Back-to-back MFMAs on operands with the attention inputs' values (Gaussian
    BF16; e4m3 codes of Gaussian data at a per-head scale; or, as in a P.V
    product, probabilities in [0, 1) against Gaussian values), sustained for
    about `seconds`: the matrix-core throughput, clock and board power the
    power limit allows on such data, the ceiling of an attention kernel on it.
    One JSON line per (dtype, operands)."""
    import ctypes

    import torch

    from bf16_causal_prefill_flashattention_amd import build as B

    if not torch.cuda.is_available():
        print("bench.py --mfma-probe needs a GPU", file=sys.stderr)
        return 1
    smi = amdsmi_gpu0()
    lib = ctypes.CDLL(B.PROBE_LIB)
    lib.mfma_probe_run.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_void_p]
    dev = torch.device("cuda:0")
    blocks = torch.cuda.get_device_properties(0).multi_processor_count  # one workgroup (8 waves) per CU
    threads = lib.mfma_probe_threads()
    g = torch.Generator(device="cpu")
    g.manual_seed(7)
    for fp8, iters in ((False, 16384), (True, 8192)):
        words = lib.mfma_probe_words(1 if fp8 else 0)  # A sets, then B sets, per thread
        per = words // 2 * (4 if fp8 else 2)  # values of A (and of B) per thread
        for label in ("gaussian", "probabilities_x_gaussian"):
            b_vals = torch.randn(blocks * threads, per, generator=g)
            if label == "gaussian":
                a_vals = torch.randn(blocks * threads, per, generator=g)
            else:  # A in [0, 1): a P.V product's probabilities (x 2^6 before e4m3 rounding in the FP8 kernel)
                a_vals = torch.rand(blocks * threads, per, generator=g) * (64.0 if fp8 else 1.0)
            if fp8:  # e4m3 codes at a per-head scale of Gaussian data (amax about 4.5 sigma -> 448)
                if label == "gaussian":
                    a_vals = a_vals * (448.0 / 4.5)
                b_vals = b_vals * (448.0 / 4.5)
                enc = lambda t: t.clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)  # noqa: E731
            else:
                enc = lambda t: t.to(torch.bfloat16)  # noqa: E731
            ops = torch.cat([enc(a_vals), enc(b_vals)], dim=1).contiguous().view(torch.int32).reshape(-1).to(dev)
            assert ops.numel() == blocks * threads * words
            out = torch.empty(blocks * threads, dtype=torch.float32, device=dev)
            stream = torch.cuda.current_stream().cuda_stream

            def launch():
                st = lib.mfma_probe_run(1 if fp8 else 0, blocks, iters, ctypes.c_void_p(ops.data_ptr()),
                                        ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(stream))
                if st != 0:
                    raise RuntimeError(f"mfma_probe_run failed: {st}")

            flops = blocks * (threads // 64) * 4 * iters * (32 * 32 * (64 if fp8 else 16) * 2)
            rec = {"study": "mfma_probe", "dtype": "fp8_e4m3" if fp8 else "bf16", "operands": label,
                   "mfma": "32x32x64 f8f6f4" if fp8 else "32x32x16 bf16", "peak_tflops": PEAK_TFLOPS["fp8" if fp8 else "bf16"]}
            rec.update(sustained(launch, seconds, smi, flops))
            rec["frac_of_peak"] = round(rec["tflops"] / rec["peak_tflops"], 4)
            print(json.dumps(rec), flush=True)
    return 0


def clock_study(seconds: float):
    """One JSON line per (dtype, input distribution): the data-dependent clock
    and energy of the attention kernel on the 32K workloads."""
    import torch

    import bf16_causal_prefill_flashattention_amd as miattn
    from bf16_causal_prefill_flashattention_amd.inputs import WORKLOADS, make_qkv

    handle = amdsmi_gpu0()
    dev = torch.device("cuda:0")
    cases = [
        ("gaussian", lambda q, k, v: (q, k, v)),
        ("outlier_channels", None),  # 4 aligned channels x20 on Q and K
        ("peaked_q_x4", lambda q, k, v: (q * 4, k, v)),  # near one-hot rows
        ("flat_q_zero", lambda q, k, v: (torch.zeros_like(q), k, v)),  # all probabilities equal
        ("zero_v", lambda q, k, v: (q, k, torch.zeros_like(v))),
    ]
    default_mode = miattn.DEFAULT_P_MODE
    # FP8 probability modes on the Gaussian inputs: lean or exact, no shift,
    # a shift per 128-key tile, or a shift per 64-key step
    fp8_modes = [default_mode] + [m for m in sorted(miattn.P_MODES) if m != default_mode]
    for wname in ("fp8_mha_n32k", "bf16_mha_n32k"):
        base = WORKLOADS[wname]
        for cname, fn in cases:
            w = base.with_(outliers=4) if fn is None else base
            q, k, v = make_qkv(w)
            if fn is not None:
                q, k, v = fn(q, k, v)
            q, k, v = (t.to(torch.bfloat16).to(dev) for t in (q, k, v))
            out = torch.empty((w.B, w.N, w.Hq, w.d_v), dtype=torch.bfloat16, device=dev)
            if w.dtype == "fp8":
                (cq, sq), (ck, sk), (cv, sv) = (miattn.attn_quantize_fp8(t) for t in (q, k, v))
                modes = fp8_modes if cname == "gaussian" else [default_mode]
            else:
                modes = [None]
            for mode in modes:
                if mode is None:
                    launch = lambda: miattn.attn_fwd(q, k, v, out=out)  # noqa: E731
                else:
                    launch = (lambda m: lambda: miattn.attn_fwd_fp8(cq, ck, cv, sq, sk, sv, out=out,  # noqa: E731
                                                                      with_lse=False, p_mode=m))(mode)
                rec = {"study": "clock_energy", "workload": wname, "inputs": cname, "p_mode": mode or "bf16"}
                rec.update(sustained(launch, seconds, handle, w.causal_flops))
                print(json.dumps(rec), flush=True)
            del out, q, k, v
            if w.dtype == "fp8":
                del cq, ck, cv, sq, sk, sv
            torch.cuda.empty_cache()
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--prewarm", type=float, default=1.5,
                    help="seconds of back-to-back launches before the counted warmup of every leg")
    ap.add_argument("--workload", default="fp8_mha_n32k")
    ap.add_argument("--bf16-workload", default="bf16_mha_n32k")
    ap.add_argument("--no-bf16", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-chunk", action="store_true")
    ap.add_argument("--no-block64", action="store_true")
    ap.add_argument("--clock-study", action="store_true")
    ap.add_argument("--mfma-probe", action="store_true",
                    help="sustain back-to-back MFMAs on attention-like operands (libmiattn_probe.so) for "
                         "--study-seconds: the throughput the board power limit allows on such data")
    ap.add_argument("--lds-probe", action="store_true",
                    help="run the LDS read patterns of known bank behaviour (libmiattn_probe.so) once each, "
                         "for reading the LDS bank-conflict counter against them under rocprofv3 --pmc")
    ap.add_argument("--study-seconds", type=float, default=3.0)
    ap.add_argument("--chunk-queries", type=int, default=8192)
    ap.add_argument("--p-mode", default=None,
                    help="FP8 probability mode of the per-head FP8 leg and the chunk (lean, lean_block, lean_tile, "
                         "exact, exact_block, exact_tile; default: the library's default)")
    ap.add_argument("--determinism", type=int, default=100,
                    help="after each leg's timed launches, this many more launches on the same inputs, each "
                         "checked bit for bit against the timed launches' output (0: none)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="before the warmup, run one plain elementwise copy (torch.neg) that reads and writes "
                         "this many bytes: the reference kernel of known traffic for scaling HBM counters")
    args = ap.parse_args(argv)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the path is a single-GPU kernel and the library has no "
              "multi-GPU mode (--gpus must be 1)", file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0 or args.determinism < 0:
        print("--steps must be at least 1, --warmup and --determinism at least 0", file=sys.stderr)
        return 2
    if args.p_mode is not None:
        from bf16_causal_prefill_flashattention_amd import P_MODES

        if args.p_mode not in P_MODES:
            print(f"--p-mode must be one of {sorted(P_MODES)}", file=sys.stderr)
            return 2
    if args.clock_study:
        return clock_study(args.study_seconds)
    if args.lds_probe:
        return lds_probe()
    if args.mfma_probe:
        return mfma_probe(args.study_seconds)

    from bf16_causal_prefill_flashattention_amd.inputs import WORKLOADS

    w = WORKLOADS[args.workload]
    pool = None
    if not args.no_cpu_baseline:
        # the oracle's worker processes start before this process touches the GPU
        from oracle.pool import HeadPool

        pool = HeadPool()
    try:
        return bench(args, w, WORKLOADS, pool)
    finally:
        if pool is not None:
            pool.close()


def bench(args, w, WORKLOADS, pool):
    import torch

    from bf16_causal_prefill_flashattention_amd import DEFAULT_P_MODE

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    amdsmi_handle()  # initialised before any launch
    if args.copy_bytes > 0:
        src = torch.ones(args.copy_bytes // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    res = run_gpu(w, args.steps, args.warmup, args.prewarm, args.determinism, args.p_mode)
    ms = res["ms"]
    value = w.causal_flops / (ms * 1e-3) / 1e12
    rec = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(value / PAGES_FP8_HD128_32K, 4) if w.name == "fp8_mha_n32k" else None,
        "dtype": "fp8_e4m3" if w.dtype == "fp8" else "bf16",
        "data": "synthetic (seeded Gaussian N(0,1) activations; FP8 codes and scales from the library's own "
                "quantizer, resident in HBM)" if w.dtype == "fp8" else "synthetic (seeded Gaussian N(0,1), BF16 in HBM)",
        "config": {
            "workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "N": w.N, "d_qk": w.d_qk, "d_v": w.d_v,
            "outlier_channels": w.outliers, "hadamard": w.hadamard,
            **({"p_mode": args.p_mode or DEFAULT_P_MODE} if w.dtype == "fp8" and w.scales == "head" else {}),
            "step": "one attn_fwd_ws call: one attention launch (launches that split their keys add a merge kernel)",
        },
        "roofline": roofline(w, res["attn_ms"], clock=res["clock"]),
        "determinism": res["determinism"],
    }
    if res["front_ms"] is not None:
        rec["front_end"] = {"what": "quantize Q, K, V (bf16 -> e4m3, per-head amax/448), timed apart from the metric",
                            "ms": round(res["front_ms"], 4)}
    if pool is not None:
        rec["cpu_baseline"], rec["parity"] = cpu_baseline(pool, w, res)
    del res
    if not args.no_bf16 and w.dtype == "fp8":
        wb = WORKLOADS[args.bf16_workload]
        rb = run_gpu(wb, args.steps, args.warmup, args.prewarm, args.determinism)
        rec["bf16"] = {
            "workload": wb.name,
            "value": round(wb.causal_flops / (rb["ms"] * 1e-3) / 1e12, 1),
            "ms_per_step": round(rb["ms"], 4),
            "roofline": roofline(wb, rb["attn_ms"], clock=rb["clock"]),
            "determinism": rb["determinism"],
        }
        if pool is not None:
            rec["bf16"]["parity"] = oracle_heads(pool, wb, rb)[0]
        del rb
    if not args.no_block64 and w.name == "fp8_mha_n32k":
        wq = WORKLOADS["fp8_mha_n32k_block64"]
        rq = run_gpu(wq, args.steps, args.warmup, args.prewarm, args.determinism)
        rec["block64"] = {
            "workload": f"{wq.name}: the same inputs with one power-of-two scale per 64 positions "
                        "(K and V scales applied by the scaled MFMAs)",
            "value": round(wq.causal_flops / (rq["ms"] * 1e-3) / 1e12, 1),
            "ms_per_step": round(rq["ms"], 4),
            "front_end_ms": round(rq["front_ms"], 4),
            "roofline": roofline(wq, rq["attn_ms"], clock=rq["clock"]),
            "determinism": rq["determinism"],
        }
        del rq
        wp = WORKLOADS["fp8_mha_n32k_block64_pscale"]
        rp = run_gpu(wp, args.steps, args.warmup, args.prewarm, args.determinism)
        rec["block64"]["p_block_scale"] = {
            "workload": f"{wp.name}: probabilities also scaled per block by powers of two",
            "value": round(wp.causal_flops / (rp["ms"] * 1e-3) / 1e12, 1),
            "ms_per_step": round(rp["ms"], 4),
            "roofline": roofline(wp, rp["attn_ms"], clock=rp["clock"]),
            "determinism": rp["determinism"],
        }
        del rp
    if not args.no_chunk and w.dtype == "fp8" and 0 < args.chunk_queries <= w.N:
        Nq = args.chunk_queries
        msc, attn_c, clock_c, det_c = run_chunk(w, Nq, args.steps, args.warmup, args.prewarm, args.determinism,
                                                args.p_mode)
        fl = chunk_flops(w.B, w.Hq, Nq, w.N, w.d_qk, w.d_v)
        rec["chunk"] = {
            "workload": f"{w.name} chunk: last {Nq} positions against {w.N} keys, LSE written",
            "Nq": Nq, "Nk": w.N,
            "value": round(fl / (msc * 1e-3) / 1e12, 1),
            "ms_per_step": round(msc, 4),
            "roofline": roofline(w, attn_c, fl, clock=clock_c),
            "determinism": det_c,
        }
        rec["chunk"]["roofline"]["traffic"] = None
    rec["kernel_source_hash"] = kernel_source_hash()
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
