"""Whole-head oracle runs in a process pool -- test infrastructure only.

The attention of one (batch, query head) depends on nothing but that head's
queries and its key/value head, so heads are independent units of work.  This
module runs the oracle of ``attention.py`` (and, for FP8, the quantizer of
``quantize.py``) on whole heads, one head per worker process, and compares each
with a given output of the same head.  Each head is computed by exactly the
functions the single-process tests pin; the pool only runs several of them at
once.

Workers are started with the ``spawn`` method (a fresh interpreter: nothing
from the parent's runtime state is inherited) and run their linear algebra on
one thread each, so the pool uses as many cores as it has workers.
"""

from __future__ import annotations

import os
import time

import numpy as np

from .attention import attn_ref
from .quantize import dequantize_ref, quantize_ref

MAX_WORKERS = 16


def host_cores() -> int:
    """Cores this process may run on, capped at MAX_WORKERS."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(n, MAX_WORKERS))


def _one_thread():
    try:
        from threadpoolctl import threadpool_limits

        threadpool_limits(1)
    except Exception:
        pass


def head_parity(task: dict) -> dict:
    """Oracle output of one head and its distance to a given output.

    task keys:
      q [N, d_qk], k [N, d_qk], v [N, d_v]: the head's inputs as real numbers
        (BF16 path: the BF16 values themselves; FP8 path: the activations the
        quantizer reads);
      out [N, d_v]: the output to compare (e.g. a GPU result upcast exactly);
      fp8: None for the BF16 path, else {"hadamard": bool} -- the inputs are
        then quantized per head with ``quantize_ref`` and attention runs on the
        dequantized values;
      codes (optional, FP8): (cq, ck, cv, sq, sk, sv) codes [N, d] uint8 and
        fp32 scalar scales of another quantizer, compared bit for bit;
      key (optional): returned unchanged, to identify the head.

    Returns sums of squares of the difference and of the oracle output (their
    ratio's square root is the head's relative Frobenius error), the largest
    absolute difference, whether the given codes matched, and the seconds
    spent in the oracle.
    """
    _one_thread()
    t0 = time.perf_counter()
    q, k, v = (np.asarray(task[n])[None, :, None, :] for n in ("q", "k", "v"))
    codes_equal = None
    fp8 = task.get("fp8")
    if fp8 is not None:
        had = bool(fp8.get("hadamard", False))
        (cq, sq), (ck, sk), (cv, sv) = quantize_ref(q, had), quantize_ref(k, had), quantize_ref(v, False)
        given = task.get("codes")
        if given is not None:
            gq, gk, gv, gsq, gsk, gsv = given
            codes_equal = bool(
                np.array_equal(cq[0, :, 0], gq) and np.array_equal(ck[0, :, 0], gk)
                and np.array_equal(cv[0, :, 0], gv)
                and np.float32(gsq).view(np.uint32) == sq.reshape(-1)[0].view(np.uint32)
                and np.float32(gsk).view(np.uint32) == sk.reshape(-1)[0].view(np.uint32)
                and np.float32(gsv).view(np.uint32) == sv.reshape(-1)[0].view(np.uint32))
        q, k, v = dequantize_ref(cq, sq), dequantize_ref(ck, sk), dequantize_ref(cv, sv)
    ref = attn_ref(q, k, v)[0, :, 0, :]
    seconds = time.perf_counter() - t0
    d = np.asarray(task["out"], dtype=np.float64) - ref
    return {
        "key": task.get("key"),
        "sq_err": float(np.sum(d * d)),
        "sq_ref": float(np.sum(ref * ref)),
        "max_abs": float(np.max(np.abs(d))) if d.size else 0.0,
        "rows": int(ref.shape[0]),
        "codes_equal": codes_equal,
        "seconds": seconds,
    }


class HeadPool:
    """A pool of oracle workers (spawned processes, one BLAS thread each)."""

    def __init__(self, workers: int | None = None):
        import concurrent.futures as cf
        import multiprocessing as mp

        self.workers = workers or host_cores()
        keep = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
        try:
            for k in keep:  # inherited by the workers before their numpy loads
                os.environ[k] = "1"
            self._ex = cf.ProcessPoolExecutor(self.workers, mp_context=mp.get_context("spawn"))
            # start every worker now (each imports numpy and this package once)
            list(self._ex.map(_noop, range(self.workers)))
        finally:
            for k, val in keep.items():
                if val is None:
                    os.environ.pop(k, None)
                else:
                    os.environ[k] = val

    def run(self, tasks):
        """head_parity over the tasks, in order."""
        return list(self._ex.map(head_parity, tasks))

    def close(self):
        self._ex.shutdown(wait=True)

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


def _noop(i):
    return i


def summarize(results) -> dict:
    """Relative Frobenius error over all heads together and per head."""
    num = sum(r["sq_err"] for r in results)
    den = sum(r["sq_ref"] for r in results)
    per = [float(np.sqrt(r["sq_err"] / r["sq_ref"])) if r["sq_ref"] > 0 else 0.0 for r in results]
    return {
        "rel_fro": float(np.sqrt(num / den)) if den > 0 else 0.0,
        "per_head_max": max(per) if per else 0.0,
        "per_head": per,
        "max_abs": max((r["max_abs"] for r in results), default=0.0),
        "codes_equal": all(r["codes_equal"] for r in results) if results and results[0]["codes_equal"] is not None
        else None,
    }
