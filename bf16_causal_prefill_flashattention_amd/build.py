"""Build libmiattn.so (the gfx950 HIP kernels plus the C ABI) in-tree with hipcc.

Usage: python -m bf16_causal_prefill_flashattention_amd.build [-v]
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmiattn.so")
PROBE_LIB = os.path.join(PKG, "libmiattn_probe.so")
ATTN_FP8 = [f"attn_fwd_fp8_{s}_d{d}.hip" for s in ("head", "block64") for d in (128, 192)]
SOURCES = ATTN_FP8 + ["attn_fwd_bf16.hip", "attn_fwd.hip", "attn_fwd_noalloc.hip", "quantize_fp8.hip",
                      "miattn_api.cpp"]
# measurement aids of bench.py --lds-probe and --mfma-probe (LDS reads of known bank behaviour,
# back-to-back MFMAs), in a library of their own
PROBE_SOURCES = ["lds_probe.hip", "mfma_probe.hip"]
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-command-line-argument",
    # no packed fp32 math: hipcc would otherwise emit v_pk_{add,mul,fma}_f32
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmiattn.so)")


# Per-source flags.  The attention kernel never sees NaN inputs (scores are
# finite or -inf), so fmax needs no NaN quieting.  The quantizer keeps strict
# IEEE and forms no FMA from a separate multiply and add, so its codes stay
# bit-identical to a step-by-step fp32 evaluation.
EXTRA_FLAGS = {src: ["-fno-honor-nans"] for src in ATTN_FP8 + ["attn_fwd_bf16.hip"]}
EXTRA_FLAGS["quantize_fp8.hip"] = ["-ffp-contract=off"]


def _compile(src: str, obj: str, verbose: bool) -> None:
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc(), *COMMON_FLAGS, *EXTRA_FLAGS.get(src, []), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{r.stdout}\n{r.stderr}")
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if ln.strip() and noise not in ln]
    if msgs and verbose:
        print("\n".join(msgs), flush=True)


def _link(objs, lib: str, tmp: str, verbose: bool) -> None:
    out_tmp = os.path.join(tmp, os.path.basename(lib))
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out_tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking {os.path.basename(lib)} failed:\n{r.stdout}\n{r.stderr}")
    shutil.copyfile(out_tmp, lib + ".tmp")
    os.replace(lib + ".tmp", lib)


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link libmiattn.so (and the LDS
    counter probe, libmiattn_probe.so) next to this file.  Always recompiles.
    Returns the path of libmiattn.so."""
    with tempfile.TemporaryDirectory(prefix="miattn_build_") as tmp:
        srcs = SOURCES + PROBE_SOURCES
        objs = [os.path.join(tmp, s + ".o") for s in srcs]
        with cf.ThreadPoolExecutor(max_workers=len(srcs)) as ex:
            list(ex.map(lambda so: _compile(so[0], so[1], verbose), zip(srcs, objs)))
        _link(objs[:len(SOURCES)], LIB, tmp, verbose)
        _link(objs[len(SOURCES):], PROBE_LIB, tmp, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv[1:]))
