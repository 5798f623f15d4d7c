"""The C ABI on the CPU: the library loads, exports every entry point that
include/miattn.h declares, and rejects invalid arguments before touching the
device (no compute call is made here)."""

import ctypes
import os
import re
import subprocess

import pytest

import bf16_causal_prefill_flashattention_amd as pkg

pytestmark = pytest.mark.cpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "miattn.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", src, flags=re.M)


def header_constant(name):
    m = re.search(rf"#define\s+{name}\s+\(?(-?\d+)\)?", open(HEADER).read())
    return int(m.group(1))


@pytest.fixture(scope="module")
def lib():
    return pkg.load_library()


def test_header_declares_the_entry_points():
    assert sorted(declared_functions()) == sorted(
        ["attn_fwd", "attn_fwd_chunk", "attn_fwd_block64", "attn_fwd_fp8", "attn_fwd_noalloc", "attn_fwd_ws",
         "attn_fwd_ws_size",
         "attn_quantize_fp8", "attn_quantize_fp8_block64", "attn_status_string", "attn_version"])


def test_probability_mode_constants_match_the_binding():
    for name, code in pkg.P_MODES.items():
        assert header_constant(f"MIATTN_P_{name.upper()}") == code
    assert header_constant("MIATTN_SCALES_HEAD") == 0 and header_constant("MIATTN_SCALES_BLOCK64") == 1
    m = re.search(r"#define\s+MIATTN_P_DEFAULT\s+MIATTN_P_(\w+)", open(HEADER).read())
    assert m.group(1).lower() == pkg.DEFAULT_P_MODE


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", pkg.library_path()], capture_output=True, text=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    for fn in declared_functions():
        assert fn in exported, fn
        assert hasattr(lib, fn)


def test_version_and_status_strings(lib):
    assert pkg.attn_version() == header_constant("MIATTN_ABI_VERSION")
    for code in range(-8, 1):
        s = pkg.attn_status_string(code)
        assert s and s != "unknown status code"
    assert pkg.attn_status_string(-99) == "unknown status code"


OK = 0
E_NULL, E_SIZE, E_SHAPE, E_DTYPE, E_HIP, E_ALIGN, E_VALUE = -1, -2, -3, -4, -5, -6, -7
P = 1 << 20  # a 16-byte-aligned stand-in address; never dereferenced on these paths


def fwd(lib, q=P, k=P, v=P, o=P, B=1, Hq=2, Hkv=2, N=8, dqk=128, dv=128, dtype=0, qs=P, ks=P, vs=P):
    return lib.attn_fwd(q, k, v, o, B, Hq, Hkv, N, dqk, dv, dtype, qs, ks, vs, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), E_NULL), (dict(k=None), E_NULL), (dict(v=None), E_NULL), (dict(o=None), E_NULL),
    (dict(dtype=1, qs=None), E_NULL), (dict(dtype=1, vs=None), E_NULL),
    (dict(B=-1), E_SIZE), (dict(N=-5), E_SIZE), (dict(Hq=0), E_SIZE), (dict(Hkv=0), E_SIZE),
    (dict(Hq=6, Hkv=4), E_SIZE),
    (dict(dqk=64, dv=64), E_SHAPE), (dict(dqk=128, dv=192), E_SHAPE), (dict(dqk=256, dv=128), E_SHAPE),
    (dict(dtype=2), E_DTYPE), (dict(dtype=-1), E_DTYPE),
    (dict(q=P + 8), E_ALIGN), (dict(o=P + 2), E_ALIGN), (dict(dtype=1, ks=P + 2), E_ALIGN),
    (dict(N=0), OK), (dict(B=0), OK), (dict(N=0, q=None, k=None, v=None, o=None), OK),
])
def test_attn_fwd_validation(lib, kw, expect):
    assert fwd(lib, **kw) == expect


def chunk(lib, q=P, k=P, v=P, o=P, lse=P, B=1, Hq=2, Hkv=2, Nq=8, Nk=20, dqk=128, dv=128, dtype=0, qs=P, ks=P,
          vs=P, tau=0.0):
    return lib.attn_fwd_chunk(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, dqk, dv, dtype, qs, ks, vs, tau, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), E_NULL), (dict(o=None), E_NULL), (dict(dtype=1, ks=None), E_NULL),
    (dict(Nq=21), E_SIZE), (dict(Nq=-1), E_SIZE), (dict(Nk=-3, Nq=0), E_SIZE), (dict(Hq=3, Hkv=2), E_SIZE),
    (dict(dqk=64), E_SHAPE), (dict(dtype=3), E_DTYPE),
    (dict(lse=P + 2), E_ALIGN), (dict(v=P + 4), E_ALIGN),
    (dict(tau=-0.5), E_VALUE), (dict(tau=float("inf")), E_VALUE), (dict(tau=float("nan")), E_VALUE),
    (dict(Nq=0), OK), (dict(B=0), OK), (dict(Nq=0, Nk=0), OK), (dict(Nq=0, q=None, k=None, v=None, o=None), OK),
])
def test_attn_fwd_chunk_validation(lib, kw, expect):
    assert chunk(lib, **kw) == expect


def quant(lib, x=P, src=0, y=P, s=P, B=1, H=2, N=8, d=128, had=0):
    return lib.attn_quantize_fp8(x, src, y, s, B, H, N, d, had, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(x=None), E_NULL), (dict(y=None), E_NULL), (dict(s=None), E_NULL),
    (dict(src=2), E_DTYPE), (dict(had=2), E_DTYPE),
    (dict(B=-1), E_SIZE), (dict(H=0), E_SIZE), (dict(N=-1), E_SIZE),
    (dict(d=64), E_SHAPE), (dict(d=256, had=1), E_SHAPE),
    (dict(x=P + 4), E_ALIGN), (dict(s=P + 1), E_ALIGN),
    (dict(B=0), OK),
])
def test_quantize_validation(lib, kw, expect):
    assert quant(lib, **kw) == expect
    # the per-64-position quantizer validates the same way
    assert lib.attn_quantize_fp8_block64(*[kw.get(n, dv) for n, dv in (
        ("x", P), ("src", 0), ("y", P), ("s", P), ("B", 1), ("H", 2), ("N", 8), ("d", 128), ("had", 0))],
        None) == expect


def test_quantize_block64_empty_sequence(lib):
    assert lib.attn_quantize_fp8_block64(P, 0, P, P, 1, 2, 0, 128, 0, None) == OK


def block64(lib, q=P, k=P, v=P, o=P, lse=P, B=1, Hq=2, Hkv=2, Nq=8, Nk=20, dqk=128, dv=128, qs=P, ks=P, vs=P,
            tau=0.0, pbs=0):
    return lib.attn_fwd_block64(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, dqk, dv, qs, ks, vs, tau, pbs, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), E_NULL), (dict(o=None), E_NULL), (dict(qs=None), E_NULL), (dict(ks=None), E_NULL),
    (dict(vs=None), E_NULL),
    (dict(Nq=21), E_SIZE), (dict(Nq=-1), E_SIZE), (dict(Hq=3, Hkv=2), E_SIZE),
    (dict(Nq=8, Nk=(1 << 20) + 1), E_SIZE),
    (dict(dqk=64), E_SHAPE), (dict(dqk=192, dv=192), E_SHAPE),
    (dict(lse=P + 2), E_ALIGN), (dict(ks=P + 2), E_ALIGN), (dict(k=P + 4), E_ALIGN),
    (dict(tau=-0.5), E_VALUE), (dict(tau=float("nan")), E_VALUE), (dict(pbs=2), E_DTYPE), (dict(pbs=-1), E_DTYPE),
    (dict(Nq=0), OK), (dict(B=0), OK), (dict(Nq=0, q=None, k=None, v=None, o=None), OK),
    (dict(Nq=0, pbs=1), OK),
])
def test_attn_fwd_block64_validation(lib, kw, expect):
    assert block64(lib, **kw) == expect


def fp8(lib, q=P, k=P, v=P, o=P, lse=P, B=1, Hq=2, Hkv=2, Nq=8, Nk=20, dqk=128, dv=128, qs=P, ks=P, vs=P,
        tau=0.0, scales=0, pmode=0):
    return lib.attn_fwd_fp8(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, dqk, dv, qs, ks, vs, tau, scales, pmode, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), E_NULL), (dict(o=None), E_NULL), (dict(qs=None), E_NULL), (dict(vs=None), E_NULL),
    (dict(Nq=21), E_SIZE), (dict(Hq=3, Hkv=2), E_SIZE),
    (dict(Nq=8, Nk=(1 << 20) + 1, scales=1), E_SIZE),
    (dict(dqk=64), E_SHAPE),
    (dict(lse=P + 2), E_ALIGN), (dict(ks=P + 2), E_ALIGN),
    (dict(tau=-1.0), E_VALUE),
    (dict(scales=2), E_DTYPE), (dict(scales=-1), E_DTYPE), (dict(pmode=6), E_DTYPE), (dict(pmode=-1), E_DTYPE),
    (dict(Nq=0), OK), (dict(B=0), OK), (dict(Nq=0, pmode=3, scales=1), OK),
    (dict(Nq=0, q=None, k=None, v=None, o=None), OK),
])
def test_attn_fwd_fp8_validation(lib, kw, expect):
    assert fp8(lib, **kw) == expect


def ws(lib, q=P, k=P, v=P, o=P, lse=P, B=1, Hq=2, Hkv=2, Nq=8, Nk=20, dqk=128, dv=128, dtype=1, qs=P, ks=P, vs=P,
       tau=0.0, scales=0, pmode=4, w=P, wb=1 << 20):
    return lib.attn_fwd_ws(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, dqk, dv, dtype, qs, ks, vs, tau, scales, pmode, w, wb,
                           None)


# (the workspace checks themselves need the device's compute-unit count: GPU tests)
@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), E_NULL), (dict(o=None), E_NULL), (dict(qs=None), E_NULL), (dict(dtype=0, v=None), E_NULL),
    (dict(Nq=21), E_SIZE), (dict(Hq=3, Hkv=2), E_SIZE), (dict(B=-1), E_SIZE),
    (dict(Nq=8, Nk=(1 << 20) + 1, scales=1), E_SIZE),
    (dict(dqk=64), E_SHAPE), (dict(dv=192), E_SHAPE),
    (dict(lse=P + 2), E_ALIGN), (dict(k=P + 4), E_ALIGN),
    (dict(tau=-1.0), E_VALUE), (dict(tau=float("nan")), E_VALUE),
    (dict(scales=2), E_DTYPE), (dict(pmode=6), E_DTYPE), (dict(dtype=2), E_DTYPE), (dict(dtype=0, pmode=7), E_DTYPE),
    (dict(Nq=0), OK), (dict(B=0), OK), (dict(Nq=0, w=None, wb=0), OK),
    (dict(Nq=0, q=None, k=None, v=None, o=None, w=None), OK),
])
def test_attn_fwd_ws_validation(lib, kw, expect):
    assert ws(lib, **kw) == expect


@pytest.mark.parametrize("args,expect", [
    ((1, 2, 2, 8, 20, 128, 128, 2, 0, 4), E_DTYPE), ((1, 2, 2, 8, 20, 128, 128, 1, 2, 4), E_DTYPE),
    ((1, 2, 2, 8, 20, 128, 128, 1, 0, 6), E_DTYPE), ((1, 3, 2, 8, 20, 128, 128, 1, 0, 4), E_SIZE),
    ((1, 2, 2, 21, 20, 128, 128, 1, 0, 4), E_SIZE), ((1, 2, 2, 8, 20, 64, 128, 1, 0, 4), E_SHAPE),
    ((0, 2, 2, 8, 20, 128, 128, 1, 0, 4), OK), ((1, 2, 2, 0, 20, 128, 128, 0, 0, 4), OK),
])
def test_attn_fwd_ws_size_validation(lib, args, expect):
    n = ctypes.c_size_t(123)
    assert lib.attn_fwd_ws_size(*args, ctypes.byref(n)) == expect
    assert n.value == 0
    assert lib.attn_fwd_ws_size(*args, None) == E_NULL


def test_binding_refuses_cpu_tensors():
    import torch

    q = torch.zeros(1, 4, 1, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        pkg.attn_fwd(q, q, q)
    with pytest.raises(ValueError):
        pkg.attn_fwd_chunk(q, q, q)
    with pytest.raises(ValueError):
        pkg.attn_quantize_fp8(q.float())
    with pytest.raises(ValueError):
        pkg.attn_quantize_fp8_block64(q.float())
    c = torch.zeros(1, 4, 1, 128, dtype=torch.uint8)
    s = torch.ones(1, 1, 1)
    with pytest.raises(ValueError):
        pkg.attn_fwd_block64(c, c, c, s, s, s)
    with pytest.raises(TypeError):
        pkg.attn_fwd_block64(q, q, q, s, s, s)
    with pytest.raises(ValueError):
        pkg.attn_fwd_fp8(c, c, c, s, s, s, p_mode="fast")
    with pytest.raises(ValueError):
        pkg.attn_fwd_fp8(c, c, c, s, s, s, scales="tensor")
    with pytest.raises(ValueError):
        pkg.attn_fwd_fp8(c, c, c, s, s, s)
    with pytest.raises(ValueError):
        pkg.attn_fwd_ws(q, q, q)
    with pytest.raises(ValueError):
        pkg.attn_fwd_ws(c, c, c, s, s, s, p_mode="fast")


def test_flash_attn_func_refuses_what_the_kernels_do_not_compute():
    import torch

    q = torch.zeros(1, 4, 1, 128, dtype=torch.bfloat16)
    with pytest.raises(NotImplementedError):
        pkg.flash_attn_func(q, q, q, causal=False)
    with pytest.raises(NotImplementedError):
        pkg.flash_attn_func(q, q, q, dropout_p=0.1)
    with pytest.raises(TypeError):
        pkg.flash_attn_func(q.float(), q.float(), q.float())
    with pytest.raises(ValueError):
        pkg.flash_attn_func(q, q, q, hadamard=True)
    with pytest.raises(ValueError):
        pkg.flash_attn_func(q, q, q, fp8=True, fp8_scales="tensor")
    with pytest.raises(ValueError):
        pkg.flash_attn_func(q, q, q, fp8=True, p_block_scale=True)
    with pytest.raises(ValueError):  # CPU tensors
        pkg.flash_attn_func(q, q, q)


def test_probe_library_exports_its_entry_points():
    """The LDS counter probe (bench.py --lds-probe) is built beside the library."""
    from bf16_causal_prefill_flashattention_amd import build as B

    out = subprocess.run(["nm", "-D", "--defined-only", B.PROBE_LIB], capture_output=True, text=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert {"lds_probe_run", "lds_probe_threads"} <= exported
    lib = ctypes.CDLL(B.PROBE_LIB)
    assert lib.lds_probe_threads() == 256
    assert lib.lds_probe_run(0, 4, 0, 16, None, None) == -1  # rejected before any launch


def test_gpu_tests_mirror_the_launch_rules():
    """The GPU tests that pick shapes by the library's launch rules (the tile
    size of short launches, the 4-wave mode's key limit) restate those rules;
    they must match the constants the library is built with."""
    src = open(os.path.join(ROOT, "bf16_causal_prefill_flashattention_amd", "csrc", "kernels.h")).read()

    def constant(name):
        return int(re.search(rf"constexpr int {name} = (\d+);", src).group(1))

    tests = os.path.dirname(os.path.abspath(__file__))
    split = open(os.path.join(tests, "test_gpu_split.py")).read()
    solo = open(os.path.join(tests, "test_gpu_solo.py")).read()
    assert int(re.search(r"^SHORT_KEYS = (\d+)", split, re.M).group(1)) == constant("kShortKeys")
    assert int(re.search(r"^SOLO_MAX_KEYS = (\d+)", solo, re.M).group(1)) == constant("kSoloMaxKeys")
    assert constant("kSoloQueryTile") == 128 and constant("kQueryTile") == 256
