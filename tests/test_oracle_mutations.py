"""Plant plausible mistakes in a copy of the oracle's source (CPU only) and
check that the pins reject each one.  The shipped oracle is never modified:
each mutant is the module text with one substitution, executed in a fresh
namespace."""

import importlib.util
import math
import os
import types

import numpy as np
import pytest
import torch
import torch.nn.functional as F

pytestmark = pytest.mark.cpu
ORACLE = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle")


def _load_mutant(fname, old, new, extra=None):
    src = open(os.path.join(ORACLE, fname)).read()
    assert old in src, f"mutation anchor not found: {old!r}"
    src = src.replace(old, new, 1)
    mod = types.ModuleType("mutant")
    mod.__dict__["__name__"] = "mutant"
    if extra:
        mod.__dict__.update(extra)
    exec(compile(src.replace("from .", "from oracle."), fname, "exec"), mod.__dict__)
    return mod


def _sdpa_ok(attn):
    g = np.random.default_rng(0)
    q = g.standard_normal((1, 40, 4, 32))
    k = g.standard_normal((1, 40, 2, 32))
    v = g.standard_normal((1, 40, 2, 16))
    ref = F.scaled_dot_product_attention(
        *(torch.from_numpy(t).permute(0, 2, 1, 3) for t in (q, k, v)), is_causal=True, enable_gqa=True
    ).permute(0, 2, 1, 3).numpy()
    return np.allclose(attn(q, k, v), ref, rtol=1e-10, atol=1e-12)


def _row0_ok(attn):
    g = np.random.default_rng(1)
    q, k, v = (g.standard_normal((1, 8, 1, 8)) for _ in range(3))
    return np.array_equal(attn(q, k, v)[0, 0, 0], v[0, 0, 0])


ATTN_MUTANTS = [
    ("tau = (1.0 / math.sqrt(dqk))", "tau = (1.0 / dqk)"),  # wrong softmax scale
    ("<= r[:, None]", "< r[:, None] + (r[:, None] == 0)"),  # strict mask except row 0
    ("g = h // group", "g = h % Hkv"),  # interleaved GQA mapping
    ("e.sum(axis=1, keepdims=True)", "e.sum(axis=0, keepdims=True)"),  # softmax over queries
    ("q[b, r, h, :] @ kh[:hi].T", "q[b, r, h, :] @ np.flip(kh[:hi], 0).T"),  # misaligned keys
]


@pytest.mark.parametrize("old,new", ATTN_MUTANTS)
def test_attention_mutants_are_caught(old, new):
    m = _load_mutant("attention.py", old, new)
    assert not (_sdpa_ok(m.attn_ref) and _row0_ok(m.attn_ref))


def test_unmutated_copy_passes():
    m = _load_mutant("attention.py", "import math", "import math")
    assert _sdpa_ok(m.attn_ref) and _row0_ok(m.attn_ref)


E4M3_MUTANTS = [
    ("(d_hi == d_lo) & (hi % 2 == 0)", "(d_hi == d_lo)"),  # ties away from zero
    ("np.ldexp(m.astype(np.float64) / 8.0, -6)", "np.ldexp(m.astype(np.float64) / 8.0, -7)"),  # subnormal exponent
    ("(e - 7)", "(e - 8)"),  # wrong bias
]


@pytest.mark.parametrize("old,new", E4M3_MUTANTS)
def test_e4m3_mutants_are_caught(old, new):
    m = _load_mutant("e4m3.py", old, new)
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    dec_ok = np.array_equal(m.e4m3_decode(codes), ref, equal_nan=True)
    vals = ref[:0x7F]
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    enc_ok = np.array_equal(m.e4m3_encode_rne_sat(mids),
                            torch.from_numpy(mids).to(torch.float8_e4m3fn).view(torch.uint8).numpy())
    assert not (dec_ok and enc_ok)


def test_hadamard_mutant_is_caught():
    import scipy.linalg

    m = _load_mutant("hadamard.py", "blocks[:, :, 1, :] = a - b", "blocks[:, :, 1, :] = b - a")
    x = np.random.default_rng(2).integers(-9, 9, size=(4, 128)).astype(np.float32)
    assert not np.array_equal(m.fwht128_f32(x).astype(np.int64), x.astype(np.int64) @ scipy.linalg.hadamard(128))


def test_quantize_mutant_is_caught():
    m = _load_mutant("quantize.py", "inv = np.float32(f448 / amax)", "inv = np.float32(f448 / amax / 2)")
    x = np.random.default_rng(3).standard_normal((1, 50, 1, 128)).astype(np.float32)
    codes, _ = m.quantize_ref(x)
    assert not np.any((codes & 0x7F) == 0x7E)  # the amax element no longer maps to 448


BLOCK64_MUTANTS = [
    ("y = (xs * np.float32(math.ldexp(1.0, -e)))", "y = (xs * np.float32(math.ldexp(1.0, e)))"),  # inverse scale
    ("math.frexp(float(amax))[1] - 9", "math.frexp(float(amax))[1] - 8"),  # exponent one too large
    ("* hadamard_norm_f32(d)).astype", ").astype"),  # normalisation dropped
    ("scales[b, h, j] = np.float32(math.ldexp(1.0, e))", "scales[b, h, j] = np.float32(math.ldexp(1.0, e - 1))"),
]


@pytest.mark.parametrize("old,new", BLOCK64_MUTANTS)
def test_block64_mutants_are_caught(old, new):
    from oracle.hadamard import hadamard_rotate_f32

    m = _load_mutant("quantize.py", old, new)
    g = np.random.default_rng(5)
    x = (g.standard_normal((1, 130, 1, 128)) * 10.0 ** g.uniform(-2, 2)).astype(np.float32)
    x[0, :64] *= np.float32(3.7)
    ok = True
    for had in (False, True):
        codes, scales = m.quantize_block64_ref(x, had)
        ref = hadamard_rotate_f32(x).astype(np.float64) * 2.0 ** -3.5 if had else x.astype(np.float64)
        deq = m.dequantize_block64_ref(codes, scales)
        ok &= bool(np.linalg.norm(deq - ref) / np.linalg.norm(ref) < 0.04)
        for j in range(3):
            amax = np.abs(ref[0, 64 * j:64 * (j + 1)]).max()
            ok &= bool(224 < amax / float(scales[0, 0, j]) <= 448 * (1 + 1e-6))
    assert not ok


WEIGHT_MUTANTS = [
    ("s = tau * (q[b, :, h, :] @ k[b, :, g, :].T)", "s = (q[b, :, h, :] @ k[b, :, g, :].T)"),  # tau dropped
    ("s = tau * (q[b, :, h, :] @ k[b, :, g, :].T)", "s = tau * tau * (q[b, :, h, :] @ k[b, :, g, :].T)"),  # tau twice
    ("np.tril(np.ones((N, N), dtype=bool))", "np.tril(np.ones((N, N), dtype=bool), 1)"),  # one key past the diagonal
    ("g = h // (Hq // Hkv)\n    N = q.shape[1]", "g = h % Hkv\n    N = q.shape[1]"),  # interleaved GQA mapping
]


def _weights_ok(weights):
    """The two-key logistic closed form and W @ V = attn_ref (the pins of the
    weight matrix in test_oracle_attention.py)."""
    from oracle import attn_ref

    g = np.random.default_rng(7)
    q, k = g.standard_normal((1, 2, 1, 64)), g.standard_normal((1, 2, 1, 64))
    gap = float(q[0, 1, 0] @ k[0, 1, 0] - q[0, 1, 0] @ k[0, 0, 0])
    ok = abs(weights(q, k)[1, 1] - 1.0 / (1.0 + math.exp(-gap / 8.0))) <= 1e-15
    q, k, v = g.standard_normal((1, 30, 4, 32)), g.standard_normal((1, 30, 2, 32)), g.standard_normal((1, 30, 2, 8))
    out = attn_ref(q, k, v)
    for h in range(4):
        w = weights(q, k, 0, h)
        ok &= bool(np.allclose(w @ v[0, :, h // 2, :], out[0, :, h, :], rtol=1e-12, atol=1e-13))
    return ok


@pytest.mark.parametrize("old,new", WEIGHT_MUTANTS)
def test_weight_mutants_are_caught(old, new):
    m = _load_mutant("attention.py", old, new)
    assert not _weights_ok(m.causal_weights_ref)


def test_unmutated_weights_pass():
    m = _load_mutant("attention.py", "import math", "import math")
    assert _weights_ok(m.causal_weights_ref)
