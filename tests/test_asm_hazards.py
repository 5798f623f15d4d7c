"""Wait states around the attention kernels' inline-assembly tile loads (CPU).

The K/V tile loads are LDS-writing buffer loads written as inline assembly.
The compiler does not insert the wait states the gfx9 family needs in front of
inline assembly, so the kernel source provides them itself.  This test
compiles every attention translation unit for gfx950 (device code only, with
the library's own flags) and checks the generated code of each kernel variant
along every control-flow path into each such load:

* no VALU instruction (``v_readfirstlane_b32`` and the like) writes an SGPR of
  the load's buffer descriptor within the 5 wait states before it;
* no SALU instruction writes M0 (the load's LDS address) within the 1 wait
  state before it.

An ``s_nop N`` counts N + 1 wait states, any other instruction 1.

A second check reads the same code for spill traffic (scratch accesses, SGPR
spill lanes) inside each kernel's main loop, where a reload would wait for
every tile load in flight.
"""

import concurrent.futures as cf
import os
import re
import subprocess
import tempfile

import pytest

from bf16_causal_prefill_flashattention_amd import build as B

pytestmark = pytest.mark.cpu
ATTN_SOURCES = B.ATTN_FP8 + ["attn_fwd_bf16.hip"]  # the translation units that instantiate the kernel
VALU_SGPR_STATES = 5
M0_STATES = 1


def _compile_asm(src: str, out: str) -> str:
    cmd = [B.hipcc(), *B.COMMON_FLAGS, *B.EXTRA_FLAGS.get(src, []), "-x", "hip", "--cuda-device-only", "-S",
           os.path.join(B.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return open(out).read()


@pytest.fixture(scope="module")
def asm_texts():
    with tempfile.TemporaryDirectory(prefix="miattn_asm_") as tmp:
        with cf.ThreadPoolExecutor(max_workers=min(8, len(ATTN_SOURCES))) as ex:
            futs = {s: ex.submit(_compile_asm, s, os.path.join(tmp, s + ".s")) for s in ATTN_SOURCES}
            return {s: f.result() for s, f in futs.items()}


def _sgprs(operand: str):
    m = re.fullmatch(r"s(\d+)", operand)
    if m:
        return {int(m.group(1))}
    m = re.fullmatch(r"s\[(\d+):(\d+)\]", operand)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    return set()


def _functions(text: str):
    """(name, [lines]) of every kernel body: instructions and labels."""
    funcs = []
    for m in re.finditer(r"^(_Z\w*attn_fwd_kernel\w*):.*?$(.*?)^\s*s_endpgm", text, re.S | re.M):
        lines = []
        for raw in m.group(2).splitlines():
            ln = raw.split(";")[0].strip()
            if not ln or ln.startswith("."):
                if re.match(r"^\.LBB\w+:", raw.strip()):
                    lines.append(raw.strip().rstrip(":").split(":")[0] + ":")
                continue
            lines.append(ln)
        funcs.append((m.group(1), lines))
    return funcs


def _wait_states(ins: str) -> int:
    m = re.match(r"s_nop\s+(\d+)", ins)
    return int(m.group(1)) + 1 if m else 1


def _predecessors(lines):
    """index of each label line -> indices of the instructions that can run just
    before it (the fall-through line and every branch to it)."""
    labels = {ln[:-1]: i for i, ln in enumerate(lines) if ln.endswith(":")}
    preds = {i: [] for i in labels.values()}
    for i, ln in enumerate(lines):
        m = re.match(r"s_(c?branch\w*)\s+(\.LBB\w+)", ln)
        if m and m.group(2) in labels:
            preds[labels[m.group(2)]].append(i)
    for i in preds:
        j = i - 1
        if j >= 0 and not re.match(r"s_branch\s", lines[j]) and not lines[j].startswith("s_setpc"):
            preds[i].append(j)
    return preds


def _violations(lines, load_idx, regs, states, writes):
    """Paths backwards from the load on which an instruction matching
    writes(ins, regs) lies within `states` wait states."""
    preds = _predecessors(lines)
    bad, stack, seen = [], [(load_idx - 1, 0)], set()
    while stack:
        i, used = stack.pop()
        if i < 0 or used >= states or (i, used) in seen:
            continue
        seen.add((i, used))
        ln = lines[i]
        if ln.endswith(":"):
            for p in preds.get(i, []):
                stack.append((p, used))
            continue
        if writes(ln, regs):
            bad.append((i, ln, used))
            continue
        stack.append((i - 1, used + _wait_states(ln)))
    return bad


def _valu_writes_sgpr(ins, regs):
    if not ins.startswith("v_"):
        return False
    ops = [o.strip() for o in ins.split(None, 1)[1].split(",")] if " " in ins else []
    return any(_sgprs(o) & regs for o in ops[:2])  # destination, or a VOP3 carry-out


def _salu_writes_m0(ins, regs):
    if not ins.startswith("s_"):
        return False
    ops = ins.split(None, 1)[1].split(",") if " " in ins else []
    return bool(ops) and ops[0].strip() == "m0"


def test_inline_lds_loads_have_their_wait_states(asm_texts):
    checked = 0
    for src, text in asm_texts.items():
        funcs = _functions(text)
        assert funcs, f"no attention kernel found in {src}"
        for name, lines in funcs:
            loads = [i for i, ln in enumerate(lines) if re.match(r"buffer_load_dwordx4\s.*\blds\b", ln)]
            assert loads, f"{name}: no LDS-writing loads found"
            for i in loads:
                rsrc = _sgprs(lines[i].split(",")[1].strip())
                assert rsrc, lines[i]
                bad = _violations(lines, i, rsrc, VALU_SGPR_STATES, _valu_writes_sgpr)
                assert not bad, f"{src} {name}: VALU writes a descriptor SGPR of '{lines[i]}' too close: {bad[:3]}"
                bad = _violations(lines, i, None, M0_STATES, _salu_writes_m0)
                assert not bad, f"{src} {name}: M0 written directly before '{lines[i]}': {bad[:3]}"
                checked += 1
    assert checked > 100


def _loop_blocks(text: str):
    """name -> [(loop header of the block or None, [instructions])] for every
    kernel, from the compiler's loop annotations of the block labels."""
    kernels = {}
    for m in re.finditer(r"^(_Z\w*attn_fwd_kernel\w*):.*?$(.*?)^\s*s_endpgm", text, re.S | re.M):
        blocks, header, ins = [], None, []
        raw_lines = m.group(2).splitlines()
        for k, raw in enumerate(raw_lines):
            s = raw.strip()
            lab = re.match(r"^(\.LBB(\w+)|; %bb\.\d+):", s)
            if lab:
                blocks.append((header, ins))
                ins = []
                comment = s + (" " + raw_lines[k + 1].strip() if k + 1 < len(raw_lines) else "")
                h = re.search(r"in Loop: Header=BB(\w+)", comment)
                if h:
                    header = h.group(1)
                elif "Inner Loop Header" in comment and lab.group(2):
                    header = lab.group(2)
                else:
                    header = None
                continue
            ln = raw.split(";")[0].strip()
            if ln and not ln.startswith("."):
                ins.append(ln)
        blocks.append((header, ins))
        kernels[m.group(1)] = blocks
    return kernels


def test_main_loops_hold_no_spill_traffic(asm_texts):
    """No scratch access and no SGPR spill lane traffic (v_readlane/v_writelane)
    inside any kernel's main loop (the innermost loop that issues the MFMAs):
    a scratch reload there waits for every tile load in flight (the vector
    memory counter retires in order)."""
    spill = re.compile(r"^(scratch_|v_readlane_b32|v_writelane_b32)")
    checked = 0
    for src, text in asm_texts.items():
        kernels = _loop_blocks(text)
        assert kernels, f"no attention kernel found in {src}"
        for name, blocks in kernels.items():
            loops = {h for h, ins in blocks if h and any(i.startswith("v_mfma") for i in ins)}
            assert loops, f"{src} {name}: no loop with MFMAs found"
            bad = [i for h, ins in blocks if h in loops for i in ins if spill.match(i)]
            assert not bad, f"{src} {name}: spill traffic in the main loop: {bad[:4]}"
            checked += 1
    assert checked >= 20
