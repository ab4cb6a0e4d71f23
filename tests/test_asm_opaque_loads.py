"""The small GEMM's n-contiguous B stages are loaded with inline-asm loads
that the compiler does not track (its own wait insertion drained every load
in flight at the unrolled loop's back edge). Their safety rests on the
kernel's explicit waits: no instruction may read or overwrite a
destination register of such a load before an s_waitcnt whose vmcnt is at
most the number of vector-memory loads issued after it on that path.

This test compiles gemm_small.hip to gfx950 assembly (host-side hipcc, no
GPU) and checks that property on every path of the control-flow graph of
every kernel, so that a compiler or source change that breaks it fails
here, on the CPU, before any GPU run.
"""
import os
import re
import shutil
import subprocess

import pytest

from unstructured_sparse_feedforward_amd import build as B


def _asm(tmp_path) -> str:
    try:
        cc = B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    out = tmp_path / "gemm_small.s"
    src = os.path.join(B.CSRC, "gemm_small.hip")
    cmd = [cc, *[f for f in B.FLAGS if f != "-fPIC"], "--cuda-device-only", "-S", src, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def _vregs(text: str) -> set:
    text = text.split(";")[0]
    regs = set()
    for m in re.finditer(r"(?<![\w\]])v\[(\d+):(\d+)\]", text):
        regs |= set(range(int(m.group(1)), int(m.group(2)) + 1))
    for m in re.finditer(r"(?<![\w\[])v(\d+)\b", text):
        regs.add(int(m.group(1)))
    return regs


def _functions(lines):
    starts = [i for i, l in enumerate(lines) if re.match(r"^_Z\w+:", l)]
    for a, b in zip(starts, starts[1:] + [len(lines)]):
        yield lines[a + 1:b]


def _hazards(body):
    """(instructions, labels) of one kernel; returns the opaque loads checked
    and the hazards found."""
    ins, labels, asm_next = [], {}, False
    for l in body:
        t = l.strip()
        if re.match(r"^\.LBB\d+_\d+:", t):
            labels[t.split(":")[0]] = len(ins)
            continue
        if t.startswith(";;#ASMSTART"):
            asm_next = True
            continue
        if not t or t.startswith(";") or t.startswith(".") or t.endswith(":"):
            continue
        ins.append((t, asm_next and t.startswith("global_load")))
        asm_next = False
        if t.startswith("s_endpgm"):
            break

    def succ(k):
        t = ins[k][0]
        m = re.match(r"s_branch (\.LBB\d+_\d+)", t)
        if m:
            return [labels[m.group(1)]]
        m = re.match(r"s_cbranch_\w+ (\.LBB\d+_\d+)", t)
        if m:
            return [labels[m.group(1)], k + 1]
        if t.startswith("s_endpgm") or t.startswith("s_setpc"):
            return []
        return [k + 1]

    checked, bad = 0, []
    for k, (t, opaque) in enumerate(ins):
        if not opaque:
            continue
        checked += 1
        dst = _vregs(t.split(None, 1)[1].split(",")[0])   # the destination operand
        stack, seen = [(s, 0) for s in succ(k)], set()
        while stack:
            p, after = stack.pop()
            if p >= len(ins) or (p, min(after, 64)) in seen:
                continue
            seen.add((p, min(after, 64)))
            tt = ins[p][0]
            m = re.match(r"s_waitcnt.*vmcnt\((\d+)\)", tt)
            if m and int(m.group(1)) <= after:
                continue          # the load has landed on this path
            if p == k or _vregs(tt) & dst:
                bad.append((t, tt, after))
                continue
            a2 = after + (1 if re.match(r"(global_load|buffer_load)", tt) else 0)
            stack.extend((s, a2) for s in succ(p))
    return checked, bad


def test_opaque_b_loads_are_waited_on(tmp_path):
    lines = _asm(tmp_path).split("\n")
    total, hazards = 0, []
    for body in _functions(lines):
        c, h = _hazards(body)
        total += c
        hazards += h
    # the n-contiguous-B instantiations load B this way
    assert total >= 16, total
    assert not hazards, hazards[:5]


def test_checker_finds_a_missing_wait():
    """The check itself: an opaque load whose register is read with no wait
    in between, and one read after a sufficient wait."""
    body = [
        ";;#ASMSTART", "global_load_dwordx4 v[4:7], v[0:1], off", ";;#ASMEND",
        "global_load_dwordx4 v[8:11], v[0:1], off",
        "v_add_f32_e32 v12, v4, v5",
        "s_endpgm",
    ]
    c, h = _hazards(body)
    assert c == 1 and len(h) == 1
    body[4:4] = ["s_waitcnt vmcnt(1)"]
    c, h = _hazards(body)
    assert c == 1 and not h
    body[4] = "s_waitcnt vmcnt(2)"      # too weak: one load after it, vmcnt(2) can leave it pending
    c, h = _hazards(body)
    assert len(h) == 1
