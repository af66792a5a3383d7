"""Hazard padding of the built decode kernels (CPU: hipcc only, no GPU).

On gfx950 nothing interlocks a vector read (or overwrite) of a matrix-core
result: the 16x16x128 FP8 product's accumulators become readable 11 wait
states after the instruction issues (measured: 9 wait states read the old
register contents, 11 the result). The compiler pads for this itself, but has
been seen to leave only 3 wait states where the scores of a tile go straight
into the softmax maximum, which silently turned every full tile's scores into
the operand bytes. This test compiles the kernels to gfx950 assembly and
checks, along every control-flow path, that no non-matrix instruction touches
a matrix-core result register within 11 wait states of the instruction that
writes it.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "sparse_attention_decode_row_amd", "csrc", "kernels.hip")
WAITS = 11


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


def _regs(tok):
    tok = tok.strip()
    m = re.match(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _touches(ins, dst):
    parts = ins.split(None, 1)
    ops = parts[1].split(",") if len(parts) > 1 else []
    op = parts[0]
    if op.startswith("v_mfma"):
        # a dependent product reads A and B early; an accumulator chain
        # (the same registers as C) is forwarded by the hardware
        return bool((_regs(ops[1]) | _regs(ops[2])) & dst)
    if op.startswith(("v_", "ds_", "global_", "buffer_", "scratch_", "flat_")):
        return any(_regs(o) & dst for o in ops)
    return False


def short_paddings(asm_lines, waits=WAITS):
    """(function, wait states, instruction, product) for every matrix-core
    result touched sooner than `waits` wait states after the product."""
    lines = [l.split(";")[0].strip() for l in asm_lines]
    labels = {l[:-1]: i for i, l in enumerate(lines) if l.endswith(":")}
    found, fn = [], None
    for i, l in enumerate(lines):
        m = re.match(r"^(_Z\S+):", asm_lines[i])
        if m:
            fn = m.group(1)
        if not l.startswith("v_mfma") or fn is None:
            continue
        dst = _regs(l.split(None, 1)[1].split(",")[0])
        stack, seen = [(i + 1, 0)], set()
        while stack:
            j, w = stack.pop()
            while j < len(lines) and w < waits and (j, w) not in seen:
                seen.add((j, w))
                ins = lines[j]
                j += 1
                if not ins or ins.endswith(":") or ins.startswith("."):
                    continue
                op = ins.split()[0]
                if op == "s_nop":
                    w += int(ins.split()[1], 0) + 1
                    continue
                if op in ("s_endpgm", "s_setpc_b64"):
                    break
                if _touches(ins, dst):
                    found.append((fn, w, ins, l))
                    break
                if op.startswith("s_cbranch") and ins.split()[1] in labels:
                    stack.append((labels[ins.split()[1]] + 1, w + 1))
                if op == "s_branch" and ins.split()[1] in labels:
                    j = labels[ins.split()[1]] + 1
                w += 1
    return found


def test_scanner_finds_a_short_padding():
    asm = ["_Zkernel:",
           "v_mfma_f32_16x16x128_f8f6f4 v[66:69], v[66:73], v[10:17], v[74:77]",
           "s_setprio 0",
           "s_cbranch_scc1 .LBB0_2",
           "v_med3_f32 v70, v66, v67, v117",
           ".LBB0_2:",
           "s_nop 7",
           "s_nop 2",
           "v_cndmask_b32_e64 v66, 0, 1, s[0:1]"]
    found = short_paddings(asm)
    assert [f[1] for f in found] == [2]
    padded = asm[:2] + ["s_nop 7", "s_nop 2"] + asm[2:]
    assert short_paddings(padded) == []


def test_decode_kernels_pad_matrix_results(tmp_path):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    out = str(tmp_path / "kernels_gfx950.s")
    cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-S",
           "--offload-device-only", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.dirname(SRC), "-o", out, SRC]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    with open(out) as f:
        asm = f.read().split("\n")
    assert sum("v_mfma" in l for l in asm) > 100
    found = short_paddings(asm)
    assert found == [], "\n".join(f"{fn[:70]}: {w} wait states before {ins} (after {p})"
                                  for fn, w, ins, p in found[:10])
