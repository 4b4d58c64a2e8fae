"""Hazard checks on the generated gfx950 code of the MLA kernel (CPU only: compiles to assembly).

The score products of the MLA kernel are inline-assembly matrix ops with VGPR
accumulators, which the compiler's hazard recognizer does not know.  Their
safety rests on two properties of the code around them, checked here on the
assembly hipcc actually produces:

* no VALU instruction writes a source register of such a matrix op within the
  two wait states before it (the wait a VALU-written operand needs);
* no instruction other than a matrix op accumulating into the same registers
  reads a result of such a matrix op within 20 wait states of it (more than
  the 16x16x32 bf16 op's longest result-read wait).
"""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "decode_attention_kv_03_amd", "csrc", "mla_bf16.hip")

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                                reason="hipcc not available")

REG = re.compile(r"\bv(\d+)\b|\bv\[(\d+):(\d+)\]")
VALU_WRITE_WAIT = 2
RESULT_READ_WAIT = 20


def regs(text):
    out = set()
    for m in REG.finditer(text):
        if m.group(1) is not None:
            out.add(int(m.group(1)))
        else:
            out.update(range(int(m.group(2)), int(m.group(3)) + 1))
    return out


def split_operands(line):
    parts = line.split(None, 1)
    if len(parts) == 1:
        return parts[0], []
    ops = [o.strip() for o in parts[1].split(",")]
    return parts[0], ops


def wait_states(op, ops):
    if op == "s_nop":
        return int(ops[0], 0) + 1
    return 1


@pytest.fixture(scope="module")
def asm_lines(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    out = tmp_path_factory.mktemp("mla_asm") / "mla.s"
    cmd = [hipcc, "-O3", "-std=c++17", "--offload-arch=gfx950", "-I", os.path.join(ROOT, "include"),
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "--cuda-device-only", "-S", "-x", "hip",
           SRC, "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    lines = []
    for raw in open(out):
        line = raw.split(";")[0].strip()
        if not line or line.startswith(".") or line.endswith(":"):
            continue
        lines.append(line)
    return lines


def vgpr_form_mfma(op, ops):
    return op.startswith("v_mfma") and ops and ops[0].startswith("v")


def test_vgpr_form_score_products_present(asm_lines):
    n = sum(1 for l in asm_lines if vgpr_form_mfma(*split_operands(l)))
    assert n >= 72, f"expected the inline-asm score products, found {n} VGPR-form matrix ops"


def test_no_valu_write_of_an_operand_just_before(asm_lines):
    bad = []
    for i, line in enumerate(asm_lines):
        op, ops = split_operands(line)
        if not vgpr_form_mfma(op, ops):
            continue
        srcs = regs(",".join(ops[1:]))
        budget, j = 0, i - 1
        while j >= 0 and budget < VALU_WRITE_WAIT:
            pop, pops = split_operands(asm_lines[j])
            if pop.startswith("v_") and not pop.startswith("v_mfma") and pops:
                if regs(pops[0]) & srcs:
                    bad.append((asm_lines[j], line))
            budget += wait_states(pop, pops)
            j -= 1
    assert not bad, f"VALU writes of matrix-op operands without wait states: {bad[:3]}"


def test_results_not_read_early(asm_lines):
    pending = {}  # vgpr -> wait states since a VGPR-form matrix op wrote it
    bad = []
    for line in asm_lines:
        op, ops = split_operands(line)
        if vgpr_form_mfma(op, ops):
            dst = regs(ops[0])
            src_c = regs(ops[3]) if len(ops) > 3 else set()
            # Accumulating into exactly its own destination is the supported back-to-back form.
            early = {r for r in regs(",".join(ops[1:3])) if r in pending}
            if early:
                bad.append(line)
            for r in dst:
                pending[r] = 0
            continue
        reads = regs(",".join(ops[1:])) if op.startswith(("v_", "ds_read", "global_load", "buffer_load")) else regs(
            ",".join(ops))
        early = [r for r in reads if r in pending]
        if early:
            bad.append(line)
        if op.startswith(("v_", "ds_read", "global_load")) and ops:
            for r in regs(ops[0]):
                pending.pop(r, None)
        ws = wait_states(op, ops)
        for r in list(pending):
            pending[r] += ws
            if pending[r] >= RESULT_READ_WAIT:
                del pending[r]
    assert not bad, f"matrix-op results read within {RESULT_READ_WAIT} wait states: {bad[:3]}"
