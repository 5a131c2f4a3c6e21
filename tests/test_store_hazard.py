"""The wait state after inline-assembly stores.

A vector store of more than 8 bytes reads its data registers one cycle after
issue, so a vector-ALU write to those registers in the next cycle needs a
wait state in between.  The compiler provides it after stores it emits
itself, but cannot see inside inline assembly, where the update's and the
probes' cache-policy stores are written.  This test compiles both sources to
gfx950 assembly (hipcc needs no GPU) and checks that every inline-assembly
block of stores ends with s_nop (stores inside one block have nothing the
compiler placed between them), and that no 16-byte store of any origin is
directly followed by a vector-ALU write to its data registers."""
import os
import re
import shutil
import subprocess

import pytest

from layer_streamed_optimizer_amd import build

HIPCC_MISSING = not os.path.exists(build.HIPCC) and shutil.which("hipcc") is None


def device_asm(source: str, tmp_path) -> list[str]:
    out = tmp_path / (os.path.basename(source) + ".s")
    flags = [f for f in build.FLAGS if f not in ("-shared", "-fPIC")]
    subprocess.check_call([build.HIPCC, *flags, "--cuda-device-only", "-S", source, "-o", str(out)],
                          stderr=subprocess.DEVNULL)
    return out.read_text().split("\n")


def vregs(spec: str) -> set[int]:
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", spec)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(r"v(\d+)", spec)
    return {int(m.group(1))} if m else set()


def next_instruction(lines: list[str], i: int) -> str:
    j = i + 1
    while j < len(lines):
        t = lines[j].strip()
        if t and not t.startswith(";"):
            return t
        j += 1
    return ""


@pytest.mark.skipif(HIPCC_MISSING, reason="hipcc not found")
@pytest.mark.parametrize("source", ["lso_adam.hip", "lso_probes.hip"])
def test_inline_stores_end_with_a_wait_state(source, tmp_path):
    lines = device_asm(os.path.join(build.CSRC, source), tmp_path)
    block, start, blocks = None, 0, 0
    for i, line in enumerate(lines):
        t = line.strip()
        if t.startswith(";;#ASMSTART"):
            block, start = [], i + 1
        elif t.startswith(";;#ASMEND"):
            if block and any(b.startswith("global_store") for b in block):
                blocks += 1
                assert block[-1].startswith("s_nop"), f"{source}:{start}: {block}"
            block = None
        elif block is not None and t and not t.startswith(";"):
            block.append(t)
    assert blocks > 0, "no inline-assembly stores found: the test looks at the wrong code"


@pytest.mark.skipif(HIPCC_MISSING, reason="hipcc not found")
def test_no_valu_write_right_after_a_16_byte_store(tmp_path):
    lines = device_asm(os.path.join(build.CSRC, "lso_adam.hip"), tmp_path)
    seen = 0
    for i, line in enumerate(lines):
        m = re.match(r"\s*global_store_dwordx4 \S+, (v\[\d+:\d+\]),", line)
        if not m:
            continue
        seen += 1
        nxt = re.match(r"(v_\w+)\s+(v\[\d+:\d+\]|v\d+)", next_instruction(lines, i))
        assert not (nxt and vregs(nxt.group(2)) & vregs(m.group(1))), f"line {i + 1}: {line.strip()}"
    assert seen > 0
