"""Host-side check of the compiled gfx950 code (no GPU needed).

The HBM -> LDS DMA instructions are issued from inline assembly, where the
compiler inserts no hazard wait states.  A vector-memory instruction must not
read an SGPR (its base address) or M0 fewer than five wait states after a
VALU instruction wrote it.  This test compiles every kernel source that issues
such DMAs to gfx950 assembly and checks each DMA site for that pattern."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "megatron_tensor_transformer_col_amd", "csrc")
SOURCES = ["attention.hip", "attn_bwd.hip", "gemv.hip", "gemm_lds.hip", "gemm_k64.hip"]
WAIT_STATES = 5

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                                reason="hipcc not available")


def _sgprs(text):
    regs = set()
    for m in re.finditer(r"s\[(\d+):(\d+)\]", text):
        regs.update(f"s{i}" for i in range(int(m.group(1)), int(m.group(2)) + 1))
    regs.update(f"s{m.group(1)}" for m in re.finditer(r"\bs(\d+)\b", text))
    if re.search(r"\bm0\b", text):
        regs.add("m0")
    return regs


def _is_inst(line):
    return bool(line) and not line.startswith((";", ".")) and not line.endswith(":")


def hazards(asm):
    lines = [l.split(";")[0].strip() for l in asm.splitlines()]
    found = []
    for i, line in enumerate(lines):
        if not line.startswith("global_load_lds"):
            continue
        operands = line.split(None, 1)[1] if " " in line else ""
        used = _sgprs(operands.split(",", 1)[1] if "," in operands else "") | {"m0"}
        waits, j = 0, i - 1
        while j >= 0 and waits < WAIT_STATES:
            prev = lines[j]
            j -= 1
            if not _is_inst(prev):
                continue
            mnemonic = prev.split()[0]
            if mnemonic == "s_nop":
                waits += int(prev.split()[1], 0) + 1
                continue
            if mnemonic.startswith("v_") and " " in prev:
                if _sgprs(prev.split(None, 1)[1].split(",")[0]) & used:
                    found.append((prev, line, waits))
            waits += 1
    return found


def _hipcc():
    return shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.mark.parametrize("src", SOURCES)
def test_no_valu_sgpr_hazard_before_lds_dma(src, tmp_path):
    flags = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops"]
    from megatron_tensor_transformer_col_amd import _build
    flags += _build.EXTRA_FLAGS.get(src, [])
    out = tmp_path / (src + ".s")
    r = subprocess.run([_hipcc(), *flags, "-S", "--cuda-device-only", "-o", str(out), os.path.join(CSRC, src)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    asm = out.read_text()
    assert asm.count("global_load_lds") > 0
    assert hazards(asm) == []


def test_checker_flags_the_hazard():
    planted = "\n".join(["v_readfirstlane_b32 s14, v4", "v_readfirstlane_b32 s15, v5", "s_nop 0",
                         "global_load_lds_dwordx4 v1, s[14:15]"])
    assert len(hazards(planted)) == 2
    fixed = planted.replace("s_nop 0", "s_nop 4")
    assert hazards(fixed) == []
