"""Static check of the compiled kernels: no MFMA accumulator chain mixes shapes.

On gfx950 a v_mfma_f32_16x16x16_bf16 whose accumulator input (SrcC) was
written by a v_mfma_f32_16x16x32_bf16 (or the reverse) needs 5 wait states
that the compiler does not insert; the kernels keep every chain within one
shape and join partial sums on the vector ALU.  This test compiles each HIP
source to gfx950 assembly and walks every kernel linearly, tracking which
registers were last written by which MFMA shape.  It needs hipcc but no GPU.
"""

import os
import re
import shutil
import subprocess

import pytest

from rwkv_wkv7_delta_amd import build as hip_build

SOURCES = [s for s in hip_build.SOURCES if s.endswith(".hip")]
MFMA = re.compile(r"^\s*v_mfma_\w*?(\d+x\d+x\d+)\w*\s+(.*)$")
REG = re.compile(r"^([va])(?:(\d+)|\[(\d+):(\d+)\])$")
NO_VGPR_DST = ("ds_write", "ds_store", "global_store", "buffer_store", "flat_store",
               "scratch_store", "s_", "v_cmp", "v_readlane", "v_readfirstlane", ";", ".")


def _regs(op):
    m = REG.match(op.strip())
    if not m:
        return []
    kind = m.group(1)
    if m.group(2) is not None:
        return [f"{kind}{m.group(2)}"]
    return [f"{kind}{i}" for i in range(int(m.group(3)), int(m.group(4)) + 1)]


def mixed_shape_chains(asm: str):
    """(line number, text) of every MFMA whose SrcC was last written by an MFMA
    of another shape, scanning each function in program order."""
    bad = []
    last = {}
    for n, line in enumerate(asm.splitlines(), 1):
        t = line.strip()
        if t.startswith("s_endpgm") or t.endswith("@function"):
            last = {}
            continue
        m = MFMA.match(line)
        if m:
            shape = m.group(1)
            ops = [o.strip() for o in m.group(2).split(",")]
            if len(ops) >= 4:
                for r in _regs(ops[3]):
                    if last.get(r) not in (None, shape):
                        bad.append((n, t))
                        break
            for r in _regs(ops[0]):
                last[r] = shape
            continue
        if not t or t.startswith(NO_VGPR_DST) or t.endswith(":"):
            continue
        parts = t.split(None, 1)
        if len(parts) == 2:
            for r in _regs(parts[1].split(",")[0]):
                last[r] = None
    return bad


def test_scanner_flags_a_mixed_chain():
    asm = "\n".join([
        "k:",
        "v_mfma_f32_16x16x16_bf16 v[4:7], v[0:1], v[2:3], 0",
        "v_mfma_f32_16x16x32_bf16 v[4:7], v[8:11], v[12:15], v[4:7]",
        "v_mfma_f32_16x16x32_bf16 v[4:7], v[8:11], v[12:15], v[4:7]",
        "v_add_f32_e32 v20, v4, v5",
        "v_mov_b32_e32 v5, 0",
        "v_mfma_f32_16x16x16_bf16 v[24:27], v[0:1], v[2:3], v[4:7]",
        "s_endpgm",
    ])
    assert [n for n, _ in mixed_shape_chains(asm)] == [3, 7]


@pytest.mark.skipif(shutil.which(hip_build.HIPCC) is None and not os.path.exists(hip_build.HIPCC),
                    reason="hipcc not available")
@pytest.mark.parametrize("src", SOURCES)
def test_no_mixed_shape_accumulator_chain(src, tmp_path):
    out = tmp_path / (src + ".s")
    cmd = [hip_build.HIPCC, *hip_build.COMMON, "--offload-device-only", "-S", "-x", "hip",
           os.path.join(hip_build.CSRC, src), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    bad = mixed_shape_chains(out.read_text())
    assert not bad, f"{src}: MFMA accumulator chains across shapes at {bad[:5]}"
