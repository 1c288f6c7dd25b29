"""Static checks of the compiled kernels' MFMA use (hipcc, no GPU needed).

1. No MFMA accumulator chain mixes shapes.  The CDNA3/CDNA4 ISA guides allow
   an MFMA to take the previous MFMA's result as its accumulator input (SrcC)
   back to back only when both are the same instruction; a SrcC written by an
   MFMA of another shape (v_mfma_f32_16x16x16_bf16 after
   v_mfma_f32_16x16x32_bf16, or the reverse) needs wait states.  The kernels
   keep every chain within one shape and join partial sums on the vector ALU.
2. No MFMA runs under a divergent branch (between an s_and_saveexec and the
   s_or_b64 exec that closes it): with part of EXEC off the product is wrong.

Each HIP source is compiled to gfx950 assembly and every kernel is walked
linearly.
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


def mfma_under_partial_exec(asm: str, allowed_depth=None):
    """(line number, text) of every MFMA issued while more divergent regions
    are open than the function may have around it.  A region opens with an
    s_and_saveexec / s_xor_saveexec into a register pair not already saved; an
    s_andn2_saveexec / s_or_saveexec enters the else half of an if/else (same
    region).  A region closes with the s_or_b64 exec that restores its pair --
    which also closes every region opened inside it (the compiler often
    restores an outer mask without restoring the inner ones) -- or, when the
    restored pair is not one saved on entry (an else half's), the innermost.
    allowed_depth maps a kernel-name fragment to the number of enclosing
    regions that are known to be wave-uniform (a role split by wave, which the
    compiler cannot prove uniform)."""
    allowed_depth = allowed_depth or {}
    bad = []
    stack = []
    allow = 0
    save = re.compile(r"s_(?:and|xor)_saveexec_b64\s+(s\[\d+:\d+\])")
    restore = re.compile(r"s_or_b64\s+exec,\s*exec,\s*(s\[\d+:\d+\])")
    for n, line in enumerate(asm.splitlines(), 1):
        t = line.strip()
        if t.endswith("@function"):
            stack = []
            allow = next((d for k, d in allowed_depth.items() if k in t), 0)
        elif t.startswith("s_endpgm"):
            stack = []
        elif save.match(t):
            reg = save.match(t).group(1)
            if reg not in stack:
                stack.append(reg)
        elif restore.match(t):
            reg = restore.match(t).group(1)
            if reg in stack:
                del stack[stack.index(reg):]
            elif stack:
                stack.pop()
        elif t.startswith("v_mfma") and len(stack) > allow:
            bad.append((n, t))
    return bad


# Kernels whose role split by wave (producers / inverse wave / consumers: an
# if, else-if, else on the wave index, two nested exec regions) encloses the
# MFMA code.
ROLE_SPLIT = {"chunk_fwd_kernel": 2, "bwd_chain_kernel": 2}


def test_scanner_flags_mfma_under_saveexec():
    asm = "\n".join([
        "k:",
        "v_mfma_f32_16x16x16_bf16 v[4:7], v[0:1], v[2:3], 0",
        "s_and_saveexec_b64 s[0:1], vcc",
        "v_mfma_f32_16x16x16_bf16 v[4:7], v[0:1], v[2:3], 0",
        "s_or_b64 exec, exec, s[0:1]",
        "v_mfma_f32_16x16x16_bf16 v[4:7], v[0:1], v[2:3], 0",
        "s_endpgm",
    ])
    assert [n for n, _ in mfma_under_partial_exec(asm)] == [4]
    role = "\n".join(["k_role: ; @function", "s_and_saveexec_b64 s[0:1], vcc",
                      "v_mfma_f32_16x16x16_bf16 v[4:7], v[0:1], v[2:3], 0",
                      "s_and_saveexec_b64 s[2:3], s[4:5]",
                      "v_mfma_f32_16x16x16_bf16 v[4:7], v[0:1], v[2:3], 0",
                      "s_or_b64 exec, exec, s[2:3]", "s_or_b64 exec, exec, s[0:1]", "s_endpgm"])
    assert [n for n, _ in mfma_under_partial_exec(role, {"k_role": 1})] == [5]
    # An if/else nested in an if whose one restore of the outer mask closes both.
    nested = "\n".join(["k2: ; @function",
                         "s_and_saveexec_b64 s[30:31], vcc",
                         "s_and_saveexec_b64 s[62:63], s[10:11]",
                         "s_xor_b64 s[62:63], exec, s[62:63]",
                         "v_mfma_f32_16x16x16_bf16 v[4:7], v[0:1], v[2:3], 0",
                         "s_andn2_saveexec_b64 s[62:63], s[62:63]",
                         "s_or_b64 exec, exec, s[30:31]",
                         "v_mfma_f32_16x16x16_bf16 v[4:7], v[0:1], v[2:3], 0",
                         "s_endpgm"])
    assert [n for n, _ in mfma_under_partial_exec(nested)] == [5]


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
def test_compiled_mfma_use(src, tmp_path):
    out = tmp_path / (src + ".s")
    cmd = [hip_build.HIPCC, *hip_build.COMMON, "--offload-device-only", "-S", "-x", "hip",
           os.path.join(hip_build.CSRC, src), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    asm = out.read_text()
    bad = mixed_shape_chains(asm)
    assert not bad, f"{src}: MFMA accumulator chains across shapes at {bad[:5]}"
    bad = mfma_under_partial_exec(asm, ROLE_SPLIT)
    assert not bad, f"{src}: MFMA under a divergent branch at {bad[:5]}"
