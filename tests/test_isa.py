"""Static checks of the generated gfx950 code (no GPU needed).

The scan kernel reads B_t / C_t through the DPP row_newbcast modifier of
hand-written VOP2 instructions (inline assembly).  On gfx9-family GPUs a VALU
write of a VGPR followed, within two wait states, by a DPP read of that VGPR
is a hazard the hardware does not interlock; the compiler does not insert wait
states for DPP reads inside inline assembly.  The kernel is written so that
every DPP source is produced by an LDS load; this test compiles the kernels to
assembly and checks that property on every DPP instruction of every
instantiation.
"""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRCS = [os.path.join(ROOT, "selective_scan_02_amd", "csrc", f) for f in ("scan_chunked.hip",)]

VGPR = re.compile(r"\bv\[?(\d+)(?::(\d+))?\]?")


def regs(tok):
    m = re.fullmatch(r"v(\d+)", tok)
    if m:
        return {int(m.group(1))}
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    return set()


@pytest.fixture(scope="module", params=SRCS, ids=lambda p: os.path.basename(p))
def asm(request, tmp_path_factory):
    src = request.param
    out = tmp_path_factory.mktemp("isa") / (os.path.basename(src) + ".s")
    cmd = ["/opt/rocm/bin/hipcc", "-O3", "-std=c++17", "--offload-arch=gfx950", "--cuda-device-only", "-S",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form",
           "-I", os.path.join(ROOT, "include"), "-o", str(out), src]
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text().splitlines()


def instructions(lines):
    """(kind, text) per line inside kernels: 'label', 'inst' (comments stripped)."""
    for l in lines:
        s = l.split(";")[0].strip()
        if not s:
            continue
        if s.endswith(":"):
            yield "label", s
        elif s.startswith("."):
            continue
        else:
            yield "inst", s


def test_dpp_sources_not_written_by_valu_within_two_wait_states(asm):
    insts = list(instructions(asm))
    n_dpp = 0
    bad = []
    for i, (kind, text) in enumerate(insts):
        if kind != "inst" or "_dpp " not in text:
            continue
        n_dpp += 1
        ops = [o.strip() for o in text.split(None, 1)[1].split(",")]
        src0 = regs(ops[1].split()[0])
        waits = 0
        j = i - 1
        while waits < 2 and j >= 0:
            k2, t2 = insts[j]
            if k2 == "label":
                # a block boundary: predecessors unknown -> treat as unsafe unless nothing VALU is in reach
                bad.append(("label-before-dpp", text))
                break
            mnem = t2.split()[0]
            if mnem.startswith("v_"):
                dst = regs(t2.split(None, 1)[1].split(",")[0].strip()) if " " in t2 else set()
                if dst & src0:
                    bad.append((t2, text))
                    break
            waits += int(t2.split()[1]) + 1 if mnem == "s_nop" else 1
            j -= 1
    assert n_dpp > 0, "no DPP instruction found: the check is not looking at the scan kernels"
    assert not bad, bad[:5]
