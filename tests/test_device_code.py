"""Properties of the compiled gfx950 device code, checked on the generated assembly (no GPU).

1. No MFMA sits in a lane-masked block without a skip branch. A matrix instruction runs on
   all 64 lanes whatever the EXEC mask holds, so an MFMA that the compiler leaves in the body
   of a divergent `if` (after an `s_and_saveexec` with no `s_cbranch_execz` around it) still
   executes in waves that take the other path, on operands those waves never loaded, and
   writes its destination registers. The kernels branch on the wave index around their MFMAs;
   these branches are uniform at run time, so the skip branch is all they need.
2. The kernels keep their state in registers: no VGPR spills, apart from the grouped-value
   gradient kernel at its largest shape, whose small spill is known and bounded.
"""
import os
import re
import shutil
import subprocess

import pytest

from chunked_gated_delta_09_amd import build as kbuild

# sources with kernels (kda_noalloc.hip holds only a device array and host code)
HIP_SOURCES = [s for s in kbuild.SOURCES if s.endswith(".hip") and s != "kda_noalloc.hip"]

# known spills: the grouped-value gradient kernel at K = V = 128, C = 64
SPILL_LIMITS = {"_ZN3kda15bwd_grad_kernelIDF16bLi128ELi128ELi64ELb1E": 16}


def masked_mfmas(asm: str):
    """(kernel, line) of every MFMA that follows a saveexec in the same basic block."""
    cur, open_at, found = None, None, []
    for i, line in enumerate(asm.splitlines(), 1):
        m = re.match(r"^(_Z\w+):", line)
        if m:
            cur, open_at = m.group(1), None
            continue
        t = line.strip()
        if t.startswith(".LBB") or t.startswith("s_cbranch") or t.startswith("s_branch"):
            open_at = None
        elif re.match(r"s_(and|andn2|or)_saveexec", t):
            open_at = i
        elif re.match(r"s_or_b64 exec, exec", t) or re.match(r"s_mov_b64 exec,", t):
            open_at = None
        elif t.startswith("v_mfma") and open_at is not None:
            found.append((cur, i))
    return found


def kernel_meta(asm: str):
    """{kernel symbol: (mfma count, vgpr spill count)} from the code and its metadata."""
    mfma, cur = {}, None
    for line in asm.splitlines():
        m = re.match(r"^(_Z\w+):", line)
        if m:
            cur = m.group(1)
            mfma[cur] = 0
        elif cur and line.strip().startswith("v_mfma"):
            mfma[cur] += 1
    spills, name = {}, None
    for line in asm.splitlines():
        t = line.strip()
        if t.startswith(".name:"):
            name = t.split()[1]
        elif t.startswith(".vgpr_spill_count:") and name:
            spills[name] = int(t.split()[1])
    return {k: (mfma.get(k, 0), spills.get(k, 0)) for k in spills}


def test_detector_flags_a_masked_mfma():
    unsafe = """_Zk:
\tv_cmp_gt_i32_e32 vcc, s4, v0
\ts_and_saveexec_b64 s[2:3], vcc
\tv_mfma_f32_16x16x32_bf16 v[2:5], v[10:13], v[14:17], v[2:5]
\ts_or_b64 exec, exec, s[2:3]
"""
    safe = unsafe.replace("vcc\n\tv_mfma", "vcc\n\ts_cbranch_execz .LBB0_2\n\tv_mfma")
    assert masked_mfmas(unsafe) == [("_Zk", 4)]
    assert masked_mfmas(safe) == []


@pytest.fixture(scope="module")
def device_asm(tmp_path_factory):
    hipcc = kbuild._hipcc()
    if not (os.path.isabs(hipcc) and os.path.exists(hipcc)) and shutil.which(hipcc) is None:
        pytest.skip("hipcc not available")
    out = {}
    d = tmp_path_factory.mktemp("asm")
    for src in HIP_SOURCES:
        path = d / (src + ".s")
        cmd = [hipcc] + kbuild.HIP_FLAGS + ["-S", "--cuda-device-only", os.path.join(kbuild.CSRC, src), "-o", str(path)]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr
        out[src] = path.read_text()
    return out


@pytest.mark.parametrize("src", HIP_SOURCES)
def test_no_mfma_in_lane_masked_block(device_asm, src):
    asm = device_asm[src]
    assert "v_mfma" in asm
    assert masked_mfmas(asm) == []


@pytest.mark.parametrize("src", HIP_SOURCES)
def test_kernels_do_not_spill(device_asm, src):
    meta = kernel_meta(device_asm[src])
    assert meta
    for name, (_, spill) in meta.items():
        limit = next((v for k, v in SPILL_LIMITS.items() if name.startswith(k)), 0)
        assert spill <= limit, (name, spill)
