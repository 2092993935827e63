"""Every gfx950 kernel of the library fits its register budget: no VGPR/SGPR
spills and no per-lane scratch.

A spill puts a kernel's registers in scratch memory (private segment) -- an
extra memory round trip inside loops that are built to keep every operand in
registers, and a per-dispatch scratch allocation.  The launch bounds and
occupancy targets of the kernels (e.g. two 256-thread workgroups per CU for
the 128x128 prefill tile, i.e. at most 256 registers per lane) leave little
room, so a source change that adds live values (a wider reduction batch, an
extra fragment set) can tip one over without any test failing on numbers.
This compiles each source for the device only (hipcc cross-compiles without a
GPU) and reads the kernel metadata the compiler emits."""
import glob
import os
import re
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "block_scaled_precision_04_amd", "csrc")


def _hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return None


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
@pytest.mark.parametrize("src", sorted(os.path.basename(p) for p in glob.glob(os.path.join(CSRC, "*.hip"))))
def test_no_spills(src, tmp_path):
    out = tmp_path / (src + ".s")
    cmd = [_hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "--cuda-device-only", "-S",
           os.path.join(CSRC, src), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    text = out.read_text()
    # one metadata block per kernel: .name, then the counts
    kernels = re.findall(r"\.name:\s+(\S+)", text)
    for key in ("vgpr_spill_count", "sgpr_spill_count", "private_segment_fixed_size"):
        vals = [int(v) for v in re.findall(rf"\.{key}:\s+(\d+)", text)]
        assert all(v == 0 for v in vals), f"{src}: {key} = {vals} (kernels {kernels})"
