"""Register budget of the fused kernel's instances, read from the compiler's
resource-usage remarks (hipcc -Rpass-analysis=kernel-resource-usage with the
library's own flags, device code for gfx950 only).

Each instance runs one workgroup of 8 waves per CU, two waves per SIMD, so a
wave may hold 256 VGPRs.  Every product instance (whole, split-key and masked
forms; D = 64 and 128; slab and plain output; either sign of the scale) must
fit with no VGPR spill; the slab-input instances at D = 128, which add the
per-lane slab offsets to the same loop, may spill at most 8 VGPRs; the
timestamped instances and the merge kernel none.  Runs on the CPU (hipcc
cross-compiles); skipped where hipcc is absent.
"""
import os
import re
import subprocess

import pytest

from flashattention_output_re_amd import build

KERNEL = re.compile(r"fa_fwd_pp_kernelILi(\d+)ELNS_9StoreModeE(\d)ELb(\d)ELb(\d)ELb(\d)ELb(\d)E(?:Li(\d)E)?")


def _remarks():
    try:
        cc = build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    src = os.path.join(build.CSRC, "fa_fwd_kernel.hip")
    cmd = ([cc, f"--offload-arch={build.ARCH}", "-O3", "-std=c++17", "-c", "--offload-device-only",
            "-I", os.path.join(build.ROOT, "include")] + build.HIP_FLAGS +
           ["-Rpass-analysis=kernel-resource-usage", src, "-o", os.devnull])
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=900)
    assert res.returncode == 0, res.stderr[-2000:]
    rows, cur = [], None
    for line in res.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = {"name": m.group(1)}
            rows.append(cur)
            continue
        m = re.search(r"remark:\s+(VGPRs|VGPRs Spill|AGPRs): (\d+)", line)
        if m and cur is not None:
            cur[m.group(1)] = int(m.group(2))
    return rows


@pytest.fixture(scope="module")
def remarks():
    return _remarks()


def test_fused_kernel_register_budget(remarks):
    seen = 0
    for r in remarks:
        m = KERNEL.search(r["name"])
        if not m:
            continue
        seen += 1
        D, mode, neg, split, masked, slab_in, instr = m.groups()
        what = (f"D={D} mode={mode} neg={neg} split={split} masked={masked} slab_in={slab_in} "
                f"instr={instr or 0}")
        assert r["VGPRs"] + r.get("AGPRs", 0) <= 256, what
        if slab_in == "1":
            assert r["VGPRs Spill"] <= 8, f"{what}: {r['VGPRs Spill']} VGPRs spilled"
        else:
            assert r["VGPRs Spill"] == 0, f"{what}: {r['VGPRs Spill']} VGPRs spilled"
    # 3 forms x 2 D x (slab: 2 signs x 2 inputs; plain: 2 signs) = 36 product
    # instances, plus the 9 timestamped ones.
    assert seen >= 45, seen


def test_merge_kernel_no_spill(remarks):
    merges = [r for r in remarks if "fa_merge_kernel" in r["name"]]
    assert len(merges) == 4            # D = 64, 128 x slab, plain
    for r in merges:
        assert r["VGPRs Spill"] == 0, r["name"]
