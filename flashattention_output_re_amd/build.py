"""Build libfa_relayout.so in-tree with hipcc for gfx950.

Usage: python -m flashattention_output_re_amd.build [--asm DIR]
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_NAME = "libfa_relayout.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = ["fa_abi.hip", "fa_fwd_kernel.hip", "fa_relayout_kernel.hip", "burst_gap.hip"]
ARCH = "gfx950"

# hipcc must not emit packed fp32 VALU ops (v_pk_fma_f32 and friends).  The
# device code never tests for NaN, so max/min need no NaN canonicalisation.
HIP_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Xarch_device", "-fno-honor-nans", "-Xarch_device", "-fno-signed-zeros",
             # MFMA accumulators in VGPRs: the softmax reads the score tile
             # every stage, and AGPR-form MFMAs would copy it across.
             "-mllvm", "-amdgpu-mfma-vgpr-form"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def compile_cmd(out: str, extra=()) -> list:
    return ([hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
             "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include")]
            + HIP_FLAGS + list(extra)
            + [os.path.join(CSRC, s) for s in SOURCES] + ["-o", out])


def build(asm_dir: str | None = None, quiet: bool = True) -> str:
    """Compile every HIP source into LIB_PATH (atomically replaced)."""
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    extra = []
    if asm_dir:
        os.makedirs(asm_dir, exist_ok=True)
        extra = ["-save-temps=cwd", "-o", tmp]
    cmd = compile_cmd(tmp)
    if asm_dir:
        cmd = cmd[:-2] + extra
    res = subprocess.run(cmd, cwd=asm_dir or PKG, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if msgs and not quiet:
        print("\n".join(msgs), file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", default=None, help="keep intermediate files (incl. gfx950 .s) here")
    a = ap.parse_args()
    print(build(a.asm, quiet=False))


if __name__ == "__main__":
    main()
