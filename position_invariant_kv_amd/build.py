"""Build libkamera.so (the C-ABI HIP library) in-tree for gfx950.

    python -m position_invariant_kv_amd.build

The library lands next to this file; it is git-ignored but travels with the
source tree.  Every build recompiles.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRCS = [os.path.join(HERE, "csrc", "kamera.hip"), os.path.join(HERE, "csrc", "kamera_form.hip"),
        os.path.join(HERE, "csrc", "kamera_attn.hip"), os.path.join(HERE, "csrc", "kamera_host.cpp")]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libkamera.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the Kamera HIP library cannot be built")


def build_command(out: str) -> list[str]:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # packed fp32 VALU instructions stay off: hipcc would otherwise pair
        # ordinary float code into them
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # keep MFMA accumulators in VGPRs (no AGPR copies around each MFMA)
        "-mllvm", "-amdgpu-mfma-vgpr-form",
        "-Wno-unused-command-line-argument",
        "-I", INCLUDE, *SRCS, "-o", out,
    ]


def build(verbose: bool = False) -> str:
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = build_command(tmp)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
