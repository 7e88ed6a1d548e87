"""Build the HIP libraries in-tree for gfx950.

    python -m position_invariant_kv_amd.build

* libkamera.so — the operator's C ABI (include/kamera.h);
* libkamera_probe.so — the copy-ceiling probe the benchmark reads the
  operator's rate against (include/kamera_probe.h).

Both land next to this file; they are git-ignored but travel with the source
tree.  Every build recompiles: each source is compiled to an object in
parallel, then the objects are linked.  Compiler warnings that matter for the
kernels' speed (register spills, launch bounds the compiler could not meet)
are always printed.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SRCS = [os.path.join(CSRC, f) for f in ("kamera.hip", "kamera_form.hip", "kamera_attn.hip", "kamera_host.cpp")]
PROBE_SRCS = [os.path.join(CSRC, "kamera_probe.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libkamera.so")
PROBE_LIB = os.path.join(HERE, "libkamera_probe.so")
OBJ_DIR = os.path.join(HERE, "_build")
ARCH = "gfx950"

# warnings about code quality that are printed even when the build succeeds
_LOUD = ("-Wpass-failed", "spill", "scratch")
# the host pass does not know the packed-fp32 target feature: harmless
_NOISE = "is not a recognized feature for this target"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the Kamera HIP library cannot be built")


def compile_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        # packed fp32 VALU instructions stay off: hipcc would otherwise pair
        # ordinary float code into them
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # keep MFMA accumulators in VGPRs (no AGPR copies around each MFMA)
        "-mllvm", "-amdgpu-mfma-vgpr-form",
        "-Wno-unused-command-line-argument",
        "-I", INCLUDE,
    ]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines() if _NOISE not in l)
    return res.returncode, err


def _compile(src: str) -> tuple[str, int, str, list[str]]:
    obj = os.path.join(OBJ_DIR, os.path.basename(src) + f".{os.getpid()}.o")
    cmd = [hipcc(), *compile_flags(), "-c", src, "-o", obj]
    rc, err = _run(cmd)
    return obj, rc, err, cmd


def _link(objs, out) -> None:
    tmp = out + f".tmp{os.getpid()}"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", *objs, "-o", tmp]
    rc, err = _run(cmd)
    if rc != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError(f"link failed ({rc}):\n{' '.join(cmd)}\n{err}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    srcs = SRCS + PROBE_SRCS
    with ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        results = list(ex.map(_compile, srcs))
    failed = [r for r in results if r[1] != 0]
    for obj, rc, err, cmd in results:
        loud = [l for l in err.splitlines() if any(k in l for k in _LOUD)]
        if loud:
            print("\n".join(loud), file=sys.stderr)
        elif verbose and err.strip():
            print(err, file=sys.stderr)
    try:
        if failed:
            obj, rc, err, cmd = failed[0]
            raise RuntimeError(f"hipcc failed ({rc}):\n{' '.join(cmd)}\n{err}")
        objs = {os.path.basename(s): r[0] for s, r in zip(srcs, results)}
        _link([objs[os.path.basename(s)] for s in SRCS], LIB)
        _link([objs[os.path.basename(s)] for s in PROBE_SRCS], PROBE_LIB)
    finally:
        for obj, *_ in results:
            if os.path.exists(obj):
                os.remove(obj)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
