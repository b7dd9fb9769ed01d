"""Build the HIP library ``libsvq.so`` in-tree for gfx950 with hipcc.

The library is the C-ABI declared in ``include/svq.h``: host packers
(``csrc/pack.cpp``) plus the gfx950 kernels and device entry points
(``csrc/svq.hip``).  Every call compiles from source; nothing is cached.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libsvq.so")
ARCH = "gfx950"

# Packed-FP32 VALU forms are kept out of the device code on purpose.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libsvq.so)")


def build(verbose: bool = False, jobs: int = 2) -> str:
    """Compile csrc/*.hip and csrc/*.cpp for gfx950 and link libsvq.so."""
    cc = hipcc()
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    common = ["-O3", "-std=c++17", "-fPIC", "-Wall", f"--offload-arch={ARCH}"] + inc
    objs = []
    procs = []
    out_dir = os.path.join(PKG, "_build")
    os.makedirs(out_dir, exist_ok=True)
    for name in sorted(os.listdir(CSRC)):
        if not name.endswith((".hip", ".cpp")):
            continue
        src = os.path.join(CSRC, name)
        obj = os.path.join(out_dir, name + ".o")
        cmd = [cc, "-c", src, "-o", obj] + common
        if name.endswith(".hip"):
            cmd += DEVICE_FLAGS
        else:
            cmd = [cc, "-x", "c++", "-c", src, "-o", obj, "-O3", "-std=c++17", "-fPIC", "-Wall"] + inc
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((subprocess.Popen(cmd, stderr=subprocess.PIPE, text=True), name))
        objs.append(obj)
        if len(procs) >= jobs:
            _wait(procs)
    _wait(procs)
    link = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", LIB + ".tmp"] + objs + ["-lpthread"]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def _wait(procs):
    while procs:
        p, name = procs.pop(0)
        _, err = p.communicate()
        noise = "is not a recognized feature for this target"
        msgs = [l for l in err.splitlines() if noise not in l]
        if msgs:
            sys.stderr.write("\n".join(msgs) + "\n")
        if p.returncode:
            raise RuntimeError(f"hipcc failed on {name}")


if __name__ == "__main__":
    print(build(verbose=True))
