"""Build the HIP library ``libsvq.so`` in-tree for gfx950 with hipcc.

The library is the C-ABI declared in ``include/svq.h``: host packers
(``csrc/pack.cpp``) plus the gfx950 kernels (``csrc/kernels.h``) and the
device entry points (``csrc/svq_*.hip``).  Every call compiles from source; nothing is cached.
"""
from __future__ import annotations

import hashlib
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


def device_source_digest() -> str:
    """sha256 over the device sources (csrc/*.hip and csrc/*.h, by name and
    content): any change to a kernel or its launch changes it."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h")):
            h.update(name.encode() + b"\0")
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libsvq.so)")


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile csrc/*.hip and csrc/*.cpp for gfx950 and link libsvq.so.

    Up to ``jobs`` compilers run at once; the largest translation units
    (the sign-plane kernels) start first.
    """
    cc = hipcc()
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    common = ["-O3", "-std=c++17", "-fPIC", "-Wall", f"--offload-arch={ARCH}"] + inc
    out_dir = os.path.join(PKG, "_build")
    os.makedirs(out_dir, exist_ok=True)
    names = [n for n in os.listdir(CSRC) if n.endswith((".hip", ".cpp"))]
    names.sort(key=lambda n: (-os.path.getsize(os.path.join(CSRC, n)), n))
    cmds = []
    objs = []
    for name in names:
        src = os.path.join(CSRC, name)
        obj = os.path.join(out_dir, name + ".o")
        if name.endswith(".hip"):
            cmd = [cc, "-c", src, "-o", obj] + common + DEVICE_FLAGS
        else:
            cmd = [cc, "-x", "c++", "-c", src, "-o", obj, "-O3", "-std=c++17", "-fPIC", "-Wall"] + inc
        if verbose:
            print(" ".join(cmd), flush=True)
        cmds.append((cmd, name))
        objs.append(obj)
    running = []
    failed = []
    while cmds or running:
        while cmds and len(running) < max(1, jobs):
            cmd, name = cmds.pop(0)
            running.append((subprocess.Popen(cmd, stderr=subprocess.PIPE, text=True), name))
        p, name = running.pop(0)
        if not _finish(p, name):
            failed.append(name)
    if failed:
        raise RuntimeError("hipcc failed on " + ", ".join(failed))
    link = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", LIB + ".tmp"] + sorted(objs) + ["-lpthread"]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def _finish(p, name) -> bool:
    _, err = p.communicate()
    noise = "is not a recognized feature for this target"
    msgs = [l for l in err.splitlines() if noise not in l]
    if msgs:
        sys.stderr.write("\n".join(msgs) + "\n")
    return p.returncode == 0


if __name__ == "__main__":
    print(build(verbose=True))
