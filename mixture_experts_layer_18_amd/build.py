"""Build the gfx950 HIP library (in-tree) with hipcc.

    python -m mixture_experts_layer_18_amd.build

Produces mixture_experts_layer_18_amd/libmoe_mi355x.so from csrc/*.hip.
Every source is compiled for gfx950 only, with packed-fp32 instructions
disabled (-packed-fp32-ops), and linked into one shared library that exports
the C ABI declared in include/moe.h.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libmoe_mi355x.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
BUILD_DIR = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _compile_one(src, obj, extra):
    cmd = [HIPCC, *FLAGS, *extra, "-c", src, "-o", obj]
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT), cmd


def build(verbose: bool = False, extra=()) -> str:
    """Compile every csrc/*.hip and link the shared library.  Always rebuilds."""
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD_DIR, exist_ok=True)
    t0 = time.time()
    procs = []
    objs = []
    for src in sources():
        obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
        objs.append(obj)
        procs.append((src, *_compile_one(src, obj, list(extra))))
    failed = False
    for src, p, cmd in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the packed-fp32 feature; that is harmless
        lines = [l for l in text.splitlines() if "packed-fp32-ops" not in l and l.strip()]
        if p.returncode != 0:
            failed = True
            sys.stderr.write(f"FAILED: {' '.join(cmd)}\n" + "\n".join(lines) + "\n")
        elif verbose and lines:
            sys.stderr.write("\n".join(lines) + "\n")
    if failed:
        raise RuntimeError("HIP compilation failed")
    tmp = LIB_PATH + ".tmp"
    link = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(link, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    shutil.move(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH} in {time.time() - t0:.1f}s")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
