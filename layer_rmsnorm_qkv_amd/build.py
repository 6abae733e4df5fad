"""Build liblrq.so (all HIP sources under csrc/) for gfx950, in-tree.

    python -m layer_rmsnorm_qkv_amd.build          # or: python layer_rmsnorm_qkv_amd/build.py

Each translation unit is compiled with hipcc (-O3, --offload-arch=gfx950, packed fp32
instructions disabled) into ``_build/`` at the repository root, then linked into
``layer_rmsnorm_qkv_amd/liblrq.so``.  Always recompiles.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "liblrq.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else "hipcc")
CFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function", "-Wno-unused-variable"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the device-only target feature; drop that line
    out = "\n".join(ln for ln in r.stdout.splitlines() if "packed-fp32-ops" not in ln)
    return r.returncode, out


def build(verbose: bool = False, extra_flags=None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    flags = CFLAGS + list(extra_flags or [])

    def compile_one(src):
        obj = os.path.join(BUILD, os.path.basename(src) + ".o")
        rc, out = _run([HIPCC, *flags, "-c", src, "-o", obj])
        return src, obj, rc, out

    objs = []
    jobs = min(len(sources), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        for src, obj, rc, out in ex.map(compile_one, sources):
            if out.strip() and (verbose or rc != 0):
                print(out, file=sys.stderr)
            if rc != 0:
                raise RuntimeError(f"hipcc failed on {os.path.basename(src)}")
            objs.append(obj)
    tmp = LIB + ".tmp"
    rc, out = _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs])
    if rc != 0:
        print(out, file=sys.stderr)
        raise RuntimeError("link of liblrq.so failed")
    shutil.move(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
