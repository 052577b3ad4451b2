"""Build libgdn.so (gfx950) from csrc/*.hip with hipcc, in place.

Each .hip file compiles to its own object (in parallel), then one shared
library is linked.  Flags: -O3, gfx950 only, packed-fp32 instructions off,
MFMA results in ordinary VGPRs (the accumulators are read by vector ALU code
every chunk; keeping them out of the accumulation registers saves the copies).
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libgdn.so")
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-mfma-vgpr-form",
         "-Wall", "-Wno-unused-function", "-I" + os.path.join(ROOT, "include")]


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    r = subprocess.run([HIPCC, *FLAGS, "-c", src, "-o", obj], capture_output=True, text=True)
    noise = "unknown target feature"  # host pass does not know the gfx feature
    msgs = [l for l in (r.stdout + r.stderr).splitlines() if noise not in l and "packed-fp32" not in l]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, "\n".join(msgs)))
    if msgs:
        sys.stderr.write("\n".join(msgs) + "\n")
    return obj


def build(jobs: int | None = None) -> str:
    os.makedirs(OBJ, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = jobs or min(len(srcs), os.cpu_count() or 4, 8)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    subprocess.run([HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, *objs, "-o", tmp],
                   check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
