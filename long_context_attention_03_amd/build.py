"""Build the HIP library (libcsah.so) in-tree for gfx950 with hipcc.

Each .hip file under csrc/ is compiled to an object and the objects are linked into one shared
library next to this file. Packed-FP32 VALU instructions are disabled on purpose.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libcsah.so")
BUILD = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-function", "-Wno-unused-variable",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]
# Per-file code generation options. attend.hip: matrix-core accumulators live in ordinary VGPRs
# (the kernels rescale them with vector multiplies; held in AGPRs, every tile copied all of them
# out and back around that rarely taken branch).
FILE_FLAGS = {
    "attend.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(ln for ln in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in ln)
    if r.returncode != 0:
        sys.stderr.write(out + "\n")
        raise RuntimeError(f"command failed: {' '.join(cmd)}")
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = []
    procs = []
    for s in srcs:
        o = os.path.join(BUILD, os.path.basename(s) + ".o")
        cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(os.path.basename(s), []), "-c", s, "-o", o]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                            text=True)))
        objs.append(o)
    failed = []
    for cmd, p in procs:
        out, _ = p.communicate()
        out = "\n".join(ln for ln in out.splitlines()
                        if "packed-fp32-ops' is not a recognized feature" not in ln)
        if verbose and out.strip():
            print(out)
        if p.returncode != 0:
            sys.stderr.write(out + "\n")
            failed.append(cmd[-3])
    if failed:
        raise RuntimeError(f"hipcc failed for: {failed}")
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
