"""Build libsaf.so (HIP kernels for gfx950 + the C-ABI host code) in-tree with hipcc.

Usage: python fixed_pattern_mixed_amd/build.py [-v]   (or __graft_entry__.build()).  Every call
recompiles.  (Run it by path: importing the package would load the library being rebuilt.)
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libsaf.so")
SOURCES = ["saf_api.cpp", "saf_pattern.hip", "saf_fwd.hip", "saf_bwd.hip", "saf_pattern_bwd.hip",
           "saf_calib.hip", "saf_fit.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
]

# per-file additions: the calibration kernels are vector-bound, and matrix products accumulated in
# AGPRs would cost one register read per score entry before the vector work
FILE_FLAGS = {"saf_calib.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def build(verbose: bool = False) -> str:
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(src, []), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                            text=True)))
    errors = []
    for src, p in procs:
        out, _ = p.communicate()
        if p.returncode != 0:
            errors.append("%s:\n%s" % (src, out))
        elif verbose and out.strip():
            print(out)
    if errors:
        raise RuntimeError("hipcc failed\n" + "\n".join(errors))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
