"""Build liblatentmoe.so (the HIP kernels + C ABI) for gfx950 with hipcc.

The library has one translation unit per part of the ABI (the forward entry
points and the backward ones); they compile in parallel and link into one
shared object.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "liblatentmoe.so")
UNITS = ("forward.hip", "backward.hip")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 vector ops stay off (hipcc's host pass warns that it does
    # not know the feature; harmless)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def build(verbose: bool = False) -> str:
    with tempfile.TemporaryDirectory(prefix="lmoe_build_") as tmpdir:
        objs, procs = [], []
        for unit in UNITS:
            obj = os.path.join(tmpdir, unit.replace(".hip", ".o"))
            cmd = ["hipcc", *HIPCC_FLAGS, "-c", "-o", obj, os.path.join(CSRC, unit)]
            procs.append((unit, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
            objs.append(obj)
        failed = []
        for unit, pr in procs:
            out, err = pr.communicate()
            if pr.returncode != 0:
                failed.append(unit)
                sys.stderr.write(out + err)
            elif verbose:
                sys.stderr.write(err)
        if failed:
            raise RuntimeError(f"hipcc failed for {', '.join(failed)}")
        tmp = LIB + ".tmp"
        r = subprocess.run(["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs],
                           capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError("linking liblatentmoe.so failed")
        os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
