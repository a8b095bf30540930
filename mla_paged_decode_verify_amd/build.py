"""Build the HIP library libmla_verify.so in-tree for gfx950 with hipcc.

    python mla_paged_decode_verify_amd/build.py

Every call recompiles. The shared library lands next to this file so that the
Python binding (and anything that copies the source tree) finds it.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libmla_verify.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
ARCH = "gfx950"

SOURCES = ["api.cpp", "plan.hip", "attn_bf16.hip", "attn_fp8.hip", "attn_persist.hip", "merge.hip",
           "scratch.hip"]

# Packed fp32 instructions are switched off: hipcc -O3 would otherwise form
# them from plain float code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Per-source extras. The attention kernels keep their 128-register output
# accumulators in VGPRs (they rescale them with plain VALU multiplies; AGPR
# copies would cost 256 moves a tile) and the query fragments in AGPRs.
_ATTN = ["-mllvm", "-amdgpu-mfma-vgpr-form", "-fno-honor-nans"]
SOURCE_FLAGS = {"attn_bf16.hip": _ATTN, "attn_fp8.hip": _ATTN, "attn_persist.hip": _ATTN}
COMMON_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
                "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l and "is not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False, resource_usage: bool = False) -> str:
    """Compile all sources and link libmla_verify.so; return its path."""
    cc = hipcc()
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        cmd = [cc, *COMMON_FLAGS, *DEVICE_FLAGS, *SOURCE_FLAGS.get(src, []),
               "-c", os.path.join(CSRC, src), "-o", obj]
        if resource_usage and src.endswith(".hip"):
            cmd += ["-Rpass-analysis=kernel-resource-usage"]
        _run(cmd, verbose or resource_usage)
        objs.append(obj)
    tmp = LIB_PATH + ".tmp"
    _run([cc, "-shared", f"--offload-arch={ARCH}", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True, resource_usage="--usage" in sys.argv))
