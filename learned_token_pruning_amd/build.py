"""Builds libtokengate.so (HIP, gfx950 only) in-tree.

    python -m learned_token_pruning_amd.build

Every .hip source under csrc/ is compiled to an object under _build/ (in
parallel), then linked into learned_token_pruning_amd/libtokengate.so.  The
library links the HIP runtime by soname, so inside a process that imported
torch first it binds to the runtime torch already loaded.
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
LIB = os.path.join(PKG, "libtokengate.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
# Packed fp32 VALU ops are turned off for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Wno-unused-function"]
# Per-source extras.  The attention kernel takes row maxima of MFMA results;
# without NaN semantics fmaxf needs no canonicalising pass over its inputs
# (NaN inputs to attention give unspecified outputs).
# The backward kernels hold more live values than the 256 architectural VGPRs
# of one wave: keeping MFMA results in VGPRs (AGPRs only as spill space) avoids
# copying accumulators between the two register files around every product.
FILE_FLAGS = {"gated_attention.hip": ["-fno-honor-nans"],
              "gated_attention_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(ln for ln in r.stdout.splitlines() if "packed-fp32-ops" not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = []
    cmds = []
    for src in sources:
        obj = os.path.join(BUILD, os.path.basename(src) + ".o")
        objs.append(obj)
        cmds.append([HIPCC, *COMMON, *DEVICE_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj])
    workers = min(len(cmds), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(workers) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
