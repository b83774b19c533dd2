"""Build libpa.so in-tree with hipcc for gfx950.

    python -m paged_kv_cache_41_amd.build

Every HIP source under csrc/ goes into one shared library next to this file.
Packed fp32 instructions are disabled on the device side (the host pass warns
that it does not know the feature; that is harmless).
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libpa.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-shared", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         # keep uniform-address atomics as written: the optimizer's rewrite reads the
         # result right after the atomic, which drains every load in flight
         "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
         # matrix-core accumulators in the vector registers: no moves between the vector
         # and accumulation register files around every product (the verify step with
         # groups of two query blocks runs 7% faster; decode 0.5-1%)
         "-mllvm", "-amdgpu-mfma-vgpr-form=1",
         "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]


def build(verbose: bool = False) -> str:
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, *FLAGS, *sources, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "not a recognized feature for this target"
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if noise not in l]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
