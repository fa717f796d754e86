"""Builds libsink_attn.so (gfx950) in-tree with hipcc.

    python -m gqa_attention_sinks_attn_amd.build

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction
selection turned off (-packed-fp32-ops), and linked with the host C-ABI
layer into one shared library next to this file.
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
LIB = os.path.join(HERE, "libsink_attn.so")
SOURCES = ["api.cpp", "decode.hip", "decode_balanced.hip", "merge.hip", "noalloc.hip",
           "prefill.hip", "rope_append.hip", "verify.hip", "verify_tile.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, extra_flags=None) -> str:
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Wall", "-Wno-unused-result",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           # device code only: no NaN canonicalisation around fmaxf (IEEE
           # mode off); the kernels never depend on NaN semantics
           "-Xarch_device", "-fno-honor-nans", "-Xarch_device", "-mno-amdgpu-ieee",
           "-I", INCLUDE, "-I", CSRC]
    cmd += list(extra_flags or [])
    cmd += [os.path.join(CSRC, s) for s in SOURCES]
    cmd += ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
