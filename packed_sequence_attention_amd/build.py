"""Builds libblockdiag.so in-tree for gfx950 with hipcc.

Every HIP source is compiled to an object under ``_build/`` (in parallel),
then linked into ``packed_sequence_attention_amd/libblockdiag.so``.  HIP code
is compiled with packed-fp32 instructions disabled.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libblockdiag.so")
ARCH = "gfx950"

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", os.path.join(ROOT, "include"),
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall", "-Wno-unused-function"]


# Per-source extra flags.  The backward kernel keeps five matrix-core
# accumulators live per iteration; letting the backend pick the accumulator
# register file per instruction makes it split the dK/dV accumulators between
# AGPRs and VGPRs and copy them every iteration, so that file uses the VGPR
# form of the MFMA instructions (AGPRs then only hold spilled values).
# The head_dim 64 instantiation of that kernel is also built with the
# max-ILP scheduler (measured faster there, slower at head_dim 128).
# The dQ kernel file takes the VGPR form too: at head_dim 256 (one wave per
# SIMD, 512 registers) the default kept one of the Q / dO fragment arrays in
# AGPRs and copied it back before every product (about four copies per
# matrix instruction in the loop); with the VGPR form the loop holds 41
# copies for 96 products and the kernel runs 17 % faster.  Its head_dim 64
# and 128 code is the same either way.  (The head_dim 256 dK/dV kernel
# measured slower with it.)
EXTRA = {
    "bwd_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "bwd_dq.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "bwd_dkdv64.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-mllvm", "-amdgpu-sched-strategy=max-ilp"],
}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, *EXTRA.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    return obj, out


def build_library(verbose=False, jobs=None):
    """Compile every source and link libblockdiag.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), 8)
    with cf.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_compile, srcs))
    for obj, out in results:
        if verbose and out.strip():
            print(out)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + [o for o, _ in results]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose=True))
