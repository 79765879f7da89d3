"""Build libkda.so (the HIP kernels and the C ABI) in-tree for gfx950.

Usage: python -m linear_attention_rule_amd.build   (or build() from Python).
Always recompiles; the output lands next to this file as libkda.so.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkda.so")
ARCH = "gfx950"

SOURCES = ["kda_api.cpp", "kda_verify.hip", "kda_commit.hip", "kda_norm.hip", "kda_conv.hip",
           "kda_prefill_intra.hip", "kda_prefill_scan.hip", "kda_scratch.hip"]

# Per-source additions (none today).  The intra kernel used the ILP-first scheduler while
# it ran two workgroups per CU; at three (168 VGPRs) the default scheduler fits without
# spills, and the ILP one cannot allocate registers under that limit.
EXTRA_FLAGS: dict = {}

# Packed fp32 VALU forms are disabled on purpose: plain fp32 code only.
HIP_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: the kernels post-process every accumulator tile
    # with VALU code, and the AGPR form would copy each one back and forth.
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libkda)")


def build(verbose: bool = False) -> str:
    """Compile every source (in parallel) and link libkda.so; returns its path."""
    from concurrent.futures import ThreadPoolExecutor

    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    cc = hipcc()

    def compile_one(src):
        obj = os.path.join(objdir, src + ".o")
        # The C ABI source includes HIP headers and launches kernels: hip mode for all.
        cmd = [cc, *HIP_FLAGS, *EXTRA_FLAGS.get(src, []), "-x", "hip", "-c",
               os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        return obj

    jobs = max(1, min(len(SOURCES), os.cpu_count() or 1, 8))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
