"""Build libfa.so in-tree with hipcc for gfx950.

    python -m exact_attention_07_amd.build

Every call recompiles (a few seconds per source).  The library lands next to
this file, where exact_attention_07_amd.api loads it from.
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
LIB = os.path.join(HERE, "libfa.so")
SOURCES = ["fa_fwd.hip", "fa_bwd.hip", "fa_fwd_fp8.hip", "fa_fp8_prepare.hip", "fa_ceiling.hip", "fa_issue.hip", "fa_noalloc.hip", "fa_api.cpp"]
ARCH = "gfx950"

# Packed fp32 VALU instructions are kept out of the device code on purpose.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Forward kernels: matrix-core results in VGPRs (-amdgpu-mfma-vgpr-form).
# Where a forward kernel may use more than 256 registers per lane (head
# dimension 256, or one wave per SIMD where LDS limits the occupancy), the
# default keeps every MFMA result in AGPRs and copies the scores to VGPRs
# and back around the softmax work.  The backward kernels keep the default:
# their dK/dV accumulators are only ever MFMA operands and are best left in
# AGPRs.  Kernels that fit in 256 VGPRs compile to the same code either way.
EXTRA_FLAGS = {src: ["-mllvm", "-amdgpu-mfma-vgpr-form=1"] for src in ("fa_fwd.hip", "fa_fwd_fp8.hip")}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libfa.so)")


def build(verbose: bool = False) -> str:
    from concurrent.futures import ThreadPoolExecutor
    os.makedirs(os.path.join(HERE, "_build"), exist_ok=True)

    def compile_one(src):
        obj = os.path.join(HERE, "_build", src + ".o")
        cmd = [hipcc(), *HIP_FLAGS, *EXTRA_FLAGS.get(src, []), "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
        return obj

    with ThreadPoolExecutor(max_workers=min(len(SOURCES), 7)) as pool:
        objs = list(pool.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
