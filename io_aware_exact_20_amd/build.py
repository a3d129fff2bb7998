"""Build the gfx950 HIP library ``libfa.so`` in-tree with hipcc.

Every HIP translation unit is compiled for gfx950 only, with packed-fp32
instruction selection disabled; objects go to ``_build/`` and the shared
library next to this file.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libfa.so")
SOURCES = ["fa_api.cpp", "fa_fwd.hip", "fa_fwd_pp.hip", "fa_fwd_fp8.hip", "fa_bwd.hip", "fa_bwd16.hip",
           "fa_dq256.hip", "fa_dkdv16.hip", "fa_noalloc.hip"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(ROOT, "include")]


# Kernel sources: the inputs are finite by contract (infinities are still
# honoured, they carry the masks), so NaN-preserving canonicalisation of
# max() is not needed.  The forward kernels (16-bit and FP8), the dK/dV
# kernel and the dQ kernel at d = 32 to 128 select matrix-core results into
# VGPRs, so that the softmax and dS arithmetic reads them without AGPR
# copies; the d = 256 dQ kernel leaves them in AGPRs, which hold its output
# accumulators.
KERNEL_FLAGS = ["-fno-honor-nans"]
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
PER_SOURCE = {"fa_fwd.hip": KERNEL_FLAGS + VGPR_FORM, "fa_fwd_pp.hip": KERNEL_FLAGS + VGPR_FORM,
              "fa_fwd_fp8.hip": KERNEL_FLAGS + VGPR_FORM, "fa_bwd16.hip": KERNEL_FLAGS + VGPR_FORM,
              "fa_dq256.hip": KERNEL_FLAGS,
              "fa_dkdv16.hip": KERNEL_FLAGS + VGPR_FORM}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *PER_SOURCE.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, err))
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build() -> str:
    """Compile every source and link ``libfa.so``; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    subprocess.run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs],
                   check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
