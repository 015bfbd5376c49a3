"""Build libbra.so (the HIP kernels and the C-ABI front end) for gfx950.

Run ``python -m vision_transformer_dynamic_region_amd.build`` (or call
``build()``); the library is written next to this file so that it travels
with the source tree.  Always recompiles.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libbra.so")
SOURCES = ["route_kernels.hip", "attend_kernels.hip", "region_kernels.hip", "image_kernels.hip",
           "module_kernels.hip",
           "block_kernels.hip", "mlp_kernels.hip", "backward_kernels.hip",
           "scratch.hip", "host_plan.cpp", "bra_api.cpp"]
# per-file extra flags: the attention and MLP files assume finite, non-NaN
# data (NaN inputs give unspecified outputs) so that max/min need no NaN
# quieting, and keep MFMA accumulators in ordinary VGPRs next to the
# softmax / GELU arithmetic
EXTRA_FLAGS = {
    "attend_kernels.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "region_kernels.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "image_kernels.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "backward_kernels.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "mlp_kernels.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}
ARCH = "gfx950"

HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed-fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libbra)")


def build(verbose: bool = False) -> str:
    cc = hipcc()
    tmpdir = os.path.join(HERE, "_build")
    os.makedirs(tmpdir, exist_ok=True)
    objs, procs = [], []
    # one compiler process per source, all at once (a handful of files)
    for src in SOURCES:
        obj = os.path.join(tmpdir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmd = [cc, *HIP_FLAGS, *EXTRA_FLAGS.get(src, []), *lang, "-c", os.path.join(CSRC, src),
               "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd)))
        objs.append(obj)
    failed = [src for src, p in procs if p.wait() != 0]
    if failed:
        raise RuntimeError(f"hipcc failed on {', '.join(failed)}")
    tmp = LIB + ".tmp"
    cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
