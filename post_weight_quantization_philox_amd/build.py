"""Build libgsq.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Usage: ``python -m post_weight_quantization_philox_amd.build`` (or call
:func:`build`). Objects go to ``_build/`` at the repository root and the shared
library into this package directory, where the binding loads it.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libgsq.so")
SOURCES = ["relax.hip", "gemm.hip", "fused.hip", "gptq.hip", "block.hip", "abi.hip"]
ARCH = os.environ.get("GSQ_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # Packed fp32 (v_pk_*_f32) is disabled for the whole library.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]

# Per-source flags. The products' K-loop carries 64 MFMA accumulator tuples
# from one K-step to the next; under the default scheduler the register
# allocator shuffles some of them between register files every step, which
# the iterative ILP strategy avoids (every accumulator stays in its AGPRs).
EXTRA_FLAGS = {
    "gemm.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"],
}


def _hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found: the GSQ library needs ROCm's hipcc to build")
    return exe


def build(verbose: bool = False) -> str:
    """Compile every source and link ``libgsq.so``. Returns its path."""
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)

    def compile_one(src: str) -> str:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        cmd = [hipcc, *HIPCC_FLAGS, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
        if verbose:
            print(" ".join(cmd), file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
