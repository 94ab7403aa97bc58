"""Build the HIP library libfp8amax.so in-tree for gfx950 (hipcc, no JIT cache).

Run as ``python -m fp8_quantized_gemm_amax_amd.build``; ``__graft_entry__.build()``
calls :func:`build_library`.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libfp8amax.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = ["api.hip", "quantize.hip", "gemm.hip", "gemv.hip"]
OBJ_DIR = os.path.join(PKG, "_build")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # exact IEEE float32 arithmetic in the quantizer: no contraction, no fast math
    "-ffp-contract=off",
    # no packed fp32 (v_pk_*_f32) instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs: the blockwise epilogue reads every slab's partial sums with
    # VALU FMAs, which cannot take AGPR operands
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wno-unused-command-line-argument",
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libfp8amax.so)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}: {' '.join(cmd[-3:])}")


def build_library(verbose=False):
    """Compile every HIP source to an object (in parallel), then link LIB_PATH.  Always
    recompiles."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    objs = [os.path.join(OBJ_DIR, os.path.splitext(src)[0] + ".o") for src in SOURCES]
    cmds = [[hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", "-o", obj, os.path.join(CSRC, src)]
            for src, obj in zip(SOURCES, objs)]
    workers = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(workers) as pool:
        list(pool.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB_PATH + ".tmp"
    _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build_library(verbose=True))
