"""Build libtpmlp.so (the C-ABI library and its gfx950 kernels) in-tree with hipcc.

    python megatron_tensor_transformer_shard_amd/build_lib.py [-v]

(run as a file: importing the package loads the library, which may not be
built yet or may be out of date)

Objects go to <package>/_build/, the library to <package>/libtpmlp.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(PKG_DIR, "_build")
LIB_NAME = "libtpmlp.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)

SOURCES = ["gemm_bf16.hip", "gemm_e4m3.hip", "partial_sum.hip", "attention.hip", "bias_grad.hip",
           "abi.cpp"]
ARCH = "gfx950"

# Packed-fp32 VALU instructions are disabled for the device code; hipcc's host
# pass warns that it does not know the feature, which is harmless. The GEMM
# k-steps are fully unrolled loops of up to 64 MFMAs with their interleaved
# loads; clang's default size limit for `#pragma unroll` would leave them
# rolled, and the accumulator arrays would then live in scratch memory.
CFLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-mcode-object-version=5", "-fPIC",
    "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-pragma-unroll-threshold=1000000",
]

# Per-source flags. The attention kernel rescales its fp32 output accumulators
# with VALU multiplies after every key block; MFMAs in the VGPR form keep them
# in VGPRs, where the accumulator-register form would copy all of them out of
# and back into AGPRs each time.
SOURCE_FLAGS = {"attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libtpmlp.so)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, file=sys.stderr)
    return r


def build(verbose: bool = False, extra_flags=None, jobs: int = 4) -> str:
    """Compile every source and link libtpmlp.so. Always rebuilds. Returns the path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    flags = CFLAGS + list(extra_flags or [])
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        lang = ["-x", "hip"]
        cmds.append([hipcc, *lang, *flags, *SOURCE_FLAGS.get(src, []), "-I", CSRC, "-c",
                     os.path.join(CSRC, src), "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB_PATH + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
