"""Build of libgdn.so with hipcc for gfx950 (in-tree, next to this file), and
of libgdn_debug.so, the same sources with every kernel's LDS filled with a
NaN pattern before use (GDN_POISON_LDS=1): a test compares the two builds bit
for bit, so that a read of LDS that no code wrote shows up."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libgdn.so")
DEBUG_LIB = os.path.join(PKG, "libgdn_debug.so")

SOURCES = ["gdn_api.hip"]
HEADERS = ["gdn_common.hpp", "chunk_fwd_pipe.hpp", "chunk_vec.hpp", "recurrent_step.hpp", "split_combine.hpp", "scan_route.hpp"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # packed fp32 VALU forms are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: the kernels read every accumulator with VALU
    # ops, and AGPR<->VGPR copies would cost a 4-cycle VALU issue each
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def _inputs():
    files = [os.path.join(CSRC, f) for f in SOURCES + HEADERS]
    files.append(os.path.join(INCLUDE, "gdn.h"))
    return files


def is_stale() -> bool:
    for lib in (LIB, DEBUG_LIB):
        if not os.path.exists(lib):
            return True
        t = os.path.getmtime(lib)
        if any(os.path.getmtime(f) > t for f in _inputs()):
            return True
    return False


def _compile(out: str, defines, verbose: bool) -> None:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc] + HIPCC_FLAGS + defines + ["-I", INCLUDE, "-I", CSRC, "-o", tmp]
    cmd += [os.path.join(CSRC, f) for f in SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile every HIP source into libgdn.so and libgdn_debug.so (always
    recompiles)."""
    _compile(LIB, [], verbose)
    _compile(DEBUG_LIB, ["-DGDN_POISON_LDS=1"], verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
