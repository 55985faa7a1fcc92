"""Build libmoeq4.so (all HIP sources, gfx950) next to this file.

Each source compiles to its own object (in parallel, with its own scheduling flags) and the
objects link into one shared library.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoeq4.so")
SOURCES = ["api.hip", "route.hip", "gemm.hip", "decode.hip", "misc.hip", "pack.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed fp32 arithmetic in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: the GEMM's register budget (two workgroups per
    # CU) fits without spills only in this form
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    # atomics stay plain: the aggregating rewrite consumes the result at once,
    # which would stall the GEMM's work-queue fetch that is meant to overlap
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-Wall", "-Wno-unused-function",
]

# iterative ILP scheduling keeps the GEMM's operand reads for a k slice grouped ahead of the
# MFMAs that use them (the default scheduler sinks each read next to its use and waits for it
# there): measured 4 us faster on the down GEMM and 1 us on routing, gate/up level
ILP = ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"]
PER_SOURCE = {"gemm.hip": ILP, "route.hip": ILP}


# Host code checked by AddressSanitizer and UndefinedBehaviorSanitizer (the GPU code is
# built as usual): every sanitizer flag is restricted to the host pass.  The library
# leaves the sanitizer runtime to the executable that loads it.
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-g"]
# Device-side index checks that record what they catch in a status word (moe_debug_status)
DEBUG = ["-DMOE_DEBUG"]


def build(verbose: bool = False, sanitize: bool = False, debug: bool = False,
          out: str = None) -> str:
    """Compile every source and link the library (default: libmoeq4.so next to this file).
    sanitize: host code with ASan + UBSan; debug: device index checks (MOE_DEBUG)."""
    lib = out or LIB
    extra = (SANITIZE if sanitize else []) + (DEBUG if debug else [])
    with tempfile.TemporaryDirectory(prefix="moeq4_") as tmpdir:
        def compile_one(src):
            obj = os.path.join(tmpdir, src.replace(".hip", ".o"))
            cmd = [HIPCC, *FLAGS, *PER_SOURCE.get(src, []), *extra, "-c", "-o", obj,
                   os.path.join(CSRC, src)]
            if verbose:
                print(" ".join(cmd), flush=True)
            subprocess.check_call(cmd)
            return obj

        with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as pool:
            objs = list(pool.map(compile_one, SOURCES))
        tmp = lib + ".tmp"
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
