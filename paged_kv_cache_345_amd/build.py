"""Build libpagedkv.so for gfx950 with hipcc, in-tree.

    python -m paged_kv_cache_345_amd.build

Every source is compiled to an object under ``_build/`` (in parallel) and linked
into ``paged_kv_cache_345_amd/libpagedkv.so``.  Device code is built with the
packed-fp32 instructions disabled.
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
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpagedkv.so")
ARCH = "gfx950"

SOURCES = ["api.hip", "decode.hip", "prefill.hip", "plan.hip", "cache_ops.hip", "step.hip", "block_manager.cpp"]

COMMON = ["-O3", "-std=c++20", "-fPIC", "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}"]
HIP_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-fgpu-flush-denormals-to-zero", "-munsafe-fp-atomics"]
# Extra flags per source file.  prefill.hip: the compiler's resource report,
# checked below.
PER_SOURCE_FLAGS: dict = {"prefill.hip": ["-Rpass-analysis=kernel-resource-usage"]}

# Kernels that must use no per-lane scratch memory.  The prefill kernel keeps
# the vector-memory counter itself around its LDS loads; a spill would add
# scratch loads and stores to its step loop that the counts do not include.
NO_SCRATCH = {"prefill.hip": "prefill_kernel"}


def _check_no_scratch(src: str, remarks: str) -> None:
    """Fail the build when a kernel listed in NO_SCRATCH reports scratch use."""
    kernel = NO_SCRATCH.get(src)
    if not kernel:
        return
    seen, fn = 0, None
    for line in remarks.splitlines():
        if "Function Name:" in line:
            fn = line.split("Function Name:")[1].split()[0]
        elif "ScratchSize [bytes/lane]:" in line and fn and kernel in fn:
            seen += 1
            size = int(line.split("ScratchSize [bytes/lane]:")[1].split()[0])
            if size != 0:
                raise RuntimeError(f"{fn} uses {size} bytes of scratch per lane; its step loop must not "
                                   f"(see the vector-memory counting in {src})")
    if seen == 0:
        raise RuntimeError(f"no resource report for {kernel} in the output of {src}")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    if src.endswith(".hip"):
        cmd = [hipcc(), "-x", "hip", *HIP_FLAGS, *PER_SOURCE_FLAGS.get(src, []), *COMMON, "-c", path, "-o", obj]
    else:
        cmd = ["g++", *COMMON, "-c", path, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{r.stdout}\n{r.stderr}")
    _check_no_scratch(src, r.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking libpagedkv.so failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
