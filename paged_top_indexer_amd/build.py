"""Build libqsa_amd.so in-tree: the HIP kernels for gfx950 plus the host-side
C ABI, linked into one shared library next to this file.

    python -m paged_top_indexer_amd.build
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIBRARY = os.path.join(HERE, "libqsa_amd.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
ARCH = "gfx950"

HIP_SOURCES = ["qsa_select.hip", "qsa_attn.hip", "qsa_metadata.hip", "qsa_noalloc.hip",
               "qsa_probe.hip"]
HOST_SOURCES = ["qsa_capi.cpp", "qsa_select_plan.cpp"]

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-munsafe-fp-atomics",
    # no packed-fp32 instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra",
              f"-I{os.path.join(ROOT, 'include')}"]


def _run(cmd: list[str], verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = (res.stdout + res.stderr).splitlines()
    # hipcc's host pass does not know the packed-fp32 feature; harmless
    noise = "is not a recognized feature for this target"
    msgs = [line for line in out if noise not in line]
    if msgs and (verbose or res.returncode):
        print("\n".join(msgs), file=sys.stderr, flush=True)
    if res.returncode:
        raise RuntimeError(f"build step failed: {' '.join(cmd)}")


def build(verbose: bool = False) -> str:
    """Compile every source and link LIBRARY; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append(["g++", *HOST_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with ThreadPoolExecutor(max_workers=min(4, len(jobs))) as pool:
        list(pool.map(lambda c: _run(c, verbose), jobs))
    tmp = LIBRARY + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
