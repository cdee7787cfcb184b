"""Build libqsa_amd.so in-tree: the HIP kernels for gfx950 plus the host-side
C ABI, linked into one shared library next to this file.

    python -m paged_top_indexer_amd.build
    python -m paged_top_indexer_amd.build --rev REV --out PATH

The second form builds the library of a git revision (its csrc/ and
include/) into PATH, e.g. the baseline of an A/B comparison (bench_ab.py).
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
# the read-ceiling probe, a measurement aid built apart from the method
PROBE_LIBRARY = os.path.join(HERE, "libqsa_probe.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
ARCH = "gfx950"

HIP_SOURCES = ["qsa_select.hip", "qsa_attn.hip", "qsa_metadata.hip", "qsa_noalloc.hip"]
PROBE_SOURCE = "qsa_probe.hip"
HOST_SOURCES = ["qsa_capi.cpp", "qsa_plan.cpp"]

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


def build(verbose: bool = False, csrc: str = CSRC, include: str | None = None,
          out: str = LIBRARY, build_dir: str = BUILD) -> str:
    """Compile every source and link the library (LIBRARY by default);
    returns its path."""
    os.makedirs(build_dir, exist_ok=True)
    inc = [f"-I{include}"] if include else []
    if csrc == CSRC:
        hip, host = HIP_SOURCES, HOST_SOURCES
        probe = os.path.join(build_dir, PROBE_SOURCE + ".o")
        _run([HIPCC, *HIP_FLAGS, "-c", os.path.join(csrc, PROBE_SOURCE), "-o", probe], verbose)
        _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", PROBE_LIBRARY + ".tmp",
              probe], verbose)
        os.replace(PROBE_LIBRARY + ".tmp", PROBE_LIBRARY)
    else:  # another revision's tree: whatever sources it has
        names = sorted(os.listdir(csrc))
        hip = [n for n in names if n.endswith(".hip") and n != PROBE_SOURCE]
        host = [n for n in names if n.endswith(".cpp")]
    jobs = []
    objs = []
    for src in hip:
        obj = os.path.join(build_dir, src + ".o")
        jobs.append([HIPCC, *HIP_FLAGS, *inc, "-c", os.path.join(csrc, src), "-o", obj])
        objs.append(obj)
    for src in host:
        obj = os.path.join(build_dir, src + ".o")
        jobs.append(["g++", *HOST_FLAGS, *inc, "-c", os.path.join(csrc, src), "-o", obj])
        objs.append(obj)
    with ThreadPoolExecutor(max_workers=min(4, len(jobs))) as pool:
        list(pool.map(lambda c: _run(c, verbose), jobs))
    tmp = out + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, out)
    return out


def build_revision(rev: str, out: str, verbose: bool = False) -> str:
    """Build the library of git revision `rev` (its csrc/ and include/
    trees, unpacked from `git archive`) into `out`."""
    import shutil
    import tempfile

    tmp = tempfile.mkdtemp(prefix="qsa_rev_")
    try:
        arch = subprocess.run(["git", "-C", ROOT, "archive", rev, "paged_top_indexer_amd/csrc",
                               "include"], capture_output=True, check=True).stdout
        subprocess.run(["tar", "-x", "-C", tmp], input=arch, check=True)
        os.makedirs(os.path.dirname(os.path.abspath(out)), exist_ok=True)
        return build(verbose, csrc=os.path.join(tmp, "paged_top_indexer_amd", "csrc"),
                     include=os.path.join(tmp, "include"), out=os.path.abspath(out),
                     build_dir=os.path.join(tmp, "_build"))
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


if __name__ == "__main__":
    import argparse

    ap = argparse.ArgumentParser()
    ap.add_argument("-v", action="store_true")
    ap.add_argument("--rev", help="build this git revision's library instead of the tree's")
    ap.add_argument("--out", help="output path (with --rev)")
    a = ap.parse_args()
    if a.rev:
        print(build_revision(a.rev, a.out or os.path.join(HERE, "_ablibs", f"libqsa_{a.rev}.so"),
                             a.v))
    else:
        print(build(verbose=a.v))
