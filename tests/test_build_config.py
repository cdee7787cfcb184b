"""The repository's own build targets gfx950 only: every device code object
bundled into libqsa_amd.so (one bundle per HIP source) and into
libqsa_probe.so is for amdgcn-amd-amdhsa--gfx950, as the ROCm offload
bundler lists them, and the HIP sources are compiled with packed-fp32
instructions disabled."""

import os
import shutil
import subprocess

import pytest

from paged_top_indexer_amd import build

ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
BUNDLER = os.path.join(ROCM, "llvm", "bin", "clang-offload-bundler")
OBJCOPY = os.path.join(ROCM, "llvm", "bin", "llvm-objcopy")
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def bundle_targets(library: str, tmp_path) -> list[list[str]]:
    """The offload targets of every bundle in the library's .hip_fatbin
    section, as clang-offload-bundler --list prints them."""
    section = tmp_path / (os.path.basename(library) + ".fatbin")
    subprocess.run([OBJCOPY, f"--dump-section=.hip_fatbin={section}", library,
                    str(tmp_path / "stripped.so")], check=True, capture_output=True)
    data = section.read_bytes()
    starts = []
    at = data.find(MAGIC)
    while at >= 0:
        starts.append(at)
        at = data.find(MAGIC, at + len(MAGIC))
    out = []
    for i, s in enumerate(starts):
        part = tmp_path / f"bundle{i}.bin"
        part.write_bytes(data[s:starts[i + 1] if i + 1 < len(starts) else len(data)])
        res = subprocess.run([BUNDLER, "--list", "--type=o", f"--input={part}"],
                             capture_output=True, text=True, check=True)
        out.append(sorted(res.stdout.split()))
    return out


@pytest.mark.parametrize("library,sources", [(build.LIBRARY, len(build.HIP_SOURCES)),
                                             (build.PROBE_LIBRARY, 1)],
                         ids=["libqsa_amd", "libqsa_probe"])
def test_device_code_is_gfx950_only(library, sources, tmp_path):
    if not (os.path.exists(BUNDLER) and os.path.exists(OBJCOPY)):
        pytest.skip("ROCm offload bundler not found")
    if not os.path.exists(library):
        build.build()
    bundles = bundle_targets(library, tmp_path)
    assert len(bundles) == sources, f"{len(bundles)} bundles for {sources} HIP sources"
    for targets in bundles:
        assert targets == ["hipv4-amdgcn-amd-amdhsa--gfx950", "host-x86_64-unknown-linux-gnu-"], \
            targets


def test_build_flags():
    assert build.ARCH == "gfx950"
    assert "--offload-arch=gfx950" in build.HIP_FLAGS
    assert not any(f.startswith("--offload-arch") and f != "--offload-arch=gfx950"
                   for f in build.HIP_FLAGS)
    flags = " ".join(build.HIP_FLAGS)
    assert "-target-feature -Xclang -packed-fp32-ops" in flags
    assert shutil.which(build.HIPCC) or os.path.exists(build.HIPCC)
