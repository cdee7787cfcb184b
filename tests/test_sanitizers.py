"""The CPU oracle and the host-side C ABI code (argument validation and
launch planning: qsa_capi.cpp, qsa_plan.cpp) built with AddressSanitizer and
UndefinedBehaviorSanitizer, then driven by the oracle pins and the host ABI
tests in a child process.  The host code is linked with stand-ins for the
kernel launchers (tests/c/launch_stubs.cpp) that abort, so a validation
path that reached a launch would fail the run too.  Built with gcc/g++ only:
no device code is involved."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_top_indexer_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
       "-fno-omit-frame-pointer", "-g", "-O1", "-fPIC", "-shared"]

RUNNER = r'''
import sys
sys.path.insert(0, {root!r})
from paged_top_indexer_amd import _binding
_binding.use_library({host!r})
import oracle
oracle._DEFAULT = oracle.Oracle({orc!r})
import pytest
sys.exit(pytest.main(["-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu", "-k", "not probe",
                      {pins!r}, {capi!r}]))
'''


def test_oracle_and_host_code_under_asan_and_ubsan(tmp_path):
    for tool in ("gcc", "g++"):
        if shutil.which(tool) is None:
            pytest.skip(f"{tool} not found")
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("libasan not found")
    orc = str(tmp_path / "libqsa_oracle_san.so")
    host = str(tmp_path / "libqsa_host_san.so")
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Wextra", *SAN, "-DQSA_ORACLE_MUTANT=0",
                    os.path.join(ROOT, "oracle", "qsa_oracle.c"), "-lm", "-o", orc], check=True)
    subprocess.run(["g++", "-std=c++17", "-Wall", "-Wextra", *SAN,
                    f"-I{os.path.join(ROOT, 'include')}", os.path.join(CSRC, "qsa_capi.cpp"),
                    os.path.join(CSRC, "qsa_plan.cpp"),
                    os.path.join(ROOT, "tests", "c", "launch_stubs.cpp"), "-o", host], check=True)
    for lib in (orc, host):  # really instrumented
        syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
        assert "__asan_report_" in syms and "__ubsan_handle_" in syms, lib
    runner = tmp_path / "run.py"
    runner.write_text(RUNNER.format(root=ROOT, host=host, orc=orc,
                                    pins=os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                                    capi=os.path.join(ROOT, "tests", "test_capi_host.py")))
    env = dict(os.environ, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:allocator_may_return_null=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([sys.executable, str(runner)], cwd=ROOT, env=env, capture_output=True,
                         text=True, timeout=900)
    log = res.stdout + res.stderr
    assert res.returncode == 0, log[-4000:]
    assert "ERROR: AddressSanitizer" not in log and "runtime error:" not in log, log[-4000:]
    assert " passed" in res.stdout
