"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

fa_api.cpp and the launch plans (fa_plan.cpp) are built with g++ into a host-only
library whose kernel launchers are counting stand-ins (tests/host_abi/stub_launch.cpp),
and tests/test_abi_cpu.py runs against it in a child process with the sanitizer
runtime preloaded.  Any invalid memory access or undefined behaviour in the argument
checks aborts that process and fails this test.  No GPU and no HIP runtime are used.
"""
import os
import shutil
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
CSRC = ROOT / "exact_io_aware_20_amd" / "csrc"
OUT = ROOT / "_build" / "libfa_host_asan.so"


def _gxx():
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    return gxx


def build_host_asan() -> Path:
    gxx = _gxx()
    OUT.parent.mkdir(exist_ok=True)
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fPIC", "-shared",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", f"-I{ROOT / 'include'}",
           str(CSRC / "fa_api.cpp"), str(CSRC / "fa_plan.cpp"), str(ROOT / "tests" / "host_abi" / "stub_launch.cpp"),
           "-o", str(OUT)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return OUT


def test_abi_checks_clean_under_asan_and_ubsan():
    lib = build_host_asan()
    asan = subprocess.run([_gxx(), "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    assert os.path.isabs(asan), asan
    env = dict(os.environ)
    env.update({"FA_MI355X_LIB": str(lib), "LD_PRELOAD": asan,
                "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
                "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"})
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        str(ROOT / "tests" / "test_abi_cpu.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " skipped" not in out.splitlines()[-1] or "passed" in out.splitlines()[-1]
