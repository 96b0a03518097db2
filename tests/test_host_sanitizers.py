"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The C-ABI layer's validation and size arithmetic (csrc/fa_api.cpp, with the
workspace layouts and split rules of csrc/fa_internal.hpp) is compiled for
the host with clang and both sanitizers, with the kernel launchers replaced by
recording stubs (tests/host_sanitize_api.cpp), and run through the argument
checks, workspace carving, dropout threshold and scale, decode splits and the
failed-launch path.  The oracle's C Philox (oracle/philox_ref.c) is built the
same way and run on the published known-answer vectors.  No device code is
built: the sanitizers apply to host code only."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests")
CLANG = "/opt/rocm/llvm/bin/clang"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _clang(cxx: bool) -> str:
    exe = CLANG + ("++" if cxx else "")
    if os.path.exists(exe):
        return exe
    found = shutil.which("clang++" if cxx else "clang")
    if not found:
        pytest.skip("clang not available")
    return found


def _build_and_run(cmd, exe, expect):
    b = subprocess.run(cmd, capture_output=True, text=True)
    assert b.returncode == 0, b.stderr[-3000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=ENV)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    assert expect in r.stdout
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr


def test_abi_layer_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "host_sanitize_api")
    cmd = [_clang(True), "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", "/opt/rocm/include", "-o", exe, os.path.join(HERE, "host_sanitize_api.cpp"),
           os.path.join(ROOT, "io_aware_exact_tiled_amd", "csrc", "fa_api.cpp")]
    _build_and_run(cmd, exe, "host sanitize ok")


def test_oracle_philox_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "host_sanitize_philox")
    cmd = [_clang(False), "-std=c99", *SAN, "-o", exe, os.path.join(HERE, "host_sanitize_philox.c"),
           os.path.join(ROOT, "oracle", "philox_ref.c")]
    _build_and_run(cmd, exe, "philox sanitize ok")
