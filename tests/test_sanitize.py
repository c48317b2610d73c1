"""AddressSanitizer and UndefinedBehaviorSanitizer runs of the host-side code (CPU only):

* the fp64 oracle, driven through every entry point on small shapes
  (tests/sanitize/oracle_driver.c, built with gcc);
* the C ABI's host code (argument validation, workspace layout), built into a copy of
  libhils.so with the sanitizers on the host side only and driven through every
  validation path (tests/sanitize/abi_driver.cpp); nothing reaches a device.

Any out-of-bounds access, use of freed memory or undefined operation aborts the driver."""
import glob
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    subprocess.check_call(["gcc", "-std=c99", "-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                           "-fno-omit-frame-pointer", "-o", exe, os.path.join(HERE, "oracle_driver.c"),
                           os.path.join(ROOT, "oracle", "hils_oracle.c"), "-lm"])
    out = subprocess.run([exe], env=dict(SAN_ENV, ASAN_OPTIONS="abort_on_error=1"), capture_output=True, text=True,
                         timeout=600)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "ok" in out.stdout


@pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc"), reason="needs hipcc")
def test_host_abi_under_asan_ubsan(tmp_path):
    lib = str(tmp_path / "libhils_san.so")
    srcs = sorted(glob.glob(os.path.join(ROOT, "long_context_chunk_amd", "csrc", "*.hip")))
    # the sanitizers apply to the host code only (each flag after -Xarch_host)
    subprocess.check_call(["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
                           "-Wno-unused-value", "-Wno-pass-failed", "-Xclang", "-target-feature", "-Xclang",
                           "-packed-fp32-ops", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
                           "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=all",
                           "-I", os.path.join(ROOT, "include")] + srcs + ["-o", lib],
                          stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    exe = str(tmp_path / "abi_driver")
    subprocess.check_call(["/opt/rocm/llvm/bin/clang++", "-std=c++17", "-g", "-O1", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=all", os.path.join(HERE, "abi_driver.cpp"), "-L", str(tmp_path),
                           "-lhils_san", "-Wl,-rpath," + str(tmp_path), "-o", exe])
    out = subprocess.run([exe], env=SAN_ENV, capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "host ABI sanitizer run: ok" in out.stdout
