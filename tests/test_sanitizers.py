"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

- The fp64 oracle and the input generator are compiled with both sanitizers
  together with tests/c/sanitize_host.c and run on small inputs through every
  exported function.
- libattnres is compiled with the sanitizers on its host code only (argument
  validation, range and overlap checks; the GPU code is built as usual but
  never runs) and driven through refusal paths of every entry point, each of
  which must return its documented status before any HIP call.

Both builds go to a temporary directory; nothing here uses a GPU."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "c", "sanitize_host.c")
SAN_FLAGS = ["-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _run(cmd, **kw):
    r = subprocess.run([str(c) for c in cmd], capture_output=True, text=True, **kw)
    return r


def test_oracle_and_generator_are_clean(tmp_path):
    exe = tmp_path / "sanitize_oracle"
    r = _run(["gcc", "-std=c11", "-fsanitize=address,undefined", *SAN_FLAGS, "-ffp-contract=off", "-DORACLE_PART",
              "-o", exe, DRIVER, os.path.join(ROOT, "oracle", "attnres_oracle.c"),
              os.path.join(ROOT, "synth", "synth.c"), "-lm"])
    assert r.returncode == 0, r.stderr
    r = _run([exe], env={**os.environ, "ASAN_OPTIONS": "detect_leaks=1", "UBSAN_OPTIONS": "print_stacktrace=1"})
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr


@pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc"), reason="needs hipcc")
def test_library_host_validation_is_clean(tmp_path):
    lib = tmp_path / "libattnres_san.so"
    src = os.path.join(ROOT, "attention_residuals_depth_amd", "csrc", "attnres.hip")
    inc = os.path.join(ROOT, "include")
    # the sanitizers apply to the host pass only (-Xarch_host before each)
    r = _run(["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-std=c++17", "-fPIC", "-shared", "-g", "-O1",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
              "-Xarch_host", "-fno-sanitize-recover=all", "-I", inc, "-o", lib, src])
    assert r.returncode == 0, r.stderr
    clang = "/opt/rocm/llvm/bin/clang"
    if not os.path.exists(clang):
        clang = shutil.which("clang") or pytest.skip("needs the ROCm clang (same sanitizer runtime as hipcc)")
    exe = tmp_path / "sanitize_abi"
    r = _run([clang, "-std=c11", "-fsanitize=address,undefined", *SAN_FLAGS, "-DABI_PART", "-D__HIP_PLATFORM_AMD__",
              "-I", inc, "-o", exe, DRIVER, f"-L{tmp_path}", "-lattnres_san", "-L/opt/rocm/lib", "-lamdhip64", "-lm",
              f"-Wl,-rpath,{tmp_path}:/opt/rocm/lib"])
    assert r.returncode == 0, r.stderr
    # leak checking stays off: the HIP runtime's own start-up allocations are not ours
    r = _run([exe], env={**os.environ, "ASAN_OPTIONS": "detect_leaks=0", "UBSAN_OPTIONS": "print_stacktrace=1"})
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
