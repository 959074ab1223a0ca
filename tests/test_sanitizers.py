"""Host-side sanitizer builds (CPU only).

1. mla_api.hip's host code (argument validation, workspace sizing, the
   device query) built with AddressSanitizer and UndefinedBehaviorSanitizer
   (every UB report fatal) into an executable with tests/sanitize/abi_harness.cpp,
   which drives every entry point at and beyond its limits; the kernel
   launchers are stubs that no call may reach without a GPU.
2. The fp64 oracle built with the same sanitizers and run through every pin
   of tests/oracle_pins.py in a child process with the sanitizer runtimes
   preloaded.
"""
import os
import shutil
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.dirname(os.path.abspath(__file__))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

pytestmark = pytest.mark.skipif(torch.cuda.is_available(),
                                reason="host sanitizer runs expect no GPU")

SAN_ENV = dict(ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def test_abi_validation_under_asan_ubsan(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not installed")
    exe = tmp_path / "abi_harness"
    cmd = [HIPCC, "--offload-arch=gfx950", "-x", "hip", "-std=c++17", "-g", "-O1",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "mla_paged_attention_amd", "csrc", "mla_api.hip"),
           os.path.join(HERE, "sanitize", "abi_harness.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300,
                       env=dict(os.environ, **SAN_ENV))
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failures, 0 launches" in r.stdout, r.stdout


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_under_asan_ubsan(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not (asan and ubsan and shutil.which("gcc")):
        pytest.skip("gcc sanitizer runtimes not installed")
    lib = tmp_path / "liboracle_san.so"
    cmd = ["gcc", "-O1", "-g", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-o", str(lib), os.path.join(ROOT, "oracle", "mla_oracle.c"), "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, LD_PRELOAD=f"{asan}:{ubsan}", OMP_NUM_THREADS="4", **SAN_ENV)
    r = subprocess.run([sys.executable, os.path.join(HERE, "oracle_pins.py"), "--lib", str(lib)],
                       capture_output=True, text=True, timeout=900, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
