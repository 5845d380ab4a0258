"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU
(no GPU is involved; the GPU kernels are not built here):

  - the C ABI's host code: head_attention_sdpa_amd/csrc/abi.cpp built with
    g++ -fsanitize=address,undefined together with stand-ins for the kernel
    launchers (tests/sanitize/abi_stubs.cpp) and a driver
    (tests/sanitize/abi_driver.cpp) that calls every entry point with valid
    and invalid arguments, including sizes at the limits of int;
  - the oracle: oracle/oracle.c built with gcc -fsanitize=address,undefined
    and the oracle pin suite run against it in a child process (the
    sanitizer runtime preloaded, the library selected by ATTN_ORACLE_LIB).

Any sanitizer report fails the test (-fno-sanitize-recover)."""
import os
import shutil
import subprocess
import sys

import pytest

from conftest import ROOT

CSRC = os.path.join(ROOT, "head_attention_sdpa_amd", "csrc")
SAN = os.path.join(ROOT, "tests", "sanitize")
FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]

needs_gcc = pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None,
                               reason="gcc/g++ not available")


def _report(r):
    return f"exit {r.returncode}\n--- stdout\n{r.stdout[-2000:]}\n--- stderr\n{r.stderr[-4000:]}"


@needs_gcc
def test_abi_host_code_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_san")
    cmd = ["g++", "-std=c++17", *FLAGS, "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include", "-I", CSRC,
           os.path.join(CSRC, "abi.cpp"), os.path.join(SAN, "abi_stubs.cpp"), os.path.join(SAN, "abi_driver.cpp"),
           "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True)
    assert b.returncode == 0, b.stderr[-3000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120,
                       env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1"))
    assert r.returncode == 0 and "abi driver: ok" in r.stdout, _report(r)


@needs_gcc
def test_oracle_under_sanitizers(tmp_path):
    lib = str(tmp_path / "liboracle_san.so")
    b = subprocess.run(["gcc", *FLAGS, "-ffp-contract=off", "-fPIC", "-shared", "-pthread", "-o", lib,
                        os.path.join(ROOT, "oracle", "oracle.c"), "-lm"], capture_output=True, text=True)
    assert b.returncode == 0, b.stderr[-3000:]
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    assert os.path.exists(asan), "libasan not found"
    env = dict(os.environ, ATTN_ORACLE_LIB=lib, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                        "-x", "-q", "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=900)
    assert r.returncode == 0, _report(r)
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, _report(r)
