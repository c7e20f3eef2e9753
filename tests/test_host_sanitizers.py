"""Host-side sanitizer builds (CPU only, no GPU code is compiled).

* The C-ABI layer (api.cpp) with AddressSanitizer and UndefinedBehavior-
  Sanitizer, linked against recording stubs of the device launch functions
  (tests/csrc/abi_host_check.cpp; HIP's host types come from a minimal
  stand-in header, tests/csrc/host_stub): every entry point's validation and
  marshalling path runs on exactly sized heap buffers.
* The CPU oracle (oracle/oracle.c) with the same sanitizers, driven by
  tests/csrc/oracle_host_check.c on small strided inputs and its edge cases.

Both check programs exit 0 only if every check holds and no sanitizer reports.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "w8a8_int8_quantized_quantize_amd", "csrc")
TCSRC = os.path.join(ROOT, "tests", "csrc")
BUILD = os.path.join(ROOT, "_build", "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="2")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True, env=ENV, timeout=600)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_abi_layer_under_asan_ubsan():
    os.makedirs(BUILD, exist_ok=True)
    exe = os.path.join(BUILD, "abi_host_check")
    _run(["g++", "-std=c++17", *SAN, "-I", os.path.join(TCSRC, "host_stub"),
          "-I", os.path.join(ROOT, "include"), "-I", CSRC,
          os.path.join(CSRC, "api.cpp"), os.path.join(TCSRC, "abi_host_check.cpp"), "-o", exe])
    assert "abi ok" in _run([exe])


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan():
    os.makedirs(BUILD, exist_ok=True)
    exe = os.path.join(BUILD, "oracle_host_check")
    _run(["gcc", "-std=gnu99", *SAN, "-fopenmp", "-ffp-contract=off",
          os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(TCSRC, "oracle_host_check.c"),
          "-o", exe, "-lm"])
    assert "oracle ok" in _run([exe])
