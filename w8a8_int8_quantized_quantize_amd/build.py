"""Builds libw8a8.so from csrc/ with hipcc for gfx950 (in-tree, no JIT cache).

Flags that the numerical contract depends on:
  -ffp-contract=off                        no fused multiply-add in the epilogue
  -fhip-fp32-correctly-rounded-divide-sqrt IEEE fp32 division in quantization
  -fno-gpu-flush-denormals-to-zero         fp32 denormals kept
Packed fp32 instructions are disabled (-packed-fp32-ops); the host pass warns
that it does not know that feature, which is harmless.

The GELU table compiled into quantize.hip is written first, into the build
folder, by csrc/gen_gelu_lut.py.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libw8a8.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["api.cpp", "quantize.hip", "gemm.hip", "noalloc.hip"]

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC, "-I", BUILD, "-Wall", "-Wno-unused-command-line-argument",
]


def _compile(src: str, save_temps: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC] + COMMON + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if save_temps:
        cmd += ["-save-temps=obj"]
    r = subprocess.run(cmd, cwd=BUILD, capture_output=True, text=True)
    errs = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{errs}")
    if errs.strip():
        sys.stderr.write(errs + "\n")
    return obj


def build(save_temps: bool | None = None) -> str:
    """Compile every source and link libw8a8.so next to this file."""
    if save_temps is None:
        save_temps = os.environ.get("W8A8_SAVE_TEMPS", "0") == "1"
    os.makedirs(BUILD, exist_ok=True)
    r = subprocess.run([sys.executable, os.path.join(CSRC, "gen_gelu_lut.py"),
                        os.path.join(BUILD, "gelu_lut.inc")], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("gen_gelu_lut.py failed:\n" + r.stderr)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES) + 1) as ex:
        objs = list(ex.map(lambda s: _compile(s, save_temps), SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
