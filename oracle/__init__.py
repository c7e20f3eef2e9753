"""CPU oracle for the W8A8 INT8 linear layer -- TEST INFRASTRUCTURE ONLY.

Only `tests/`, `__graft_entry__.smoke()` and the CPU-baseline leg of `bench.py`
may import this package.  The GPU library never imports, links or calls it,
and it never imports the GPU library.  The arithmetic lives in `oracle.c`
(plain C, one IEEE operation per step, no FMA contraction, fp64 for GELU);
this module only builds it, loads it and marshals numpy arrays.

Definitions follow "Realizing Native INT8 Compute for Diffusion Transformers on
Consumer GPUs" (arXiv 2606.14598), Abstract (per-token activation and
per-channel weight int8 quantization, int8 x int8 -> int32 accumulation,
dequantization and bias in the epilogue), with the readings listed at the top
of `oracle.c`.

Pins: every function here is checked by `tests/test_oracle_pins.py` against
closed forms, invariants, brute force on tiny inputs and library routines
(torch's bf16 conversion, numpy's int64 matmul, scipy's erfc).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

ORACLE_OK = 0
ORACLE_ERR_INT32 = 1


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (portable x86-64 code, no -march=native)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-std=gnu99", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        P, I64 = ctypes.c_void_p, ctypes.c_int64
        L.oracle_num_threads.restype = ctypes.c_int
        for name, args, res in [
            ("oracle_bf16_to_f32", [P, P, I64], None),
            ("oracle_f32_to_bf16", [P, P, I64], None),
            ("oracle_f64_to_bf16", [P, P, I64], None),
            ("oracle_quantize_rows_f32", [P, I64, I64, I64, P, I64, P], None),
            ("oracle_quantize_rows_bf16", [P, I64, I64, I64, P, I64, P, P], None),
            ("oracle_gemm_i64", [P, I64, P, I64, I64, I64, I64, P], None),
            ("oracle_epilogue", [P, I64, I64, P, P, P, P], ctypes.c_int),
            ("oracle_gelu_f64", [P, P, I64], None),
            ("oracle_gelu_bf16", [P, I64, P], None),
            ("oracle_e4m3_decode", [P, P, I64], None),
            ("oracle_e4m3_encode", [P, P, I64], None),
            ("oracle_quantize_rows_f32_fp8", [P, I64, I64, I64, P, I64, P], None),
            ("oracle_quantize_rows_bf16_fp8", [P, I64, I64, I64, P, I64, P, P], None),
            ("oracle_gemm_fp8", [P, I64, P, I64, I64, I64, I64, P], None),
            ("oracle_epilogue_f64acc", [P, I64, I64, P, P, P, P], None),
        ]:
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def num_threads() -> int:
    return int(lib().oracle_num_threads())


# ------------------------------------------------------------------ bf16 --
def bf16_to_f32(h) -> np.ndarray:
    h = _c(h, np.uint16)
    out = np.empty(h.shape, np.float32)
    lib().oracle_bf16_to_f32(_p(h), _p(out), h.size)
    return out


def f32_to_bf16(f) -> np.ndarray:
    f = _c(f, np.float32)
    out = np.empty(f.shape, np.uint16)
    lib().oracle_f32_to_bf16(_p(f), _p(out), f.size)
    return out


def f64_to_bf16(d) -> np.ndarray:
    d = _c(d, np.float64)
    out = np.empty(d.shape, np.uint16)
    lib().oracle_f64_to_bf16(_p(d), _p(out), d.size)
    return out


# ---------------------------------------------------------- quantization --
def quantize_rows_f32(x):
    """Per-row symmetric int8 quantization of fp32 rows -> (q int8, scale fp32)."""
    x = _c(x, np.float32)
    assert x.ndim == 2
    R, K = x.shape
    q = np.empty((R, K), np.int8)
    s = np.empty((R,), np.float32)
    lib().oracle_quantize_rows_f32(_p(x), R, K, K, _p(q), K, _p(s))
    return q, s


def quantize_rows_bf16(x_bits):
    """Per-row (per-token) quantization of bf16 rows given as uint16 bit patterns."""
    x = _c(x_bits, np.uint16)
    assert x.ndim == 2
    R, K = x.shape
    q = np.empty((R, K), np.int8)
    s = np.empty((R,), np.float32)
    tmp = np.empty((R, K), np.float32)
    lib().oracle_quantize_rows_bf16(_p(x), R, K, K, _p(q), K, _p(s), _p(tmp))
    return q, s


# -------------------------------------------------------------- int GEMM --
def gemm_i64(a, b) -> np.ndarray:
    """acc[m, n] = sum_k a[m, k] * b[n, k] in int64, a: [M, K] int8, b: [N, K] int8."""
    a = _c(a, np.int8)
    b = _c(b, np.int8)
    M, K = a.shape
    N, K2 = b.shape
    assert K == K2
    acc = np.empty((M, N), np.int64)
    lib().oracle_gemm_i64(_p(a), K, _p(b), K, M, N, K, _p(acc))
    return acc


# -------------------------------------------------------------- epilogue --
def epilogue(acc, s_x, s_w, bias_bits=None) -> np.ndarray:
    """bf16 bits of (s_x[m]*s_w[n])*float(acc) + bias[n]; raises if acc overflows int32."""
    acc = _c(acc, np.int64)
    M, N = acc.shape
    s_x = _c(s_x, np.float32)
    s_w = _c(s_w, np.float32)
    assert s_x.shape == (M,) and s_w.shape == (N,)
    y = np.empty((M, N), np.uint16)
    if bias_bits is not None:
        bias = _c(bias_bits, np.uint16)
        assert bias.shape == (N,)
        bp = _p(bias)
    else:
        bp = None
    rc = lib().oracle_epilogue(_p(acc), M, N, _p(s_x), _p(s_w), bp, _p(y))
    if rc != ORACLE_OK:
        raise OverflowError("accumulator outside int32 range")
    return y


# ------------------------------------------------------------------ GELU --
def gelu_f64(v) -> np.ndarray:
    v = _c(v, np.float64)
    out = np.empty(v.shape, np.float64)
    lib().oracle_gelu_f64(_p(v), _p(out), v.size)
    return out


def gelu_bf16(y_bits) -> np.ndarray:
    y = _c(y_bits, np.uint16)
    h = np.empty(y.shape, np.uint16)
    lib().oracle_gelu_bf16(_p(y), y.size, _p(h))
    return h


# ------------------------------------------------------------ FP8 (e4m3) --
def e4m3_decode(codes) -> np.ndarray:
    c = _c(codes, np.uint8)
    out = np.empty(c.shape, np.float64)
    lib().oracle_e4m3_decode(_p(c), _p(out), c.size)
    return out


def e4m3_encode(f) -> np.ndarray:
    f = _c(f, np.float32)
    out = np.empty(f.shape, np.uint8)
    lib().oracle_e4m3_encode(_p(f), _p(out), f.size)
    return out


def quantize_rows_f32_fp8(x):
    """Per-row e4m3 quantization of fp32 rows -> (codes uint8, scale fp32)."""
    x = _c(x, np.float32)
    assert x.ndim == 2
    R, K = x.shape
    q = np.empty((R, K), np.uint8)
    s = np.empty((R,), np.float32)
    lib().oracle_quantize_rows_f32_fp8(_p(x), R, K, K, _p(q), K, _p(s))
    return q, s


def quantize_rows_bf16_fp8(x_bits):
    """Per-row (per-token) e4m3 quantization of bf16 rows (uint16 bit patterns)."""
    x = _c(x_bits, np.uint16)
    assert x.ndim == 2
    R, K = x.shape
    q = np.empty((R, K), np.uint8)
    s = np.empty((R,), np.float32)
    tmp = np.empty((R, K), np.float32)
    lib().oracle_quantize_rows_bf16_fp8(_p(x), R, K, K, _p(q), K, _p(s), _p(tmp))
    return q, s


def gemm_fp8(a, b) -> np.ndarray:
    """acc[m, n] = sum_k e4m3(a[m, k]) * e4m3(b[n, k]), exact, as fp64."""
    a = _c(a, np.uint8)
    b = _c(b, np.uint8)
    M, K = a.shape
    N, K2 = b.shape
    assert K == K2
    acc = np.empty((M, N), np.float64)
    lib().oracle_gemm_fp8(_p(a), K, _p(b), K, M, N, K, _p(acc))
    return acc


def epilogue_f64acc(acc, s_x, s_w, bias_bits=None) -> np.ndarray:
    """bf16 bits of (s_x[m]*s_w[n])*fp32(acc) + bias[n] for an exact fp64 acc."""
    acc = _c(acc, np.float64)
    M, N = acc.shape
    s_x = _c(s_x, np.float32)
    s_w = _c(s_w, np.float32)
    y = np.empty((M, N), np.uint16)
    bias = _c(bias_bits, np.uint16) if bias_bits is not None else None
    bp = _p(bias) if bias is not None else None
    lib().oracle_epilogue_f64acc(_p(acc), M, N, _p(s_x), _p(s_w), bp, _p(y))
    return y


def linear_fp8(x_bits, wq, s_w, bias_bits=None):
    """The FP8 layer: per-token e4m3 quantize -> exact product sums -> epilogue."""
    q_x, s_x = quantize_rows_bf16_fp8(x_bits)
    acc = gemm_fp8(q_x, wq)
    return {"q_x": q_x, "s_x": s_x, "acc": acc, "y": epilogue_f64acc(acc, s_x, s_w, bias_bits)}


# ------------------------------------------------------------ composites --
def linear(x_bits, wq, s_w, bias_bits=None):
    """The whole layer: per-token quantize -> int GEMM -> epilogue.

    Returns a dict with q_x, s_x, acc (int64) and y (bf16 bits)."""
    q_x, s_x = quantize_rows_bf16(x_bits)
    acc = gemm_i64(q_x, wq)
    y = epilogue(acc, s_x, s_w, bias_bits)
    return {"q_x": q_x, "s_x": s_x, "acc": acc, "y": y}


def linear_prequant(q_x, s_x, wq, s_w, bias_bits=None):
    acc = gemm_i64(q_x, wq)
    return {"acc": acc, "y": epilogue(acc, s_x, s_w, bias_bits)}
