"""Python binding of libw8a8.so, the MI355X W8A8 INT8 linear library.

Thin marshalling only: each function checks dtypes, devices and shapes of
torch tensors, allocates outputs when the caller passes none, and calls the C
entry point of the same name (declared in include/w8a8.h) on torch's current
HIP stream.  Every step of the computation runs in the library's HIP kernels;
there is no CPU or PyTorch fallback, and importing fails loudly if the library
cannot be loaded.

Operation: the fused W8A8 linear of "Realizing Native INT8 Compute for
Diffusion Transformers on Consumer GPUs" (arXiv 2606.14598), Abstract.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libw8a8.so")
_HEADER = os.path.join(os.path.dirname(_PKG), "include", "w8a8.h")

W8A8_MAX_K = 133136


class W8A8Error(RuntimeError):
    def __init__(self, status: int, fn: str):
        self.status = status
        super().__init__(f"{fn}: {w8a8_status_string(status)}")


def library_path() -> str:
    return _LIB_PATH


def _load() -> ctypes.CDLL:
    if not os.path.exists(_LIB_PATH):
        from . import build as _build  # build only if nothing is built yet
        _build.build()
    L = ctypes.CDLL(_LIB_PATH)
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    sig = {
        "w8a8_status_string": ([I], ctypes.c_char_p),
        "w8a8_quantize_act": ([P, I64, I64, I64, P, I64, P, P], I),
        "w8a8_quantize_weight": ([P, I64, I64, I64, P, I64, P, P], I),
        "w8a8_gemm_i32": ([P, P, I64, I64, I64, P, P], I),
        "w8a8_gemm_dequant": ([P, P, P, P, P, I64, I64, I64, P, P], I),
        "w8a8_linear_workspace_bytes": ([I64, I64], ctypes.c_size_t),
        "w8a8_linear": ([P, P, P, P, I64, I64, I64, P, P, ctypes.c_size_t, P], I),
        "w8a8_linear_noalloc": ([P, P, P, P, I64, I64, I64, P, P], I),
        "w8a8_gemm_dequant_gelu_amax": ([P, P, P, P, P, I64, I64, I64, P, P, P], I),
        "w8a8_quantize_act_amax": ([P, I64, I64, I64, P, P, I64, P, P], I),
        "w8a8_linear_noalloc_max_bytes": ([], ctypes.c_size_t),
        "w8a8_gelu_quantize_act": ([P, I64, I64, I64, P, I64, P, P, P], I),
        "w8a8_gemm_num_configs": ([], I),
        "w8a8_gemm_config_name": ([I], ctypes.c_char_p),
        "w8a8_gemm_select_config": ([I64, I64, I64], I),
        "w8a8_gemm_ex": ([P, P, P, P, P, I64, I64, I64, P, I, I, P], I),
        "w8a8_quantize_act_fp8": ([P, I64, I64, I64, P, I64, P, P], I),
        "w8a8_quantize_weight_fp8": ([P, I64, I64, I64, P, I64, P, P], I),
        "w8a8_gemm_dequant_fp8": ([P, P, P, P, P, I64, I64, I64, P, P], I),
        "w8a8_gemm_fp8_ex": ([P, P, P, P, P, I64, I64, I64, P, I, P], I),
        "w8a8_gemm_fp8_num_configs": ([], I),
        "w8a8_gemm_fp8_config_name": ([I], ctypes.c_char_p),
        "w8a8_linear_fp8": ([P, P, P, P, I64, I64, I64, P, P, ctypes.c_size_t, P], I),
        "w8a8_gelu_quantize_act_fp8": ([P, I64, I64, I64, P, I64, P, P, P], I),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    return L


_lib = _load()


def header_functions() -> list[str]:
    """Names of the functions include/w8a8.h declares."""
    txt = open(_HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(w8a8_\w+)\s*\(", txt)))


def raw() -> ctypes.CDLL:
    """The loaded C library (for tests of the ABI itself)."""
    return _lib


# ------------------------------------------------------------- helpers --
def _ptr(t: torch.Tensor | None):
    if t is None or t.numel() == 0:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, ndim: int):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions (got {tuple(t.shape)})")


def _rows(t: torch.Tensor, name: str) -> int:
    """Row stride of a 2-D tensor whose rows are contiguous."""
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} rows must be contiguous")
    return t.stride(0) if t.shape[0] > 1 else max(t.shape[1], t.stride(0))


def _check(rc: int, fn: str):
    if rc != 0:
        raise W8A8Error(rc, fn)


def _same_device(*ts):
    devs = {t.device for t in ts if t is not None}
    if len(devs) > 1:
        raise ValueError(f"tensors on different devices: {devs}")


# ---------------------------------------------------------- entry points --
def w8a8_status_string(status: int) -> str:
    return _lib.w8a8_status_string(int(status)).decode()


def w8a8_quantize_act(x: torch.Tensor, q: torch.Tensor | None = None,
                      scale: torch.Tensor | None = None):
    """Per-token quantization: bf16 [M, K] -> (int8 [M, K], fp32 [M])."""
    _need(x, "x", torch.bfloat16, 2)
    M, K = x.shape
    q = torch.empty((M, K), dtype=torch.int8, device=x.device) if q is None else q
    scale = torch.empty((M,), dtype=torch.float32, device=x.device) if scale is None else scale
    _need(q, "q", torch.int8, 2)
    _need(scale, "scale", torch.float32, 1)
    _same_device(x, q, scale)
    if tuple(q.shape) != (M, K) or tuple(scale.shape) != (M,) or not scale.is_contiguous():
        raise ValueError("output shapes do not match x")
    rc = _lib.w8a8_quantize_act(_ptr(x), M, K, _rows(x, "x"), _ptr(q), _rows(q, "q"), _ptr(scale),
                                _stream(x.device))
    _check(rc, "w8a8_quantize_act")
    return q, scale


def w8a8_quantize_weight(w: torch.Tensor, q: torch.Tensor | None = None,
                         scale: torch.Tensor | None = None):
    """Per-output-channel quantization: fp32 [N, K] -> (int8 [N, K], fp32 [N])."""
    _need(w, "w", torch.float32, 2)
    N, K = w.shape
    q = torch.empty((N, K), dtype=torch.int8, device=w.device) if q is None else q
    scale = torch.empty((N,), dtype=torch.float32, device=w.device) if scale is None else scale
    _need(q, "q", torch.int8, 2)
    _need(scale, "scale", torch.float32, 1)
    _same_device(w, q, scale)
    if tuple(q.shape) != (N, K) or tuple(scale.shape) != (N,) or not scale.is_contiguous():
        raise ValueError("output shapes do not match w")
    rc = _lib.w8a8_quantize_weight(_ptr(w), N, K, _rows(w, "w"), _ptr(q), _rows(q, "q"),
                                   _ptr(scale), _stream(w.device))
    _check(rc, "w8a8_quantize_weight")
    return q, scale


def _gemm_inputs(q_x, w_q):
    _need(q_x, "q_x", torch.int8, 2)
    _need(w_q, "w_q", torch.int8, 2)
    M, K = q_x.shape
    N, K2 = w_q.shape
    if K != K2:
        raise ValueError(f"K mismatch: q_x {tuple(q_x.shape)} vs w_q {tuple(w_q.shape)}")
    if not (q_x.is_contiguous() and w_q.is_contiguous()):
        raise ValueError("q_x and w_q must be contiguous")
    return M, N, K


def _vec(t, name, dtype, n):
    if t is None:
        return None
    _need(t, name, dtype, 1)
    if t.shape[0] != n or not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous with {n} elements")
    return t


def w8a8_gemm_i32(q_x: torch.Tensor, w_q: torch.Tensor, out: torch.Tensor | None = None):
    """Debug entry: int32 accumulators [M, N] = q_x . w_q^T."""
    M, N, K = _gemm_inputs(q_x, w_q)
    out = torch.empty((M, N), dtype=torch.int32, device=q_x.device) if out is None else out
    _need(out, "out", torch.int32, 2)
    _same_device(q_x, w_q, out)
    if tuple(out.shape) != (M, N) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [M, N] int32 tensor")
    rc = _lib.w8a8_gemm_i32(_ptr(q_x), _ptr(w_q), M, N, K, _ptr(out), _stream(q_x.device))
    _check(rc, "w8a8_gemm_i32")
    return out


def w8a8_gemm_dequant(q_x, s_x, w_q, s_w, bias=None, out=None):
    """int8 GEMM + dequant/bias epilogue on pre-quantized activations -> bf16 [M, N]."""
    M, N, K = _gemm_inputs(q_x, w_q)
    _vec(s_x, "s_x", torch.float32, M)
    _vec(s_w, "s_w", torch.float32, N)
    _vec(bias, "bias", torch.bfloat16, N)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=q_x.device) if out is None else out
    _need(out, "out", torch.bfloat16, 2)
    _same_device(q_x, s_x, w_q, s_w, bias, out)
    if tuple(out.shape) != (M, N) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [M, N] bf16 tensor")
    rc = _lib.w8a8_gemm_dequant(_ptr(q_x), _ptr(s_x), _ptr(w_q), _ptr(s_w), _ptr(bias), M, N, K,
                                _ptr(out), _stream(q_x.device))
    _check(rc, "w8a8_gemm_dequant")
    return out


def w8a8_gemm_dequant_gelu_amax(q_x, s_x, w_q, s_w, bias=None, h_out=None, amax=None):
    """The GEMM with GELU and the row maxima of |h| in its epilogue (the
    inter-layer fusion variant): -> (h bf16 [M, N], amax int32 [M] holding
    the fp32 bit patterns of max_n |h[m, n]|)."""
    M, N, K = _gemm_inputs(q_x, w_q)
    _vec(s_x, "s_x", torch.float32, M)
    _vec(s_w, "s_w", torch.float32, N)
    _vec(bias, "bias", torch.bfloat16, N)
    h_out = torch.empty((M, N), dtype=torch.bfloat16, device=q_x.device) if h_out is None else h_out
    amax = torch.empty((M,), dtype=torch.int32, device=q_x.device) if amax is None else amax
    _need(h_out, "h_out", torch.bfloat16, 2)
    _vec(amax, "amax", torch.int32, M)
    _same_device(q_x, s_x, w_q, s_w, bias, h_out, amax)
    if tuple(h_out.shape) != (M, N) or not h_out.is_contiguous():
        raise ValueError("h_out must be a contiguous [M, N] bf16 tensor")
    rc = _lib.w8a8_gemm_dequant_gelu_amax(_ptr(q_x), _ptr(s_x), _ptr(w_q), _ptr(s_w), _ptr(bias), M, N,
                                          K, _ptr(h_out), _ptr(amax), _stream(q_x.device))
    _check(rc, "w8a8_gemm_dequant_gelu_amax")
    return h_out, amax


def w8a8_quantize_act_amax(h, amax, q=None, scale=None):
    """Per-token quantization of bf16 rows whose absmax is given (fp32 bits in
    an int32 [M] tensor, from w8a8_gemm_dequant_gelu_amax) -> (q, scale)."""
    _need(h, "h", torch.bfloat16, 2)
    M, K = h.shape
    _vec(amax, "amax", torch.int32, M)
    q = torch.empty((M, K), dtype=torch.int8, device=h.device) if q is None else q
    scale = torch.empty((M,), dtype=torch.float32, device=h.device) if scale is None else scale
    _need(q, "q", torch.int8, 2)
    _need(scale, "scale", torch.float32, 1)
    _same_device(h, amax, q, scale)
    if tuple(q.shape) != (M, K) or tuple(scale.shape) != (M,) or not scale.is_contiguous():
        raise ValueError("output shapes do not match h")
    rc = _lib.w8a8_quantize_act_amax(_ptr(h), M, K, _rows(h, "h"), _ptr(amax), _ptr(q), _rows(q, "q"),
                                     _ptr(scale), _stream(h.device))
    _check(rc, "w8a8_quantize_act_amax")
    return q, scale


def w8a8_gemm_ex(q_x, s_x, w_q, s_w, bias=None, out=None, out_int32=False, config=-1):
    """The GEMM with an explicit kernel configuration (-1 = the library's choice)."""
    M, N, K = _gemm_inputs(q_x, w_q)
    if not out_int32:
        _vec(s_x, "s_x", torch.float32, M)
        _vec(s_w, "s_w", torch.float32, N)
        _vec(bias, "bias", torch.bfloat16, N)
    dt = torch.int32 if out_int32 else torch.bfloat16
    out = torch.empty((M, N), dtype=dt, device=q_x.device) if out is None else out
    _need(out, "out", dt, 2)
    _same_device(q_x, s_x, w_q, s_w, bias, out)
    if tuple(out.shape) != (M, N) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [M, N] tensor")
    rc = _lib.w8a8_gemm_ex(_ptr(q_x), _ptr(s_x), _ptr(w_q), _ptr(s_w), _ptr(bias), M, N, K,
                           _ptr(out), 1 if out_int32 else 0, int(config), _stream(q_x.device))
    _check(rc, "w8a8_gemm_ex")
    return out


def w8a8_linear_workspace_bytes(M: int, K: int) -> int:
    return int(_lib.w8a8_linear_workspace_bytes(int(M), int(K)))


def w8a8_linear(x, w_q, s_w, bias=None, out=None, workspace=None):
    """The fused W8A8 linear: bf16 x [M, K] -> bf16 y [M, N].

    `workspace` (uint8 GPU tensor of at least w8a8_linear_workspace_bytes(M, K)
    bytes) receives the activation codes and scales; allocated if None."""
    _need(x, "x", torch.bfloat16, 2)
    _need(w_q, "w_q", torch.int8, 2)
    M, K = x.shape
    N, K2 = w_q.shape
    if K != K2:
        raise ValueError(f"K mismatch: x {tuple(x.shape)} vs w_q {tuple(w_q.shape)}")
    if not (x.is_contiguous() and w_q.is_contiguous()):
        raise ValueError("x and w_q must be contiguous")
    _vec(s_w, "s_w", torch.float32, N)
    _vec(bias, "bias", torch.bfloat16, N)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device) if out is None else out
    _need(out, "out", torch.bfloat16, 2)
    if tuple(out.shape) != (M, N) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [M, N] bf16 tensor")
    need = w8a8_linear_workspace_bytes(M, K)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=x.device)
    _need(workspace, "workspace", torch.uint8, 1)
    _same_device(x, w_q, s_w, bias, out, workspace)
    rc = _lib.w8a8_linear(_ptr(x), _ptr(w_q), _ptr(s_w), _ptr(bias), M, N, K, _ptr(out),
                          _ptr(workspace), workspace.numel(), _stream(x.device))
    _check(rc, "w8a8_linear")
    return out


def w8a8_linear_noalloc_max_bytes() -> int:
    return int(_lib.w8a8_linear_noalloc_max_bytes())


def w8a8_linear_noalloc(x, w_q, s_w, bias=None, out=None):
    """The fused W8A8 linear without a workspace: the activation codes and
    scales go to the library's static device scratch (for callers that cannot
    allocate; calls on one GPU must be ordered).  bf16 x [M, K] -> bf16 y."""
    _need(x, "x", torch.bfloat16, 2)
    _need(w_q, "w_q", torch.int8, 2)
    M, K = x.shape
    N, K2 = w_q.shape
    if K != K2:
        raise ValueError(f"K mismatch: x {tuple(x.shape)} vs w_q {tuple(w_q.shape)}")
    if not (x.is_contiguous() and w_q.is_contiguous()):
        raise ValueError("x and w_q must be contiguous")
    _vec(s_w, "s_w", torch.float32, N)
    _vec(bias, "bias", torch.bfloat16, N)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device) if out is None else out
    _need(out, "out", torch.bfloat16, 2)
    if tuple(out.shape) != (M, N) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [M, N] bf16 tensor")
    _same_device(x, w_q, s_w, bias, out)
    with torch.cuda.device(x.device):
        rc = _lib.w8a8_linear_noalloc(_ptr(x), _ptr(w_q), _ptr(s_w), _ptr(bias), M, N, K, _ptr(out),
                                      _stream(x.device))
    _check(rc, "w8a8_linear_noalloc")
    return out


def w8a8_gelu_quantize_act(y, q=None, scale=None, h_out=None, want_h=False):
    """GELU then per-token quantization: bf16 [M, K] -> (int8 [M, K], fp32 [M], h or None)."""
    _need(y, "y", torch.bfloat16, 2)
    M, K = y.shape
    q = torch.empty((M, K), dtype=torch.int8, device=y.device) if q is None else q
    scale = torch.empty((M,), dtype=torch.float32, device=y.device) if scale is None else scale
    if h_out is None and want_h:
        h_out = torch.empty((M, K), dtype=torch.bfloat16, device=y.device)
    _need(q, "q", torch.int8, 2)
    _need(scale, "scale", torch.float32, 1)
    if h_out is not None:
        _need(h_out, "h_out", torch.bfloat16, 2)
        if tuple(h_out.shape) != (M, K) or not h_out.is_contiguous():
            raise ValueError("h_out must be a contiguous [M, K] bf16 tensor")
    _same_device(y, q, scale, h_out)
    if tuple(q.shape) != (M, K) or tuple(scale.shape) != (M,) or not scale.is_contiguous():
        raise ValueError("output shapes do not match y")
    rc = _lib.w8a8_gelu_quantize_act(_ptr(y), M, K, _rows(y, "y"), _ptr(q), _rows(q, "q"),
                                     _ptr(scale), _ptr(h_out), _stream(y.device))
    _check(rc, "w8a8_gelu_quantize_act")
    return q, scale, h_out


def w8a8_gemm_num_configs() -> int:
    return int(_lib.w8a8_gemm_num_configs())


def w8a8_gemm_config_name(config: int) -> str | None:
    r = _lib.w8a8_gemm_config_name(int(config))
    return r.decode() if r is not None else None


def w8a8_gemm_select_config(M: int, N: int, K: int) -> int:
    return int(_lib.w8a8_gemm_select_config(int(M), int(N), int(K)))


# ------------------------------------------------------------------ FP8 --
# OCP e4m3 codes travel as uint8 tensors (view them as torch.float8_e4m3fn
# for their values).
def _quantize_rows_fp8(fn, x, dtype, q, scale, what):
    _need(x, what, dtype, 2)
    R, K = x.shape
    q = torch.empty((R, K), dtype=torch.uint8, device=x.device) if q is None else q
    scale = torch.empty((R,), dtype=torch.float32, device=x.device) if scale is None else scale
    _need(q, "q", torch.uint8, 2)
    _need(scale, "scale", torch.float32, 1)
    _same_device(x, q, scale)
    if tuple(q.shape) != (R, K) or tuple(scale.shape) != (R,) or not scale.is_contiguous():
        raise ValueError(f"output shapes do not match {what}")
    rc = getattr(_lib, fn)(_ptr(x), R, K, _rows(x, what), _ptr(q), _rows(q, "q"), _ptr(scale),
                           _stream(x.device))
    _check(rc, fn)
    return q, scale


def w8a8_quantize_act_fp8(x, q=None, scale=None):
    """Per-token e4m3 quantization: bf16 [M, K] -> (uint8 codes [M, K], fp32 [M])."""
    return _quantize_rows_fp8("w8a8_quantize_act_fp8", x, torch.bfloat16, q, scale, "x")


def w8a8_quantize_weight_fp8(w, q=None, scale=None):
    """Per-output-channel e4m3 quantization: fp32 [N, K] -> (uint8 codes [N, K], fp32 [N])."""
    return _quantize_rows_fp8("w8a8_quantize_weight_fp8", w, torch.float32, q, scale, "w")


def w8a8_gelu_quantize_act_fp8(y, q=None, scale=None, h_out=None, want_h=False):
    """GELU then per-token e4m3 quantization -> (uint8 codes, fp32 scales, h or None)."""
    _need(y, "y", torch.bfloat16, 2)
    M, K = y.shape
    q = torch.empty((M, K), dtype=torch.uint8, device=y.device) if q is None else q
    scale = torch.empty((M,), dtype=torch.float32, device=y.device) if scale is None else scale
    if want_h and h_out is None:
        h_out = torch.empty((M, K), dtype=torch.bfloat16, device=y.device)
    _need(q, "q", torch.uint8, 2)
    _need(scale, "scale", torch.float32, 1)
    if h_out is not None:
        _need(h_out, "h_out", torch.bfloat16, 2)
        if tuple(h_out.shape) != (M, K) or not h_out.is_contiguous():
            raise ValueError("h_out must be a contiguous [M, K] bf16 tensor")
    _same_device(y, q, scale, h_out)
    if tuple(q.shape) != (M, K) or tuple(scale.shape) != (M,) or not scale.is_contiguous():
        raise ValueError("output shapes do not match y")
    rc = _lib.w8a8_gelu_quantize_act_fp8(_ptr(y), M, K, _rows(y, "y"), _ptr(q), _rows(q, "q"),
                                         _ptr(scale), _ptr(h_out), _stream(y.device))
    _check(rc, "w8a8_gelu_quantize_act_fp8")
    return q, scale, h_out


def w8a8_gemm_dequant_fp8(q_x, s_x, w_q, s_w, bias=None, out=None, config=-1):
    """e4m3 GEMM (fp32 accumulation) + dequant/bias epilogue -> bf16 [M, N];
    config -1 is the library's choice."""
    _need(q_x, "q_x", torch.uint8, 2)
    _need(w_q, "w_q", torch.uint8, 2)
    M, K = q_x.shape
    N, K2 = w_q.shape
    if K != K2:
        raise ValueError(f"K mismatch: q_x {tuple(q_x.shape)} vs w_q {tuple(w_q.shape)}")
    if not (q_x.is_contiguous() and w_q.is_contiguous()):
        raise ValueError("q_x and w_q must be contiguous")
    _vec(s_x, "s_x", torch.float32, M)
    _vec(s_w, "s_w", torch.float32, N)
    _vec(bias, "bias", torch.bfloat16, N)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=q_x.device) if out is None else out
    _need(out, "out", torch.bfloat16, 2)
    _same_device(q_x, s_x, w_q, s_w, bias, out)
    if tuple(out.shape) != (M, N) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [M, N] bf16 tensor")
    rc = _lib.w8a8_gemm_fp8_ex(_ptr(q_x), _ptr(s_x), _ptr(w_q), _ptr(s_w), _ptr(bias), M, N, K,
                               _ptr(out), int(config), _stream(q_x.device))
    _check(rc, "w8a8_gemm_fp8_ex")
    return out


def w8a8_gemm_fp8_ex(q_x, s_x, w_q, s_w, bias=None, out=None, config=-1):
    """Same as w8a8_gemm_dequant_fp8 (the C entry with an explicit configuration)."""
    return w8a8_gemm_dequant_fp8(q_x, s_x, w_q, s_w, bias, out, config)


def w8a8_linear_fp8(x, w_q, s_w, bias=None, out=None, workspace=None):
    """The fused FP8 linear: bf16 x [M, K] -> bf16 y [M, N] (w_q, s_w from
    w8a8_quantize_weight_fp8; workspace as for w8a8_linear)."""
    _need(x, "x", torch.bfloat16, 2)
    _need(w_q, "w_q", torch.uint8, 2)
    M, K = x.shape
    N, K2 = w_q.shape
    if K != K2:
        raise ValueError(f"K mismatch: x {tuple(x.shape)} vs w_q {tuple(w_q.shape)}")
    if not (x.is_contiguous() and w_q.is_contiguous()):
        raise ValueError("x and w_q must be contiguous")
    _vec(s_w, "s_w", torch.float32, N)
    _vec(bias, "bias", torch.bfloat16, N)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device) if out is None else out
    _need(out, "out", torch.bfloat16, 2)
    if tuple(out.shape) != (M, N) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [M, N] bf16 tensor")
    need = w8a8_linear_workspace_bytes(M, K)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=x.device)
    _need(workspace, "workspace", torch.uint8, 1)
    _same_device(x, w_q, s_w, bias, out, workspace)
    rc = _lib.w8a8_linear_fp8(_ptr(x), _ptr(w_q), _ptr(s_w), _ptr(bias), M, N, K, _ptr(out),
                              _ptr(workspace), workspace.numel(), _stream(x.device))
    _check(rc, "w8a8_linear_fp8")
    return out


def w8a8_gemm_fp8_num_configs() -> int:
    return int(_lib.w8a8_gemm_fp8_num_configs())


def w8a8_gemm_fp8_config_name(config: int) -> str | None:
    r = _lib.w8a8_gemm_fp8_config_name(int(config))
    return r.decode() if r else None


class W8A8Linear(torch.nn.Module):
    """Drop-in replacement for a bf16 ``nn.Linear``: weights quantized once per
    output channel on the GPU, activations per token at every call, one fused
    int8 GEMM with the dequant/bias epilogue per call (the layer the paper
    swaps into the model's linears, Abstract).  The quantized weights, their
    scales and the bf16 bias are buffers, so ``state_dict()`` exports them and
    ``load_state_dict`` restores them.  Inputs must be bf16 on the GPU; leading
    dimensions are flattened to tokens.  With uint8 e4m3 codes for w_q (from
    ``from_float(..., fp8=True)``) the layer runs the FP8 variant instead."""

    def __init__(self, w_q: torch.Tensor, s_w: torch.Tensor, bias: torch.Tensor | None = None):
        super().__init__()
        if w_q.dtype not in (torch.int8, torch.uint8) or w_q.dim() != 2:
            raise ValueError("w_q must be an int8 (or uint8 e4m3) [N, K] tensor")
        self.fp8 = w_q.dtype == torch.uint8
        self.out_features, self.in_features = int(w_q.shape[0]), int(w_q.shape[1])
        self.register_buffer("w_q", w_q)
        self.register_buffer("s_w", s_w)
        self.register_buffer("bias", bias)

    @classmethod
    def from_float(cls, weight: torch.Tensor, bias: torch.Tensor | None = None,
                   fp8: bool = False) -> "W8A8Linear":
        """Quantize a float weight [N, K] (and take a bias) already on the GPU."""
        quant = w8a8_quantize_weight_fp8 if fp8 else w8a8_quantize_weight
        w_q, s_w = quant(weight.detach().float().contiguous())
        b = bias.detach().to(torch.bfloat16).contiguous() if bias is not None else None
        return cls(w_q, s_w, b)

    @classmethod
    def from_linear(cls, linear: torch.nn.Linear, fp8: bool = False) -> "W8A8Linear":
        return cls.from_float(linear.weight, linear.bias, fp8)

    def extra_repr(self) -> str:
        return (f"in_features={self.in_features}, out_features={self.out_features}, "
                f"bias={self.bias is not None}, codes={'e4m3' if self.fp8 else 'int8'}")

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        lead = x.shape[:-1]
        x2 = x.reshape(-1, x.shape[-1]).contiguous()
        # the workspace (activation codes + scales) is taken from torch's
        # caching allocator for each call, like any temporary: it is then
        # stream- and graph-pool-aware, and no layer holds memory between calls
        fn = w8a8_linear_fp8 if self.fp8 else w8a8_linear
        y = fn(x2, self.w_q, self.s_w, self.bias)
        return y.reshape(*lead, self.out_features)


def quantize_linears(module: torch.nn.Module, include=None, fp8: bool = False) -> int:
    """Replace, in place, every ``nn.Linear`` inside ``module`` whose input
    width the library takes (a multiple of 16, at most W8A8_MAX_K) by a
    W8A8Linear quantized from its weights (e4m3 codes with ``fp8``);
    ``include(name, linear)`` may narrow the choice.  The linears must already
    be on the GPU.  Returns the number of layers replaced."""
    count = 0
    for name, child in list(module.named_children()):
        if isinstance(child, torch.nn.Linear):
            k = child.in_features
            if k % 16 == 0 and 0 < k <= W8A8_MAX_K and (include is None or include(name, child)):
                if child.weight.device.type != "cuda":
                    raise ValueError(f"quantize_linears: layer {name!r} is not on a GPU "
                                     f"(weights are quantized by the library's GPU kernel)")
                setattr(module, name, W8A8Linear.from_linear(child, fp8))
                count += 1
        else:
            count += quantize_linears(child, include, fp8)
    return count
