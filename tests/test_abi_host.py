"""Host-side tests of the C-ABI library: it loads, exports every function the
header declares, and rejects bad arguments with the documented status before
any HIP call (so these run on a machine without a GPU)."""
from __future__ import annotations

import ctypes
import subprocess

import pytest

import w8a8_int8_quantized_quantize_amd as w8

L = w8.raw()
P = ctypes.c_void_p
A = P(0x10000)      # a fake, 16-byte aligned address: never dereferenced, as
MIS = P(0x10001)    # every call below fails validation before any launch

OK, NULL, SHAPE, ALIGN, KOVF, WS, HIP, CFG = range(8)


def test_exports_every_declared_function():
    names = w8.header_functions()
    assert len(names) >= 12
    out = subprocess.run(["nm", "-D", "--defined-only", w8.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for n in names:
        assert n in exported, n
        assert getattr(L, n) is not None


def test_status_strings():
    for s in range(8):
        assert w8.w8a8_status_string(s).startswith("W8A8_")
    assert "unknown" in w8.w8a8_status_string(123)


def test_quantize_validation():
    q = L.w8a8_quantize_act
    assert q(None, 0, 16, 16, None, 16, None, None) == OK          # nothing to do
    assert q(None, -1, 16, 16, None, 16, None, None) == SHAPE
    assert q(A, 4, 17, 17, A, 32, A, None) == SHAPE                 # K % 16
    assert q(A, 4, 32, 16, A, 32, A, None) == SHAPE                 # ldx < K
    assert q(A, 4, 32, 32, A, 16, A, None) == SHAPE                 # ldq < K
    assert q(None, 4, 16, 16, A, 16, A, None) == NULL
    assert q(A, 4, 16, 16, None, 16, A, None) == NULL
    assert q(A, 4, 16, 16, A, 16, None, None) == NULL
    assert q(MIS, 4, 16, 16, A, 16, A, None) == ALIGN
    assert q(A, 4, 16, 16, MIS, 16, A, None) == ALIGN
    assert q(A, 4, 16, 20, A, 16, A, None) == ALIGN                 # bf16 row stride 40 B
    assert q(A, 4, 16, 16, A, 24, A, None) == ALIGN                 # int8 row stride 24 B
    assert q(A, 4, 16, 16, A, 16, P(0x10002), None) == ALIGN        # fp32 scale
    assert q(A, 4, 133152, 133152, A, 133152, A, None) == KOVF
    w = L.w8a8_quantize_weight
    assert w(A, 4, 16, 18, A, 16, A, None) == ALIGN                 # fp32 row stride 72 B
    assert w(A, 4, 16, 16, A, 16, None, None) == NULL
    g = L.w8a8_gelu_quantize_act
    assert g(A, 4, 16, 16, A, 16, A, MIS, None) == ALIGN
    assert g(A, 4, 15, 16, A, 16, A, None, None) == SHAPE


def test_gemm_validation():
    g = L.w8a8_gemm_i32
    assert g(None, None, 0, 5, 16, None, None) == OK
    assert g(None, None, 5, 0, 16, None, None) == OK
    assert g(A, A, -1, 4, 16, A, None) == SHAPE
    assert g(A, A, 4, 4, 8, A, None) == SHAPE
    assert g(A, A, 4, 4, 133152, A, None) == KOVF
    assert g(A, A, 4, 4, 16, None, None) == NULL
    assert g(None, A, 4, 4, 16, A, None) == NULL
    assert g(A, MIS, 4, 4, 16, A, None) == ALIGN
    d = L.w8a8_gemm_dequant
    assert d(A, None, A, A, None, 4, 4, 16, A, None) == NULL        # s_x
    assert d(A, A, A, None, None, 4, 4, 16, A, None) == NULL        # s_w
    assert d(A, P(0x10002), A, A, None, 4, 4, 16, A, None) == ALIGN
    assert d(A, A, A, A, P(0x10001), 4, 4, 16, A, None) == ALIGN    # bias
    e = L.w8a8_gemm_ex
    assert e(A, A, A, A, None, 4, 4, 16, A, 0, 99, None) == CFG
    assert e(A, A, A, A, None, 4, 4, 16, A, 0, -2, None) == CFG
    assert e(A, A, A, A, None, 4, 4, 16, A, 1, w8.w8a8_gemm_num_configs(), None) == CFG


def test_linear_validation_and_workspace():
    ws = w8.w8a8_linear_workspace_bytes
    assert ws(0, 16) == 0
    assert ws(1, 16) == 256 + 256
    assert ws(4096, 3072) == 4096 * 3072 + 4096 * 4
    assert ws(3, 48) == 256 + 256
    assert ws(300, 1040) == (300 * 1040 + 255) // 256 * 256 + (1200 + 255) // 256 * 256
    lin = L.w8a8_linear
    need = ws(4, 16)
    assert lin(A, A, A, None, 4, 4, 16, A, None, need, None) == WS
    assert lin(A, A, A, None, 4, 4, 16, A, A, need - 1, None) == WS
    assert lin(A, A, A, None, 4, 4, 16, A, MIS, need, None) == ALIGN
    assert lin(A, A, A, None, 4, 4, 17, A, A, need, None) == SHAPE
    assert lin(A, A, A, None, 4, 4, 133152, A, A, 1 << 40, None) == KOVF
    assert lin(None, A, A, None, 4, 4, 16, A, A, need, None) == NULL
    assert lin(A, A, None, None, 4, 4, 16, A, A, need, None) == NULL
    assert lin(None, None, None, None, 0, 4, 16, None, None, 0, None) == OK


def test_config_selection_table():
    n = w8.w8a8_gemm_num_configs()
    names = [w8.w8a8_gemm_config_name(i) for i in range(n)]
    assert all(names) and len(set(names)) == n
    assert w8.w8a8_gemm_config_name(n) is None and w8.w8a8_gemm_config_name(-1) is None
    import synthetic
    for shapes in synthetic.CONFIGS.values():
        for s in shapes:
            c = w8.w8a8_gemm_select_config(s.M, s.N, s.K)
            assert 0 <= c < n, s
    assert w8.w8a8_gemm_select_config(0, 4, 16) == -1
    # the 256 x 384 ping-pong tile: the measured choice for the 1024px
    # up-projection; the cost model takes it only for shapes of whole tiles
    wide = names.index("bm256_bn384_bk64_s3_mf16_pp")
    assert w8.w8a8_gemm_select_config(4096, 12288, 3072) == wide
    assert w8.w8a8_gemm_select_config(8192, 12288, 3072) == wide
    assert w8.w8a8_gemm_select_config(8192, 12160, 3072) != wide   # N not a multiple of 384
    assert w8.w8a8_gemm_select_config(8192, 12288, 3000) != wide   # K not a multiple of 64
    # the K-split ping-pong tile: the measured choice for the 1024px
    # down-projection only (the cost model never takes it)
    ksplit = names.index("bm256_bn192_bk64_s5_mf16_ppk")
    assert w8.w8a8_gemm_select_config(4096, 3072, 12288) == ksplit
    assert w8.w8a8_gemm_select_config(8192, 3072, 12288) != ksplit
    assert w8.w8a8_gemm_select_config(4096, 3072, 6144) != ksplit


def test_fp8_entry_validation():
    q = L.w8a8_quantize_act_fp8
    assert q(None, 0, 16, 16, None, 16, None, None) == OK
    assert q(A, 4, 17, 17, A, 32, A, None) == SHAPE
    assert q(A, 4, 16, 16, A, 24, A, None) == ALIGN                 # code row stride 24 B
    assert q(A, 4, 16, 16, A, 16, None, None) == NULL
    w = L.w8a8_quantize_weight_fp8
    assert w(A, 4, 16, 18, A, 16, A, None) == ALIGN                 # fp32 row stride 72 B
    assert w(A, 4, 133152, 133152, A, 133152, A, None) == KOVF
    d = L.w8a8_gemm_dequant_fp8
    assert d(None, None, None, None, None, 0, 4, 16, None, None) == OK
    assert d(A, None, A, A, None, 4, 4, 16, A, None) == NULL        # s_x
    assert d(A, A, A, A, P(0x10001), 4, 4, 16, A, None) == ALIGN    # bias
    assert d(A, A, MIS, A, None, 4, 4, 16, A, None) == ALIGN
    e = L.w8a8_gemm_fp8_ex
    n = w8.w8a8_gemm_fp8_num_configs()
    assert n >= 1 and all(w8.w8a8_gemm_fp8_config_name(i) for i in range(n))
    assert w8.w8a8_gemm_fp8_config_name(n) is None
    assert e(A, A, A, A, None, 4, 4, 16, A, n, None) == CFG
    assert e(A, A, A, A, None, 4, 4, 16, A, -2, None) == CFG
    lin = L.w8a8_linear_fp8
    need = w8.w8a8_linear_workspace_bytes(4, 16)
    assert lin(A, A, A, None, 4, 4, 16, A, A, need - 1, None) == WS
    assert lin(A, A, A, None, 4, 4, 17, A, A, need, None) == SHAPE
    assert lin(None, None, None, None, 0, 4, 16, None, None, 0, None) == OK


def test_python_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros((4, 16), dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        w8.w8a8_quantize_act(x)
    with pytest.raises(TypeError):
        w8.w8a8_gemm_i32(torch.zeros((4, 16), dtype=torch.int8), torch.zeros((4, 16), dtype=torch.int8))


def test_module_swap_host_checks():
    import torch
    with pytest.raises(ValueError):
        w8.W8A8Linear(torch.zeros((4, 16), dtype=torch.float32), torch.ones(4))
    m = w8.W8A8Linear(torch.zeros((8, 32), dtype=torch.int8), torch.ones(8))
    assert (m.in_features, m.out_features) == (32, 8) and m.bias is None
    assert set(m.state_dict()) == {"w_q", "s_w"} and not m.fp8
    # uint8 codes select the FP8 (e4m3) variant
    f = w8.W8A8Linear(torch.zeros((8, 32), dtype=torch.uint8), torch.ones(8))
    assert f.fp8 and "e4m3" in repr(f)
    with pytest.raises(ValueError, match="not on a GPU"):
        w8.quantize_linears(torch.nn.Sequential(torch.nn.Linear(32, 64)), fp8=True)
    # a CPU model: layers the library takes are refused (no CPU path) ...
    cpu = torch.nn.Sequential(torch.nn.Linear(32, 64), torch.nn.GELU(), torch.nn.Linear(64, 8))
    with pytest.raises(ValueError, match="not on a GPU"):
        w8.quantize_linears(cpu)
    # ... layers it does not take (K % 16 != 0) are left alone, as is a filtered-out one
    odd = torch.nn.Sequential(torch.nn.Linear(24, 8), torch.nn.Linear(8, 3))
    assert w8.quantize_linears(odd) == 0
    assert w8.quantize_linears(cpu, include=lambda name, lin: False) == 0
    assert isinstance(cpu[0], torch.nn.Linear)
