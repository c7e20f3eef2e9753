"""The allocation-free fused linear (w8a8_linear_noalloc), called through the
C ABI: its output must equal w8a8_linear's (caller workspace) on the same
inputs, element for element, and the oracle's, on calls in a row, each with a
smaller input than the one before (the static scratch then still holds the
earlier calls' larger codes beyond the current one's; the last call, 8 token
rows, runs the single-launch few-row kernel); a problem larger than the
scratch is rejected with W8A8_ERR_SCRATCH before anything is enqueued."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import oracle
import w8a8_int8_quantized_quantize_amd as w8
from gpu_helpers import DEV, bits, dev_bf16, host
from test_gpu_parity import rand_bits

pytestmark = pytest.mark.gpu

W8A8_ERR_SCRATCH = 8


def _call_noalloc(x, wq, sw, b, y):
    lib = w8.raw()
    P = ctypes.c_void_p
    M, K = x.shape
    N = wq.shape[0]
    stream = P(torch.cuda.current_stream().cuda_stream)
    return lib.w8a8_linear_noalloc(P(x.data_ptr()), P(wq.data_ptr()), P(sw.data_ptr()),
                                   P(b.data_ptr()) if b is not None else None, M, N, K,
                                   P(y.data_ptr()), stream)


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_linear_matches_workspace_entry(order):
    assert w8.w8a8_linear_noalloc_max_bytes() == 64 << 20
    rng = np.random.default_rng(2024)
    for M, N, K, with_bias in [(4096, 1536, 3072, True), (300, 520, 1040, False),
                               (8, 3072, 3072, True)]:
        xb = rand_bits(rng, M, K, outliers=max(1, K // 100))
        w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
        bb = rand_bits(rng, 1, N, scale=0.1)[0] if with_bias else None
        wq, sw = w8.w8a8_quantize_weight(torch.from_numpy(w).to(DEV))
        x = dev_bf16(xb)
        b = dev_bf16(bb) if with_bias else None
        y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
        assert _call_noalloc(x, wq, sw, b, y) == 0
        ref = w8.w8a8_linear(x, wq, sw, b)       # caller-workspace entry, same kernels
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), (M, N, K)
        want = oracle.linear(xb, host(wq), host(sw), bb)
        assert np.array_equal(bits(y), want["y"]), (M, N, K)
        # the binding's wrapper of the same entry
        y2 = w8.w8a8_linear_noalloc(x, wq, sw, b)
        torch.cuda.synchronize()
        assert torch.equal(y2.view(torch.int16), y.view(torch.int16)), (M, N, K)


def test_noalloc_linear_rejects_problems_beyond_the_scratch():
    # 8193 x 8192 codes + scales exceed 64 MiB: rejected before any launch
    M, K, N = 8193, 8192, 16
    x = torch.zeros((M, K), dtype=torch.bfloat16, device=DEV)
    wq = torch.zeros((N, K), dtype=torch.int8, device=DEV)
    sw = torch.ones((N,), dtype=torch.float32, device=DEV)
    y = torch.full((M, N), 7.0, dtype=torch.bfloat16, device=DEV)
    assert w8.w8a8_linear_workspace_bytes(M, K) > w8.w8a8_linear_noalloc_max_bytes()
    assert _call_noalloc(x, wq, sw, None, y) == W8A8_ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())
    with pytest.raises(w8.W8A8Error):
        w8.w8a8_linear_noalloc(x, wq, sw)
