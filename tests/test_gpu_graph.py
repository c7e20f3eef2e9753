"""The fused linear and the GELU + quantize entry captured in a HIP graph.

The library enqueues kernels only (no allocation, no memset, no host
synchronization), so a caller can capture it.  The graph is replayed several
times with fresh inputs written eagerly in between; every replay is compared
with the eager result on the same inputs (bit-exact), and the eager result
with the oracle.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import w8a8_int8_quantized_quantize_amd as w8
from gpu_helpers import DEV, bits, dev_bf16, host

pytestmark = pytest.mark.gpu


def rand_bf16_bits(rng, M, K, scale=1.0):
    x = (rng.standard_normal((M, K)) * scale).astype(np.float32)
    return host(torch.from_numpy(x).to(torch.bfloat16).view(torch.int16)).view(np.uint16)


# (2304, 9216, 3072): the 768px QKV projection, whose GEMM runs the 256 x 384
# ping-pong tile
@pytest.mark.parametrize("M,N,K", [(2, 3072, 3072), (5, 3072, 3072), (300, 528, 1040), (1024, 1536, 3072),
                                   (2304, 9216, 3072)])
def test_graph_replay_matches_eager(M, N, K):
    rng = np.random.default_rng(M + N)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    wq, sw = w8.w8a8_quantize_weight(torch.from_numpy(w).to(DEV))
    b = dev_bf16(rand_bf16_bits(rng, 1, N, 0.1)[0])
    x = dev_bf16(rand_bf16_bits(rng, M, K))
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty((w8.w8a8_linear_workspace_bytes(M, K),), dtype=torch.uint8, device=DEV)
    q = torch.empty((M, N), dtype=torch.int8, device=DEV)
    s = torch.empty((M,), dtype=torch.float32, device=DEV)

    def body():
        w8.w8a8_linear(x, wq, sw, b, out=y, workspace=ws)
        w8.w8a8_gelu_quantize_act(y, q, s)

    side = torch.cuda.Stream()  # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        body()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        body()
    torch.cuda.synchronize()

    for rep in range(4):
        xb = rand_bf16_bits(rng, M, K)
        x.copy_(dev_bf16(xb))  # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        got_y, got_q, got_s = y.clone(), q.clone(), s.clone()
        # eager on the same input
        y2 = w8.w8a8_linear(x, wq, sw, b)
        q2, s2, _ = w8.w8a8_gelu_quantize_act(y2)
        torch.cuda.synchronize()
        assert torch.equal(got_y.view(torch.int16), y2.view(torch.int16)), rep
        assert torch.equal(got_q, q2) and torch.equal(got_s, s2), rep
        if rep == 0:
            rows = np.arange(0, M, max(1, M // 16))
            want = oracle.linear(xb[rows], host(wq), host(sw), bits(b))
            assert np.array_equal(bits(got_y)[rows], want["y"])


def test_graph_replay_fp8_linear():
    rng = np.random.default_rng(77)
    M, N, K = 300, 528, 1040
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    wq, sw = w8.w8a8_quantize_weight_fp8(torch.from_numpy(w).to(DEV))
    x = dev_bf16(rand_bf16_bits(rng, M, K))
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty((w8.w8a8_linear_workspace_bytes(M, K),), dtype=torch.uint8, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        w8.w8a8_linear_fp8(x, wq, sw, out=y, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        w8.w8a8_linear_fp8(x, wq, sw, out=y, workspace=ws)
    torch.cuda.synchronize()
    for rep in range(3):
        x.copy_(dev_bf16(rand_bf16_bits(rng, M, K)))
        g.replay()
        torch.cuda.synchronize()
        got = y.clone()
        want = w8.w8a8_linear_fp8(x, wq, sw)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), rep
    from test_gpu_fp8 import assert_fp8_gemm_bound
    qx, sx = oracle.quantize_rows_bf16_fp8(bits(x))
    assert_fp8_gemm_bound(bits(got), qx, sx, host(wq), host(sw), None, "graph fp8")


def test_module_graph_replay_after_larger_eager_calls():
    """W8A8Linear captured in a graph: its per-call workspace comes from the
    graph's memory pool, so eager calls with more tokens between replays
    (which take larger workspaces from the ordinary pool) cannot disturb the
    captured one.  Every replay equals the eager result on the same input."""
    rng = np.random.default_rng(91)
    M, N, K = 257, 1536, 3072
    w = torch.from_numpy((rng.standard_normal((N, K)) * 0.02).astype(np.float32)).to(DEV)
    b = torch.from_numpy((rng.standard_normal(N) * 0.1).astype(np.float32)).to(DEV)
    lin = w8.W8A8Linear.from_float(w, b)
    x = dev_bf16(rand_bf16_bits(rng, M, K))
    side = torch.cuda.Stream()  # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        lin(x)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        y = lin(x)
    torch.cuda.synchronize()
    for rep in range(3):
        big = dev_bf16(rand_bf16_bits(rng, 4 * M + rep, K))
        yb = lin(big)                       # eager, more tokens, own workspace
        x.copy_(dev_bf16(rand_bf16_bits(rng, M, K)))
        g.replay()
        torch.cuda.synchronize()
        got = y.clone()
        want = lin(x)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), rep
        wq, sw = host(lin.w_q), host(lin.s_w)
        rows = np.arange(0, 4 * M + rep, 97)
        ref = oracle.linear(bits(big)[rows], wq, sw, bits(lin.bias))
        assert np.array_equal(bits(yb)[rows], ref["y"]), rep
