"""The library on several streams and host threads at once.

The entry points keep no per-call state on the host (only per-device caches
of values that depend on the device alone), and every kernel reads and writes
only the caller's buffers, so calls on different streams may overlap freely.
Here three problems of different shapes (so different kernels: the
ping-pong tile, the tiled kernel with edge tiles, the single-launch few-row
linear) run interleaved on three streams, then from three host threads each
with its own stream; every output must equal the oracle's, bit for bit.
"""
from __future__ import annotations

import threading

import numpy as np
import pytest
import torch

import oracle
import w8a8_int8_quantized_quantize_amd as w8
from gpu_helpers import DEV, bits, dev_bf16
from test_gpu_parity import rand_bits

pytestmark = pytest.mark.gpu

SHAPES = [(1024, 1536, 3072), (300, 528, 1040), (3, 3072, 3072)]
CALLS = 4


def _problems():
    probs = []
    for i, (M, N, K) in enumerate(SHAPES):
        rng = np.random.default_rng(100 + i)
        w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
        wqo, swo = oracle.quantize_rows_f32(w)
        wq, sw = w8.w8a8_quantize_weight(torch.from_numpy(w).to(DEV))
        bb = rand_bits(rng, 1, N, scale=0.1)[0]
        xs = [rand_bits(rng, M, K, outliers=max(1, K // 100)) for _ in range(CALLS)]
        wants = [oracle.linear(xb, wqo, swo, bb)["y"] for xb in xs]
        probs.append(dict(
            x=[dev_bf16(xb) for xb in xs], wq=wq, sw=sw, b=dev_bf16(bb), want=wants,
            y=[torch.empty((M, N), dtype=torch.bfloat16, device=DEV) for _ in range(CALLS)],
            ws=torch.empty((w8.w8a8_linear_workspace_bytes(M, K),), dtype=torch.uint8, device=DEV)))
    torch.cuda.synchronize()
    return probs


def _check(probs):
    for p in probs:
        for c in range(CALLS):
            assert np.array_equal(bits(p["y"][c]), p["want"][c])


def test_interleaved_streams():
    probs = _problems()
    streams = [torch.cuda.Stream() for _ in probs]  # default priority
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for c in range(CALLS):
        for p, s in zip(probs, streams):
            with torch.cuda.stream(s):
                # a call's workspace is reused by the next call on the same stream only
                w8.w8a8_linear(p["x"][c], p["wq"], p["sw"], p["b"], out=p["y"][c], workspace=p["ws"])
    torch.cuda.synchronize()
    _check(probs)


def test_host_threads_each_with_a_stream():
    probs = _problems()
    errors = []

    def run(p):
        try:
            s = torch.cuda.Stream()  # default priority
            with torch.cuda.stream(s):
                for c in range(CALLS):
                    w8.w8a8_linear(p["x"][c], p["wq"], p["sw"], p["b"], out=p["y"][c],
                                   workspace=p["ws"])
            s.synchronize()
        except Exception as e:  # reported in the main thread
            errors.append(e)

    threads = [threading.Thread(target=run, args=(p,)) for p in probs]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    torch.cuda.synchronize()
    _check(probs)
