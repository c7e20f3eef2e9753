"""The inter-layer fusion variant of the DiT MLP (GELU and the per-token
absmax of the next quantization folded into the up-projection's epilogue,
then a quantization pass that reuses those row maxima):

  w8a8_gemm_dequant_gelu_amax -> h, amax;  w8a8_quantize_act_amax(h, amax) -> q, s

Bar: h bit-exact against the oracle's GELU of the oracle's linear output
(both sides round the same exact GELU value of the same bf16 y once); amax
equal to max |h| per row; codes and scales bit-exact against the oracle's
quantization of h, and equal to what w8a8_gelu_quantize_act computes from
the plain GEMM's output (the path this variant replaces).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synthetic
import w8a8_int8_quantized_quantize_amd as w8
from gpu_helpers import DEV, bits, dev_bf16, host, shape_inputs
from test_gpu_parity import rand_bits

pytestmark = pytest.mark.gpu


def _check(xb, w, bb, M, N, K):
    wq, sw = w8.w8a8_quantize_weight(torch.from_numpy(w).to(DEV))
    wqo, swo = oracle.quantize_rows_f32(w)
    x = dev_bf16(xb)
    q, s = w8.w8a8_quantize_act(x)
    bias = dev_bf16(bb) if bb is not None else None
    h, amax = w8.w8a8_gemm_dequant_gelu_amax(q, s, wq, sw, bias)
    qh, sh = w8.w8a8_quantize_act_amax(h, amax)
    torch.cuda.synchronize()
    want_y = oracle.linear(xb, wqo, swo, bb)["y"]
    want_h = oracle.gelu_bf16(want_y)
    hb = bits(h)
    assert np.array_equal(hb, want_h)
    mag = oracle.bf16_to_f32(hb & 0x7FFF).reshape(M, N).max(axis=1)
    assert np.array_equal(host(amax).view(np.uint32), mag.astype(np.float32).view(np.uint32))
    qo, so = oracle.quantize_rows_bf16(want_h)
    assert np.array_equal(host(qh), qo) and np.array_equal(host(sh), so)
    # the path it replaces: plain GEMM, then GELU + quantization
    y = w8.w8a8_gemm_dequant(q, s, wq, sw, bias)
    q2, s2, _ = w8.w8a8_gelu_quantize_act(y)
    assert torch.equal(q2, qh) and torch.equal(s2, sh)


@pytest.mark.parametrize("M,N,K,with_bias", [(512, 768, 1024, True), (256, 256, 256, False),
                                             (768, 512, 3072, True)])
def test_gelu_epilogue_and_amax_quantizer(M, N, K, with_bias):
    rng = np.random.default_rng(M + N + K)
    xb = rand_bits(rng, M, K, outliers=max(1, K // 100))
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    bb = rand_bits(rng, 1, N, scale=0.1)[0] if with_bias else None
    _check(xb, w, bb, M, N, K)


def test_gelu_epilogue_full_size_mlp_up():
    shape = synthetic.CONFIGS["dit1024_mlp"][0]
    x, w, b = shape_inputs(shape)
    _check(x, w, b, shape.M, shape.N, shape.K)


def test_gelu_epilogue_rejects_shapes_it_does_not_take():
    rng = np.random.default_rng(3)
    q = torch.from_numpy(rng.integers(-127, 128, (300, 512)).astype(np.int8)).to(DEV)
    wq = torch.from_numpy(rng.integers(-127, 128, (256, 512)).astype(np.int8)).to(DEV)
    s = torch.ones(300, device=DEV)
    sw = torch.ones(256, device=DEV)
    with pytest.raises(w8.W8A8Error):
        w8.w8a8_gemm_dequant_gelu_amax(q, s, wq, sw)
