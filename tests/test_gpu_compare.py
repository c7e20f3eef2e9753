"""The pages' comparison baseline, the "fake INT8" forward (bench.py
--compare): per-token int8 quantization, then activations and weights
dequantized to bf16 and multiplied by a bf16 GEMM (Abstract; news write-up,
second paragraph).  Checked at one small shape:
  * its dequantized operands equal the oracle's codes times scales, one fp32
    product each, rounded once to bf16 (the oracle's own bf16 rounding);
  * its output is within a bf16-GEMM bound of the fp64 product of those
    operands: the products of bf16 values are exact in fp32, the GEMM sums K
    of them in fp32 (|error| <= K * 2^-24 * sum_k |xd_k wd_k|, the classical
    bound for any summation order), adds the bias, and rounds to bf16
    (<= 2^-8 of |y|; a GEMM that rounds its sum to bf16 before the bias add
    adds at most 2^-9 of |sum| more);
  * against the fused INT8 linear its cosine is >= 0.9999 (same codes and
    scales; the two differ by the bf16 rounding of the dequantized operands).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import bench
import oracle
import w8a8_int8_quantized_quantize_amd as w8
from gpu_helpers import DEV, bits, cosine, dev_bf16, host
from test_gpu_parity import rand_bits

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,K,N", [(256, 3072, 512), (64, 256, 128)])
def test_fake_int8_leg(M, K, N):
    rng = np.random.default_rng(M + K + N)
    xb = rand_bits(rng, M, K, outliers=max(1, K // 100))
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    bb = rand_bits(rng, 1, N, scale=0.1)[0]
    wq, sw = w8.w8a8_quantize_weight(torch.from_numpy(w).to(DEV))
    x, b = dev_bf16(xb), dev_bf16(bb)
    y, xd, wd = bench.fake_int8_forward(w8, x, wq, sw, b, operands=True)
    torch.cuda.synchronize()
    # the dequantized operands: the oracle's codes x scales, fp32, then bf16
    qo, so = oracle.quantize_rows_bf16(xb)
    wqo, swo = oracle.quantize_rows_f32(w)
    xd_want = oracle.f32_to_bf16((qo.astype(np.float32) * so[:, None]).astype(np.float32))
    wd_want = oracle.f32_to_bf16((wqo.astype(np.float32) * swo[:, None]).astype(np.float32))
    assert np.array_equal(bits(xd), xd_want)
    assert np.array_equal(bits(wd), wd_want)
    # the bf16 GEMM against the fp64 product of those operands
    xv = oracle.bf16_to_f32(xd_want).astype(np.float64)
    wv = oracle.bf16_to_f32(wd_want).astype(np.float64)
    bv = oracle.bf16_to_f32(bb).astype(np.float64)
    prod = xv @ wv.T
    exact = prod + bv[None, :]
    mag = np.abs(xv) @ np.abs(wv).T + np.abs(bv)[None, :]
    got = oracle.bf16_to_f32(bits(y)).astype(np.float64)
    assert np.all(np.isfinite(got))
    tol = (K + 1) * 2.0 ** -24 * mag + 2.0 ** -8 * np.abs(exact) + 2.0 ** -9 * np.abs(prod) + 1e-30
    assert np.all(np.abs(got - exact) <= tol), float((np.abs(got - exact) / tol).max())
    # the fused INT8 linear on the same inputs
    yi = w8.w8a8_linear(x, wq, sw, b)
    assert cosine(bits(yi), bits(y)) >= 0.9999
