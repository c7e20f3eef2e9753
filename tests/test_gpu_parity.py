"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bar: int8 codes, fp32 scales and int32 accumulators bit-exact; bf16 outputs
within 1 ulp (both sides use the same fp32 operation order, so they are
expected to be bit-exact and the count of non-identical elements is checked
to be zero as well), cosine >= 0.99999, no NaN/Inf.

Every comparison covers the whole output, element by element: small and mid
sizes that span several tiles of every kernel configuration with ragged M, N
and K tails, shapes where each persistent workgroup runs several tiles in a
row at the workloads' own K, and every GEMM of the five workloads at full
size, with the launch configuration the library selects (the one the
benchmark times).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synthetic
import w8a8_int8_quantized_quantize_amd as w8
from gpu_helpers import (DEV, assert_bf16_parity, bits, dev_bf16, host, shape_inputs,
                         ulp_dist)

pytestmark = pytest.mark.gpu

NCFG = None


def ncfg():
    global NCFG
    if NCFG is None:
        NCFG = w8.w8a8_gemm_num_configs()
    return NCFG


def rand_bits(rng, M, K, scale=1.0, outliers=0):
    x = rng.standard_normal((M, K)).astype(np.float32) * np.float32(scale)
    if outliers:
        x[:, rng.permutation(K)[:outliers]] *= np.float32(20.0)
    return synthetic.bf16_bits(synthetic.bf16_from_f32(x))


# ------------------------------------------------------------ quantization --
# (rows of 13-24 chunks per lane, K 6152..12288, are split between two waves:
# 5 x 12288, 3000 x 8192 and 7 x 10240, whose halves are shorter than 12 chunks)
QSHAPES = [(1, 16), (7, 48), (33, 1040), (64, 256), (257, 3072), (5, 12288), (3, 16384),
           (2, 24592), (1, 133136), (3000, 8192), (7, 10240)]


@pytest.mark.parametrize("M,K", QSHAPES)
def test_quantize_act_bit_exact(M, K):
    rng = np.random.default_rng(M * 7919 + K)
    xb = rand_bits(rng, M, K, outliers=max(1, K // 100))
    if M > 2:
        xb[1] = 0                                    # all-zero row
        xb[2] = rand_bits(rng, 1, K, scale=1e-39)[0]  # subnormal-range row
    q, s = w8.w8a8_quantize_act(dev_bf16(xb))
    qo, so = oracle.quantize_rows_bf16(xb)
    assert np.array_equal(host(s).view(np.uint32), so.view(np.uint32))
    assert np.array_equal(host(q), qo)


def test_quantize_act_ties_and_strided_rows():
    # rows with absmax 127 (scale 1) and exact .5 ties; a row stride > K
    vals = np.array([127, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5, 3.5, -3.5, 0, -127, 63.5, 64.5, 1, 2],
                    np.float32)
    xb = synthetic.bf16_bits(synthetic.bf16_from_f32(np.tile(vals, (3, 4))))
    big = np.zeros((3, 128), np.uint16)
    big[:, :64] = xb
    xt = dev_bf16(big)[:, :64]
    q, s = w8.w8a8_quantize_act(xt)
    qo, so = oracle.quantize_rows_bf16(xb)
    assert np.array_equal(host(q), qo) and np.array_equal(host(s), so)
    assert host(q)[0, :16].tolist() == [127, 0, 2, 2, 0, -2, -2, 126, 4, -4, 0, -127, 64, 64, 1, 2]


@pytest.mark.parametrize("N,K", [(128, 256), (300, 1040), (64, 12288), (3, 16)])
def test_quantize_weight_bit_exact(N, K):
    rng = np.random.default_rng(N + K)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    if N > 2:
        w[1] = 0
        w[2] = np.float32(2.0 ** -149) * rng.integers(-200, 200, K).astype(np.float32)
    q, s = w8.w8a8_quantize_weight(torch.from_numpy(w).to(DEV))
    qo, so = oracle.quantize_rows_f32(w)
    assert np.array_equal(host(s).view(np.uint32), so.view(np.uint32))
    assert np.array_equal(host(q), qo)


# large M: the persistent grid of 256 workgroups x 16 waves (one row per wave
# at a time) covers 4096 rows per pass; 4133 and 6000 take a second, partial
# pass.  Rows of 13-24 chunks per lane (K 6152..12288) are split between two
# waves, 8 rows per workgroup round: 4500 x 12288 takes a third, partial round
# (pairs past M idle through its barrier), 700 x 10240 and 37 x 7008 halves
# shorter than the per-lane chunk count, 100 x 8192 the 8-chunk halves.
@pytest.mark.parametrize("M,K", [(64, 256), (33, 3072), (8, 12288), (2, 16384), (4, 48),
                                 (4133, 3072), (6000, 1040), (4096, 12288), (4500, 12288),
                                 (700, 10240), (100, 8192), (37, 7008)])
def test_gelu_quantize_teacher_forced(M, K):
    rng = np.random.default_rng(M + 3 * K)
    yb = rand_bits(rng, M, K, scale=3.0, outliers=max(1, K // 100))
    q, s, h = w8.w8a8_gelu_quantize_act(dev_bf16(yb), want_h=True)
    ho = oracle.gelu_bf16(yb)
    hg = bits(h)
    d = ulp_dist(hg, ho)
    assert d.max() <= 1
    assert np.count_nonzero(d) == 0      # both sides round the same exact value once
    # codes and scales: bit-exact against the oracle's quantization of the
    # GPU's own GELU values (a 1-ulp GELU difference at a row's absmax would
    # otherwise move that row's scale)
    qo, so = oracle.quantize_rows_bf16(hg)
    assert np.array_equal(host(s), so) and np.array_equal(host(q), qo)
    # without the debug copy the codes are the same
    q2, s2, _ = w8.w8a8_gelu_quantize_act(dev_bf16(yb))
    assert torch.equal(q2, q) and torch.equal(s2, s)


def test_gelu_quantize_every_finite_bf16_pattern():
    # all 65280 finite bf16 inputs, 16 rows of 4080: h bit-exact, and the
    # codes and scales bit-exact against the oracle's own GELU + quantization
    pats = np.arange(65536, dtype=np.uint32)
    finite = (pats & 0x7F80) != 0x7F80
    yb = pats[finite].astype(np.uint16)
    np.random.default_rng(5).shuffle(yb)
    yb = yb.reshape(16, 4080)
    q, s, h = w8.w8a8_gelu_quantize_act(dev_bf16(yb), want_h=True)
    ho = oracle.gelu_bf16(yb)
    assert np.array_equal(bits(h), ho)
    qo, so = oracle.quantize_rows_bf16(ho)
    assert np.array_equal(host(s), so) and np.array_equal(host(q), qo)


# -------------------------------------------------------------------- GEMM --
# (600, 700, 1024): K a whole number of stages with ragged M and N, so that
# every tiled configuration runs both its interior-tile and edge-tile kernels;
# (520, 530, 256) and (520, 530, 128): interior tiles with no more K stages
# than LDS buffers (their epilogue vectors are waited for explicitly);
# (300, 768, 256) and (512, 768, 128): N a multiple of the 384-column tile but
# M ragged, or K shorter than its 3 stages, which the 256 x 384 ping-pong
# configuration hands to the 256 x 256 one
GSHAPES = [(64, 128, 256), (300, 520, 1040), (1, 16, 16), (7, 48, 48), (33, 272, 4112),
           (257, 16, 16), (16, 1000, 3072), (129, 257, 144), (3, 200, 12304), (600, 700, 1024),
           (520, 530, 256), (520, 530, 128), (300, 768, 256), (512, 768, 128)]


@pytest.mark.parametrize("M,N,K", GSHAPES)
def test_gemm_i32_bit_exact_every_config(M, N, K):
    rng = np.random.default_rng(M * 31 + N * 7 + K)
    a = rng.integers(-127, 128, (M, K)).astype(np.int8)
    b = rng.integers(-127, 128, (N, K)).astype(np.int8)
    want = oracle.gemm_i64(a, b)
    qa, qb = torch.from_numpy(a).to(DEV), torch.from_numpy(b).to(DEV)
    got = host(w8.w8a8_gemm_i32(qa, qb))
    assert np.array_equal(got.astype(np.int64), want)
    for c in range(ncfg()):
        g = host(w8.w8a8_gemm_ex(qa, None, qb, None, out_int32=True, config=c))
        assert np.array_equal(g.astype(np.int64), want), w8.w8a8_gemm_config_name(c)


def test_gemm_i32_extremes_at_max_k():
    K = w8.W8A8_MAX_K
    a = np.full((17, K), 127, np.int8)
    a[1::2] = -127
    b = np.full((18, K), 127, np.int8)
    b[::3] = -127
    qa, qb = torch.from_numpy(a).to(DEV), torch.from_numpy(b).to(DEV)
    got = host(w8.w8a8_gemm_i32(qa, qb))
    want = oracle.gemm_i64(a, b)
    assert np.abs(want).max() == 16129 * K
    assert np.array_equal(got.astype(np.int64), want)
    for c in range(ncfg()):
        g = host(w8.w8a8_gemm_ex(qa, None, qb, None, out_int32=True, config=c))
        assert np.array_equal(g.astype(np.int64), want), w8.w8a8_gemm_config_name(c)


@pytest.mark.parametrize("M,N,K", GSHAPES)
@pytest.mark.parametrize("with_bias", [True, False])
def test_linear_bf16_parity_every_config(M, N, K, with_bias):
    rng = np.random.default_rng(M + N + K + with_bias)
    xb = rand_bits(rng, M, K, outliers=max(1, K // 100))
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    bb = rand_bits(rng, 1, N, scale=0.1)[0] if with_bias else None
    wq, sw = w8.w8a8_quantize_weight(torch.from_numpy(w).to(DEV))
    wqo, swo = oracle.quantize_rows_f32(w)
    assert np.array_equal(host(wq), wqo) and np.array_equal(host(sw), swo)
    want = oracle.linear(xb, wqo, swo, bb)
    x = dev_bf16(xb)
    bias = dev_bf16(bb) if with_bias else None
    y = w8.w8a8_linear(x, wq, sw, bias)
    n_diff = assert_bf16_parity(bits(y), want["y"], f"linear {M}x{N}x{K}")
    assert n_diff == 0
    q, s = w8.w8a8_quantize_act(x)
    for c in range(ncfg()):
        yc = w8.w8a8_gemm_ex(q, s, wq, sw, bias, config=c)
        assert np.array_equal(bits(yc), want["y"]), w8.w8a8_gemm_config_name(c)


# More interior tiles than persistent workgroups, so workgroups run several
# tiles in a row.  M = 4096, N = 4352 (272 to 1088 interior tiles by
# configuration) with K from one LDS stage (tiles too short to prefetch the
# next tile's first stages from their own refills) to several; and the
# up-projection's own M = 4096, N = 12288 (768 tiles of 256 x 256: three per
# workgroup of that configuration, more for smaller tiles) at K = 384, 640 and
# 3072, where a workgroup's second and later tiles run the K-loop waits that
# let the previous tile's epilogue stores stay in flight (at least S - 1
# stages of the tile's own refills: K >= 384 for the 64-deep 4-stage tiles,
# K >= 512 for the 128-deep 3-stage ones).
@pytest.mark.parametrize("M,N,K", [(4096, 4352, 64), (4096, 4352, 128), (4096, 4352, 192),
                                   (4096, 4352, 320), (4096, 12288, 384), (4096, 12288, 640),
                                   (4096, 12288, 3072)])
def test_consecutive_interior_tiles_every_config(M, N, K):
    rng = np.random.default_rng(K)
    a = rng.integers(-127, 128, (M, K)).astype(np.int8)
    b = rng.integers(-127, 128, (N, K)).astype(np.int8)
    want = oracle.gemm_i64(a, b)
    qa, qb = torch.from_numpy(a).to(DEV), torch.from_numpy(b).to(DEV)
    for c in range(ncfg()):
        g = host(w8.w8a8_gemm_ex(qa, None, qb, None, out_int32=True, config=c))
        assert np.array_equal(g.astype(np.int64), want), w8.w8a8_gemm_config_name(c)
    del want, qa, qb
    xb = rand_bits(rng, M, K, outliers=1)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    bb = rand_bits(rng, 1, N, scale=0.1)[0]
    wq, sw = w8.w8a8_quantize_weight(torch.from_numpy(w).to(DEV))
    wqo, swo = oracle.quantize_rows_f32(w)
    assert np.array_equal(host(wq), wqo) and np.array_equal(host(sw), swo)
    yo = oracle.linear(xb, wqo, swo, bb)["y"]
    q, s = w8.w8a8_quantize_act(dev_bf16(xb))
    bias = dev_bf16(bb)
    for c in range(ncfg()):
        yc = w8.w8a8_gemm_ex(q, s, wq, sw, bias, config=c)
        assert np.array_equal(bits(yc), yo), w8.w8a8_gemm_config_name(c)


# The 256 x 384 ping-pong tile (configuration 14) on shapes of whole tiles:
# one tile at the minimum depth (3 stages, K = 192), four tiles, 216 tiles
# (one per workgroup, the 768px QKV projection's grid at a short K) and 432
# tiles at K = 192 (workgroups chain tiles whose K loop is no longer than
# the pipeline), each bit-exact against the oracle with and without a bias.
@pytest.mark.parametrize("M,N,K", [(256, 384, 192), (512, 768, 256), (2304, 9216, 320),
                                   (4608, 9216, 192)])
@pytest.mark.parametrize("with_bias", [True, False])
def test_wide_pingpong_tile_whole_tiles(M, N, K, with_bias):
    rng = np.random.default_rng(M + N + K + with_bias)
    xb = rand_bits(rng, M, K, outliers=max(1, K // 100))
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    bb = rand_bits(rng, 1, N, scale=0.1)[0] if with_bias else None
    wq, sw = w8.w8a8_quantize_weight(torch.from_numpy(w).to(DEV))
    wqo, swo = oracle.quantize_rows_f32(w)
    assert np.array_equal(host(wq), wqo) and np.array_equal(host(sw), swo)
    want = oracle.linear(xb, wqo, swo, bb)["y"]
    q, s = w8.w8a8_quantize_act(dev_bf16(xb))
    bias = dev_bf16(bb) if with_bias else None
    cfg = [c for c in range(ncfg()) if w8.w8a8_gemm_config_name(c) == "bm256_bn384_bk64_s3_mf16_pp"]
    assert len(cfg) == 1
    y = w8.w8a8_gemm_ex(q, s, wq, sw, bias, config=cfg[0])
    assert np.array_equal(bits(y), want)


# The K-split ping-pong kernel (configuration 15) on shapes of whole 256 x 192
# tiles: one tile at the minimum depth (K = 256: two k-steps per group),
# four tiles, 256 tiles (one per workgroup, the 1024px down-projection's grid
# at a short K) and 288 tiles (workgroups that run a second tile after
# draining the first), each bit-exact against the oracle with and without a
# bias.
@pytest.mark.parametrize("M,N,K", [(256, 192, 256), (512, 384, 384), (4096, 3072, 512),
                                   (4608, 3072, 256)])
@pytest.mark.parametrize("with_bias", [True, False])
def test_ksplit_pingpong_whole_tiles(M, N, K, with_bias):
    rng = np.random.default_rng(3 * M + N + K + with_bias)
    xb = rand_bits(rng, M, K, outliers=max(1, K // 100))
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    bb = rand_bits(rng, 1, N, scale=0.1)[0] if with_bias else None
    wq, sw = w8.w8a8_quantize_weight(torch.from_numpy(w).to(DEV))
    wqo, swo = oracle.quantize_rows_f32(w)
    assert np.array_equal(host(wq), wqo) and np.array_equal(host(sw), swo)
    want = oracle.linear(xb, wqo, swo, bb)["y"]
    q, s = w8.w8a8_quantize_act(dev_bf16(xb))
    bias = dev_bf16(bb) if with_bias else None
    cfg = [c for c in range(ncfg()) if w8.w8a8_gemm_config_name(c) == "bm256_bn192_bk64_s5_mf16_ppk"]
    assert len(cfg) == 1
    y = w8.w8a8_gemm_ex(q, s, wq, sw, bias, config=cfg[0])
    assert np.array_equal(bits(y), want)


def _at_offset(t: torch.Tensor, k: int) -> torch.Tensor:
    """A copy of 1-D t that starts k elements into a fresh allocation."""
    big = torch.zeros(t.numel() + k, dtype=t.dtype, device=DEV)
    big[k:] = t
    return big[k:]


# Scale and bias vectors at offsets the ABI accepts but the vector epilogue
# cannot take (s_x, s_w 4 bytes past a 16-byte boundary, bias 2 bytes): the
# interior tiles then read them element by element (and the 256 x 256
# ping-pong configuration runs its 8-wave generic kernel).  Every int8
# configuration bit-exact against the oracle, every FP8 one equal to its own
# output with aligned vectors.
@pytest.mark.parametrize("M,N,K", [(512, 768, 512), (600, 700, 1024)])
def test_unaligned_scale_and_bias_vectors_every_config(M, N, K):
    rng = np.random.default_rng(M + 3 * N + K)
    xb = rand_bits(rng, M, K, outliers=max(1, K // 100))
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    bb = rand_bits(rng, 1, N, scale=0.1)[0]
    wd = torch.from_numpy(w).to(DEV)
    wq, sw = w8.w8a8_quantize_weight(wd)
    wqo, swo = oracle.quantize_rows_f32(w)
    want = oracle.linear(xb, wqo, swo, bb)["y"]
    x, bias = dev_bf16(xb), dev_bf16(bb)
    q, s = w8.w8a8_quantize_act(x)
    s1, sw1, b1 = _at_offset(s, 1), _at_offset(sw, 1), _at_offset(bias, 1)
    assert s1.data_ptr() % 16 == 4 and sw1.data_ptr() % 16 == 4 and b1.data_ptr() % 16 == 2
    for c in range(ncfg()):
        yc = w8.w8a8_gemm_ex(q, s1, wq, sw1, b1, config=c)
        assert np.array_equal(bits(yc), want), w8.w8a8_gemm_config_name(c)
    qf, sf = w8.w8a8_quantize_act_fp8(x)
    wf, swf = w8.w8a8_quantize_weight_fp8(wd)
    sf1, swf1 = _at_offset(sf, 1), _at_offset(swf, 1)
    for c in range(w8.w8a8_gemm_fp8_num_configs()):
        ya = w8.w8a8_gemm_dequant_fp8(qf, sf, wf, swf, bias, config=c)
        yu = w8.w8a8_gemm_dequant_fp8(qf, sf1, wf, swf1, b1, config=c)
        assert torch.equal(ya, yu), w8.w8a8_gemm_fp8_config_name(c)


def test_linear_k_zero_is_bias_and_empty_batches():
    N = 40
    rng = np.random.default_rng(5)
    bb = rand_bits(rng, 1, N, scale=0.1)[0]
    wq = torch.zeros((N, 0), dtype=torch.int8, device=DEV)
    sw = torch.ones((N,), dtype=torch.float32, device=DEV)
    x = torch.zeros((3, 0), dtype=torch.bfloat16, device=DEV)
    y = w8.w8a8_linear(x, wq, sw, dev_bf16(bb))
    assert np.array_equal(bits(y), np.tile(bb, (3, 1)))
    y0 = w8.w8a8_linear(x, wq, sw)  # no bias: (s_x * s_w) * 0 = +0
    assert np.all(bits(y0) == 0)
    # every kernel configuration with K == 0 (no operand bytes exist to load)
    q0 = torch.zeros((3, 0), dtype=torch.int8, device=DEV)
    sx0 = torch.ones((3,), dtype=torch.float32, device=DEV)
    for c in range(ncfg()):
        yc = w8.w8a8_gemm_ex(q0, sx0, wq, sw, dev_bf16(bb), config=c)
        assert np.array_equal(bits(yc), np.tile(bb, (3, 1))), w8.w8a8_gemm_config_name(c)
        gi = w8.w8a8_gemm_ex(q0, None, wq, None, None, out_int32=True, config=c)
        assert not host(gi).any(), w8.w8a8_gemm_config_name(c)
    # M = 0 and N = 0
    e = w8.w8a8_linear(torch.zeros((0, 32), dtype=torch.bfloat16, device=DEV),
                       torch.zeros((N, 32), dtype=torch.int8, device=DEV), sw)
    assert e.shape == (0, N)
    e2 = w8.w8a8_gemm_i32(torch.zeros((5, 32), dtype=torch.int8, device=DEV),
                          torch.zeros((0, 32), dtype=torch.int8, device=DEV))
    assert e2.shape == (5, 0)
    q, s = w8.w8a8_quantize_act(torch.zeros((0, 64), dtype=torch.bfloat16, device=DEV))
    assert q.shape == (0, 64) and s.shape == (0,)


def test_deterministic_and_stream_ordered():
    rng = np.random.default_rng(11)
    M, N, K = 300, 520, 1040
    x = dev_bf16(rand_bits(rng, M, K))
    wq, sw = w8.w8a8_quantize_weight(torch.from_numpy((rng.standard_normal((N, K)) * 0.02).astype(np.float32)).to(DEV))
    ref = w8.w8a8_linear(x, wq, sw)
    s = torch.cuda.Stream()  # default priority
    with torch.cuda.stream(s):
        outs = [w8.w8a8_linear(x, wq, sw) for _ in range(3)]
    s.synchronize()
    for o in outs:
        assert torch.equal(o.view(torch.int16), ref.view(torch.int16))


def test_int_mm_cross_check_where_available():
    # The pages check the int32 accumulators against torch._int_mm; do the same
    # where this PyTorch build provides it on the device.
    rng = np.random.default_rng(12)
    M, N, K = 64, 128, 256
    a = torch.from_numpy(rng.integers(-127, 128, (M, K)).astype(np.int8)).to(DEV)
    b = torch.from_numpy(rng.integers(-127, 128, (N, K)).astype(np.int8)).to(DEV)
    try:
        ref = torch._int_mm(a, b.t().contiguous())
    except Exception as e:  # not supported by this PyTorch or shape
        pytest.skip(f"torch._int_mm unavailable: {e}")
    assert torch.equal(w8.w8a8_gemm_i32(a, b), ref)


# ---------------------------------------------------- full workload sizes --
def _full_linear_check(shape, x_bits):
    """The fused linear at full size on the GPU against the oracle, whole
    output: int8 codes and scales bit-exact, every bf16 element identical."""
    _, w, b = shape_inputs(shape)
    wq, sw = w8.w8a8_quantize_weight(torch.from_numpy(w).to(DEV))
    wqo, swo = oracle.quantize_rows_f32(w)
    assert np.array_equal(host(wq), wqo) and np.array_equal(host(sw), swo)
    x = dev_bf16(x_bits)
    y = w8.w8a8_linear(x, wq, sw, dev_bf16(b))
    q, s = w8.w8a8_quantize_act(x)
    want = oracle.linear(x_bits, wqo, swo, b)
    assert np.array_equal(host(q), want["q_x"]) and np.array_equal(host(s), want["s_x"])
    assert np.abs(want["acc"]).max() <= 16129 * shape.K
    yb = bits(y)
    n_diff = assert_bf16_parity(yb, want["y"], shape.name)
    assert n_diff == 0
    return yb


FULL = [s for k in ("unit", "dit768_attn", "skinny") for s in synthetic.CONFIGS[k]] + \
       [synthetic.CONFIGS["dit1024_mlp"][0]]


@pytest.mark.parametrize("shape", FULL, ids=lambda s: s.name)
def test_full_size_linear(shape):
    x, _, _ = shape_inputs(shape)
    _full_linear_check(shape, x)


def test_full_size_mlp_down_with_gelu_input():
    # down-proj input: GELU of a random bf16 tensor with outlier columns
    shape = synthetic.CONFIGS["dit1024_mlp"][1]
    r, _, _ = shape_inputs(shape)
    q, s, h = w8.w8a8_gelu_quantize_act(dev_bf16(r), want_h=True)
    hb = bits(h)
    assert np.array_equal(hb, oracle.gelu_bf16(r))
    qo, so = oracle.quantize_rows_bf16(hb)
    assert np.array_equal(host(q), qo) and np.array_equal(host(s), so)
    _, w, b = shape_inputs(shape)
    wq, sw = w8.w8a8_quantize_weight(torch.from_numpy(w).to(DEV))
    y = bits(w8.w8a8_gemm_dequant(q, s, wq, sw, dev_bf16(b)))
    wqo, swo = oracle.quantize_rows_f32(w)
    want = oracle.linear_prequant(qo, so, wqo, swo, b)
    assert assert_bf16_parity(y, want["y"], shape.name) == 0


def test_full_size_dit_block_chain():
    """QKV -> out-proj (random stand-in for attention) -> up -> GELU -> down,
    re-quantizing per token between layers, all 4608 rows.  Each stage
    teacher-forced on the GPU's own input (whole outputs bit-exact); the whole
    chain also against an un-forced oracle chain by cosine."""
    qkv, out, up, down = synthetic.CONFIGS["dit1024_chain"]
    M = qkv.M
    layers = {}
    for s in (qkv, out, up, down):
        _, w, b = shape_inputs(s)
        wq, sw = w8.w8a8_quantize_weight(torch.from_numpy(w).to(DEV))
        layers[s.name] = (wq, sw, dev_bf16(b), oracle.quantize_rows_f32(w), b)
    x0, _, _ = shape_inputs(qkv)
    a_bits, _, _ = shape_inputs(synthetic.GemmShape("attn_standin", M, 3072, 3072, 0.0, 5, 9))

    def run(s, xb_dev):
        wq, sw, bd, _, _ = layers[s.name]
        return w8.w8a8_linear(xb_dev, wq, sw, bd)

    def oracle_y(s, x_bits):
        _, _, _, (wqo, swo), b = layers[s.name]
        return oracle.linear(x_bits, wqo, swo, b)["y"]

    y_qkv = bits(run(qkv, dev_bf16(x0)))
    assert assert_bf16_parity(y_qkv, oracle_y(qkv, x0), "qkv") == 0
    del y_qkv
    y1 = run(out, dev_bf16(a_bits))
    y1b = bits(y1)
    c1 = oracle_y(out, a_bits)
    assert assert_bf16_parity(y1b, c1, "out") == 0
    y2 = run(up, y1)
    y2b = bits(y2)
    assert assert_bf16_parity(y2b, oracle_y(up, y1b), "up") == 0
    qh, sh, h = w8.w8a8_gelu_quantize_act(y2, want_h=True)
    hb = bits(h)
    assert np.array_equal(hb, oracle.gelu_bf16(y2b))
    qo, so = oracle.quantize_rows_bf16(hb)
    assert np.array_equal(host(qh), qo) and np.array_equal(host(sh), so)
    wq, sw, bd, (wqo, swo), b = layers[down.name]
    y3 = bits(w8.w8a8_gemm_dequant(qh, sh, wq, sw, bd))
    want3 = oracle.linear_prequant(qo, so, wqo, swo, b)["y"]
    assert assert_bf16_parity(y3, want3, "down") == 0
    # the un-forced oracle chain (the stages above agree bit for bit, so the
    # chains agree too; the cosine is the end-to-end bar)
    c2 = oracle_y(up, c1)
    qo2, so2 = oracle.quantize_rows_bf16(oracle.gelu_bf16(c2))
    c3 = oracle.linear_prequant(qo2, so2, wqo, swo, b)["y"]
    from gpu_helpers import cosine
    assert cosine(y3, c3) >= 0.99999


# A handful of token rows: w8a8_linear runs quantization, GEMM and epilogue in
# one launch (up to 16 rows with at most 256 column blocks, 12 with more; K <=
# 3072) and leaves the codes and scales in its workspace either way; (13,
# 4112, 1040) and (16, 18432, 3072) take the two launches.  Every row split of
# that kernel (4 waves: 4 or 2 waves per row or one row per wave; 8 waves: one
# or two rows per wave).  Rows include an all-zero row and one whose scale is
# subnormal (the division path of the quantizer), K with a ragged 64-element
# step, and N not a multiple of 16.
@pytest.mark.parametrize("M,N,K", [(1, 3072, 3072), (4, 3072, 3072), (3, 100, 1040), (3, 16, 16),
                                   (1, 18432, 3072), (2, 40, 48), (4, 272, 2000), (1, 16, 3072),
                                   (2, 3072, 3072), (6, 528, 1040), (8, 3072, 3072),
                                   (12, 3072, 3072), (16, 3072, 3072), (9, 272, 2000),
                                   (12, 18432, 3072), (13, 4112, 1040), (16, 18432, 3072),
                                   (16, 272, 2000), (12, 16, 16), (5, 48, 48), (7, 40, 48),
                                   (14, 100, 1040)])
def test_few_rows_single_launch_linear_and_workspace(M, N, K):
    rng = np.random.default_rng(M * 100 + K + N)
    xb = rand_bits(rng, M, K, outliers=max(1, K // 100))
    if M >= 3:
        xb[1] = 0                                    # all-zero row
        xb[2] = rand_bits(rng, 1, K, scale=1e-39)[0]  # subnormal-range row
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    bb = rand_bits(rng, 1, N, scale=0.1)[0]
    wq, sw = w8.w8a8_quantize_weight(torch.from_numpy(w).to(DEV))
    wqo, swo = oracle.quantize_rows_f32(w)
    ws = torch.full((w8.w8a8_linear_workspace_bytes(M, K),), 0x55, dtype=torch.uint8, device=DEV)
    for bias in (dev_bf16(bb), None):
        y = w8.w8a8_linear(dev_bf16(xb), wq, sw, bias, workspace=ws)
        want = oracle.linear(xb, wqo, swo, bb if bias is not None else None)
        assert np.array_equal(bits(y), want["y"])
        pad = (M * K + 255) // 256 * 256
        codes = host(ws[:M * K]).view(np.int8).reshape(M, K)
        scales = host(ws[pad:pad + 4 * M]).view(np.float32)
        assert np.array_equal(codes, want["q_x"])
        assert np.array_equal(scales.view(np.uint32), want["s_x"].view(np.uint32))
