"""Pins for the CPU oracle: it is checked against what the mathematics fixes,
never against itself or the GPU path.

Each group names the plausible mistake it is there to catch.  Sources of truth:
hand-worked examples (tests/golden), closed forms, invariants, brute force with
exact Python integers / fractions on tiny inputs, and independent library
routines (torch's bf16 conversion, numpy's int64 matmul, scipy's erfc and
normal CDF).
"""
from __future__ import annotations

import bisect
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synthetic

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ helpers --
def torch_bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def all_bf16_finite_fractions():
    """Sorted list of (Fraction value, bits) for every finite non-negative bf16."""
    out = []
    for bits in range(0, 0x7F80):
        f = np.array([bits << 16], np.uint32).view(np.float32)[0]
        out.append((Fraction(float(f)), bits))
    return out


_BF16_TABLE = None


def brute_bf16_rne(d: float) -> int:
    """Nearest bf16 to the double d by exhaustive search over bf16 values;
    ties go to the pattern with an even last bit; beyond the largest finite
    value by half an ulp or more -> inf."""
    global _BF16_TABLE
    if _BF16_TABLE is None:
        _BF16_TABLE = all_bf16_finite_fractions()
        _BF16_TABLE_VALS = [v for v, _ in _BF16_TABLE]
        brute_bf16_rne.vals = _BF16_TABLE_VALS
    vals = brute_bf16_rne.vals
    sign = 0x8000 if math.copysign(1.0, d) < 0 else 0
    a = Fraction(abs(d))
    i = bisect.bisect_left(vals, a)
    if i < len(vals) and vals[i] == a:
        return sign | _BF16_TABLE[i][1]
    lo_v, lo_b = _BF16_TABLE[i - 1]
    if i == len(vals):  # above the largest finite value
        ulp = vals[-1] - vals[-2]
        hi_v, hi_b = vals[-1] + ulp, 0x7F80
    else:
        hi_v, hi_b = _BF16_TABLE[i]
    dl, dh = a - lo_v, hi_v - a
    if dl < dh:
        b = lo_b
    elif dh < dl:
        b = hi_b
    else:
        b = lo_b if lo_b % 2 == 0 else hi_b
    return sign | b


def read_quantize_cases():
    cases = []
    cur = {}
    with open(os.path.join(GOLDEN, "quantize_worked.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, vals = line.split(":", 1)
            cur[key] = vals.split()
            if key == "q":
                cases.append((np.array([float(v) for v in cur["x"]], np.float32),
                              float(cur["s"][0]),
                              np.array([int(v) for v in cur["q"]], np.int8)))
                cur = {}
    return cases


# ------------------------------------------------------------- bf16 (pins) --
def test_bf16_widening_all_patterns_matches_torch():
    # mistake caught: wrong shift / byte order in the widening
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.bf16_to_f32(bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    same = (ours.view(np.uint32) == ref.view(np.uint32))
    nan = np.isnan(ours) & np.isnan(ref)
    assert np.all(same | nan)


def test_f32_to_bf16_matches_torch_rne():
    # mistake caught: truncation, ties-away, mishandled subnormal/overflow
    rng = np.random.default_rng(1)
    parts = [rng.standard_normal(20000).astype(np.float32) * np.float32(10.0) ** rng.integers(-40, 38, 20000)]
    # exact ties: bf16 value + half an ulp
    base = torch_bf16_bits_from_f32(rng.standard_normal(5000).astype(np.float32)).astype(np.uint32) << 16
    parts.append((base | 0x8000).view(np.float32))
    parts.append((base | 0x7FFF).view(np.float32))
    parts.append((base | 0x8001).view(np.float32))
    # subnormals, extremes, zeros, infinities
    parts.append(np.array([0.0, -0.0, 1e-45, -1e-45, 3e-41, 9.2e-41, 4.6e-41, 1.1754942e-38,
                           3.3895314e38, 3.3961776e38, 3.4028235e38, -3.4028235e38,
                           np.inf, -np.inf], np.float32))
    x = np.concatenate(parts).astype(np.float32)
    ours = oracle.f32_to_bf16(x)
    ref = torch_bf16_bits_from_f32(x)
    assert np.array_equal(ours, ref)


def test_f64_to_bf16_single_rounding_brute_force():
    # mistake caught: rounding double -> float -> bf16 (double rounding), or a
    # wrong subnormal quantum.  Brute force over the whole bf16 value set.
    rng = np.random.default_rng(2)
    vals = list(rng.standard_normal(300) * 10.0 ** rng.integers(-30, 30, 300))
    # doubles just off a bf16 midpoint (where double rounding through fp32 errs)
    for _ in range(300):
        b = int(rng.integers(0x0080, 0x7F00))
        lo = float(np.array([b << 16], np.uint32).view(np.float32)[0])
        hi = float(np.array([(b + 1) << 16], np.uint32).view(np.float32)[0])
        mid = (lo + hi) / 2
        vals += [mid, mid + (hi - lo) * 2.0 ** -30, mid - (hi - lo) * 2.0 ** -30]
    # subnormal bf16 range and tiny values
    vals += [2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -135, 2.0 ** -126 - 2.0 ** -140, 1e-300, -2.5 * 2.0 ** -133]
    vals += [3.3961775e38, 3.39617752e38, 3.4e38, -1.0e39, 0.0, -0.0]
    vals = np.array(vals, np.float64)
    ours = oracle.f64_to_bf16(vals)
    ref = np.array([brute_bf16_rne(float(v)) for v in vals], np.uint16)
    assert np.array_equal(ours, ref)


# -------------------------------------------------------- quantize (pins) --
def test_quantize_worked_examples_golden():
    # mistakes caught: ties away from zero, divisor 128 / 127.5, asymmetric
    # zero point, clamp to -128, 0/0 on a zero row
    for x, s_exp, q_exp in read_quantize_cases():
        q, s = oracle.quantize_rows_f32(x[None, :])
        assert s[0] == np.float32(s_exp)
        assert np.array_equal(q[0], q_exp), (x, q[0], q_exp)
        xb = torch_bf16_bits_from_f32(x)[None, :]
        qb, sb = oracle.quantize_rows_bf16(xb)
        assert sb[0] == np.float32(s_exp) and np.array_equal(qb[0], q_exp)


def _fl32_div_exact(x: float, s: float) -> float:
    """The fp32 value nearest to x / s (ties to even), from exact fractions:
    search the neighbours of the double quotient in fp32."""
    exact = Fraction(x) / Fraction(s)
    c = np.float32(float(exact))
    cands = [np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))]
    best = min(cands, key=lambda v: (abs(Fraction(float(v)) - exact),
                                     int(np.array([v], np.float32).view(np.uint32)[0]) & 1))
    return float(best)


def _rne_int(v: float) -> int:
    f = math.floor(v)
    r = v - f
    if r > 0.5:
        return f + 1
    if r < 0.5:
        return f
    return f if f % 2 == 0 else f + 1


def test_quantize_brute_force_exact_fractions():
    # mistakes caught: reciprocal-multiply instead of division (differs on a
    # few elements per million), scale computed in double, missing abs in the
    # absmax.  Each code recomputed from exact rational arithmetic.
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((24, 96)) * np.exp(rng.uniform(-8, 8, (24, 1)))).astype(np.float32)
    x[5] *= -1
    x[6, 7] = -np.abs(x[6]).max() * 2  # negative absmax
    q, s = oracle.quantize_rows_f32(x)
    for r in range(x.shape[0]):
        amax = max(abs(float(v)) for v in x[r])
        s_ref = np.float32(_fl32_div_exact(amax, 127.0))
        assert s[r] == s_ref
        for k in range(x.shape[1]):
            t = _fl32_div_exact(float(x[r, k]), float(s_ref))
            qr = max(-127, min(127, _rne_int(t)))
            assert q[r, k] == qr, (r, k)


def test_quantize_division_not_reciprocal():
    # The quotient x / s and the product x * (127 / amax) disagree on some
    # elements; the oracle must follow the division.  Find such elements in a
    # large random draw and check the oracle picks the division's code.
    rng = np.random.default_rng(4)
    x = rng.standard_normal((512, 3072)).astype(np.float32)
    q, s = oracle.quantize_rows_f32(x)
    amax = np.abs(x).max(axis=1)
    s_np = (amax / np.float32(127.0)).astype(np.float32)
    assert np.array_equal(s, s_np)  # numpy fp32 division is IEEE
    div = np.clip(np.rint((x / s_np[:, None]).astype(np.float32)), -127, 127).astype(np.int8)
    rcp = np.clip(np.rint((x * (np.float32(127.0) / amax)[:, None]).astype(np.float32)), -127, 127).astype(np.int8)
    differ = div != rcp
    assert differ.sum() > 0  # the two readings are distinguishable on this draw
    assert np.array_equal(q[differ], div[differ])
    assert np.array_equal(q, div)


def test_quantize_invariants():
    rng = np.random.default_rng(5)
    xb = synthetic.bf16_bits(synthetic.bf16_from_f32(
        rng.standard_normal((64, 512)).astype(np.float32) * np.float32(3.0)))
    q, s = oracle.quantize_rows_bf16(xb)
    x = oracle.bf16_to_f32(xb).astype(np.float64)
    # every nonzero row reaches the full code range at its absmax
    assert np.all(np.abs(q.astype(np.int32)).max(axis=1) == 127)
    # symmetric: q(-x) = -q(x), same scale
    qn, sn = oracle.quantize_rows_bf16(xb ^ np.uint16(0x8000))
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)
    # scaling a row by 2^j scales the scale by 2^j and keeps the codes
    for j in (-20, -3, 1, 7, 40):
        xs = synthetic.bf16_bits(synthetic.bf16_from_f32((x * 2.0 ** j).astype(np.float32)))
        qj, sj = oracle.quantize_rows_bf16(xs)
        assert np.array_equal(qj, q)
        assert np.array_equal(sj.astype(np.float64), s.astype(np.float64) * 2.0 ** j)
    # reconstruction error: |x - q s| <= s (1/2 + 2^-17)  (exact in float64 here)
    err = np.abs(x - q.astype(np.float64) * s[:, None].astype(np.float64))
    assert np.all(err <= s[:, None] * (0.5 + 2.0 ** -17))


def test_quantize_tiny_and_zero_rows():
    # subnormal bf16 values keep a nonzero scale; an all-zero row -> scale 0
    tiny = np.array([[2.0 ** -133, -2.0 ** -132, 0.0, 3 * 2.0 ** -133]], np.float32)
    xb = torch_bf16_bits_from_f32(tiny)
    q, s = oracle.quantize_rows_bf16(xb)
    assert s[0] == np.float32(3 * 2.0 ** -133) / np.float32(127.0) and s[0] > 0
    assert abs(int(q[0, 3])) == 127
    zq, zs = oracle.quantize_rows_bf16(np.zeros((3, 32), np.uint16))
    assert np.all(zs == 0) and np.all(zq == 0)
    # fp32 weights so small that absmax / 127 underflows to zero -> zero codes
    w = np.array([[1e-45, -1e-45, 0.0]], np.float32)
    qw, sw = oracle.quantize_rows_f32(w)
    assert sw[0] == 0 and np.all(qw == 0)
    # a subnormal scale loses precision: absmax = 143 * 2^-149 gives scale
    # 2^-149, quotients +-143, and the clamp to [-127, 127] engages (never -128)
    t = np.array([[143 * 2.0 ** -149, -143 * 2.0 ** -149, 2.0 ** -149]], np.float32)
    qt, st_ = oracle.quantize_rows_f32(t)
    assert st_[0] == np.float32(2.0 ** -149)
    assert qt[0].tolist() == [127, -127, 1]


# ------------------------------------------------------------ GEMM (pins) --
def test_gemm_brute_force_python_ints():
    # mistakes caught: transposed operand, wrong index, narrow accumulator
    rng = np.random.default_rng(6)
    for M in range(1, 7):
        for N in (1, 3, 8):
            for K in (1, 2, 5, 8):
                a = rng.integers(-127, 128, (M, K)).astype(np.int8)
                b = rng.integers(-127, 128, (N, K)).astype(np.int8)
                acc = oracle.gemm_i64(a, b)
                for m in range(M):
                    for n in range(N):
                        assert acc[m, n] == sum(int(a[m, k]) * int(b[n, k]) for k in range(K))


def test_gemm_matches_numpy_int64_matmul():
    rng = np.random.default_rng(7)
    a = rng.integers(-127, 128, (37, 1040)).astype(np.int8)
    b = rng.integers(-127, 128, (53, 1040)).astype(np.int8)
    assert np.array_equal(oracle.gemm_i64(a, b), a.astype(np.int64) @ b.astype(np.int64).T)


def test_gemm_closed_forms():
    K = 3072
    ones = np.ones((4, K), np.int8)
    assert np.all(oracle.gemm_i64(ones, ones[:3]) == K)
    # W = 127 * I  (K = N) -> acc = 127 * q_x
    rng = np.random.default_rng(8)
    qx = rng.integers(-127, 128, (5, 64)).astype(np.int8)
    eye = (np.eye(64, dtype=np.int64) * 127).astype(np.int8)
    assert np.array_equal(oracle.gemm_i64(qx, eye), 127 * qx.astype(np.int64))
    # extremes at the largest K whose sums always fit int32 (K = 133136)
    Kmax = 133136
    p = np.full((1, Kmax), 127, np.int8)
    n = np.full((1, Kmax), -127, np.int8)
    assert oracle.gemm_i64(p, p)[0, 0] == 16129 * Kmax == 2147350544
    assert oracle.gemm_i64(p, n)[0, 0] == -16129 * Kmax
    assert 16129 * Kmax <= 2 ** 31 - 1 < 16129 * (Kmax + 16)


def test_gemm_k_permutation_invariance():
    rng = np.random.default_rng(9)
    a = rng.integers(-127, 128, (9, 200)).astype(np.int8)
    b = rng.integers(-127, 128, (11, 200)).astype(np.int8)
    perm = rng.permutation(200)
    assert np.array_equal(oracle.gemm_i64(a, b), oracle.gemm_i64(a[:, perm], b[:, perm]))


# -------------------------------------------------------- epilogue (pins) --
def test_epilogue_unit_scales_is_bf16_of_acc():
    # s_x = s_w = 1, no bias -> y = bf16_rne(float(acc)); float(acc) is exact
    # for |acc| <= 2^24 and RNE beyond; checked against torch's conversions.
    rng = np.random.default_rng(10)
    acc = rng.integers(-2 ** 31, 2 ** 31, (8, 16)).astype(np.int64)
    acc[0, :4] = [0, 1, -1, 2 ** 24 + 1]
    y = oracle.epilogue(acc, np.ones(8, np.float32), np.ones(16, np.float32))
    ref = torch.from_numpy(acc.astype(np.int32)).float().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(y, ref)


def test_epilogue_power_of_two_scales_exact():
    # mistakes caught: s_x indexed by n (or s_w by m), a scale dropped
    rng = np.random.default_rng(11)
    M, N = 6, 10
    acc = rng.integers(-3000, 3000, (M, N)).astype(np.int64)
    ex = rng.integers(-10, 10, M)
    ew = rng.integers(-10, 10, N)
    sx = (2.0 ** ex).astype(np.float32)
    sw = (2.0 ** ew).astype(np.float32)
    y = oracle.epilogue(acc, sx, sw)
    exact = acc * (2.0 ** ex)[:, None] * (2.0 ** ew)[None, :]  # exact in float64
    assert np.array_equal(y, torch_bf16_bits_from_f32(exact.astype(np.float32)))


def test_epilogue_bias_added_before_rounding():
    # mistakes caught: bias dropped, bias subtracted, bias added after the bf16
    # rounding.  Exact-sum cases: |acc| < 2^15, bias on a 2^-8 grid -> the fp32
    # sum is exact, so y = bf16_rne(acc + bias).
    rng = np.random.default_rng(12)
    M, N = 5, 64
    acc = rng.integers(-2 ** 15, 2 ** 15, (M, N)).astype(np.int64)
    bias_f = (rng.integers(-2 ** 14, 2 ** 14, N) / 256.0).astype(np.float32)
    bias_bits = torch_bf16_bits_from_f32(bias_f)
    bias_v = oracle.bf16_to_f32(bias_bits).astype(np.float64)
    y = oracle.epilogue(acc, np.ones(M, np.float32), np.ones(N, np.float32), bias_bits)
    exact = acc + bias_v[None, :]
    assert np.all(exact.astype(np.float32).astype(np.float64) == exact)
    assert np.array_equal(y, torch_bf16_bits_from_f32(exact.astype(np.float32)))
    # a case where adding the bias before vs after rounding differs
    a1 = np.array([[257]], np.int64)  # bf16(257) = 256
    b1 = torch_bf16_bits_from_f32(np.array([1.0], np.float32))
    y1 = oracle.epilogue(a1, np.ones(1, np.float32), np.ones(1, np.float32), b1)
    assert y1[0, 0] == torch_bf16_bits_from_f32(np.array([258.0], np.float32))[0]


def test_epilogue_order_without_fma_numpy_scalars():
    # General scales: each step is one IEEE fp32 operation, (s_x*s_w) first,
    # no fused multiply-add.  numpy float32 array operations are IEEE.  The
    # draw is large enough to contain elements where a fused multiply-add of
    # (s_x*s_w)*acc + bias rounds to a different bf16 (a few per million at
    # this accumulator range).
    rng = np.random.default_rng(13)
    M, N = 2048, 2048
    acc = rng.integers(-2 ** 20, 2 ** 20, (M, N)).astype(np.int64)
    sx = rng.uniform(1e-3, 1e-1, M).astype(np.float32)
    sw = rng.uniform(1e-5, 1e-3, N).astype(np.float32)
    bias_bits = torch_bf16_bits_from_f32(rng.standard_normal(N).astype(np.float32))
    y = oracle.epilogue(acc, sx, sw, bias_bits)
    bias_v = oracle.bf16_to_f32(bias_bits)
    f = (sx[:, None] * sw[None, :]).astype(np.float32)
    v = (f * acc.astype(np.float32)).astype(np.float32)
    o = (v + bias_v[None, :]).astype(np.float32)
    assert np.array_equal(y, torch_bf16_bits_from_f32(o))
    # the fused form: f*float(acc) is exact in float64 (24 + 24 bits)
    fused = (f.astype(np.float64) * acc.astype(np.float32).astype(np.float64)
             + bias_v[None, :].astype(np.float64)).astype(np.float32)
    assert np.count_nonzero(torch_bf16_bits_from_f32(fused) != y) > 0


def test_epilogue_rejects_int32_overflow():
    with pytest.raises(OverflowError):
        oracle.epilogue(np.array([[2 ** 31]], np.int64), np.ones(1, np.float32), np.ones(1, np.float32))


# ------------------------------------------------------------ GELU (pins) --
def test_gelu_table_values():
    rows = np.loadtxt(os.path.join(GOLDEN, "gelu_table.txt"))
    v, phi, g = rows[:, 0], rows[:, 1], rows[:, 2]
    ours = oracle.gelu_f64(v)
    assert np.allclose(ours, v * phi, rtol=1e-14, atol=1e-300)
    assert np.allclose(ours, g, rtol=1e-14, atol=1e-300)


def test_gelu_identity_and_libraries():
    import scipy.special
    import scipy.stats
    rng = np.random.default_rng(14)
    v = np.concatenate([rng.standard_normal(5000) * 4, rng.uniform(-30, 30, 2000)])
    g = oracle.gelu_f64(v)
    gn = oracle.gelu_f64(-v)
    # gelu(v) - gelu(-v) = v  (Phi(v) + Phi(-v) = 1)
    assert np.allclose(g - gn, v, rtol=1e-13, atol=1e-300)
    # independent implementations of erfc / Phi
    assert np.allclose(g, 0.5 * v * scipy.special.erfc(-v / np.sqrt(2.0)), rtol=1e-13, atol=1e-300)
    ok = np.abs(v) < 8
    assert np.allclose(g[ok], v[ok] * scipy.stats.norm.cdf(v[ok]), rtol=1e-9, atol=1e-300)


def test_gelu_bf16_special_values():
    vals = np.array([0.0, -0.0, 6.0, 8.0, 100.0, -1.0, -5.0, -6.0, -10.0, -13.0, -40.0], np.float32)
    bits = torch_bf16_bits_from_f32(vals)
    h = oracle.gelu_bf16(bits)
    hv = oracle.bf16_to_f32(h)
    assert hv[0] == 0 and hv[1] == 0
    assert np.array_equal(hv[2:5], vals[2:5])          # gelu(v) = v in bf16 for v >= 6
    assert np.all(hv[5:9] < 0)                          # small negative, not -0 (erfc form)
    assert hv[10] == 0 and np.signbit(hv[10])           # erfc underflow -> -0
    # every bf16 result is the single rounding of the fp64 value
    v = oracle.bf16_to_f32(bits).astype(np.float64)
    ref = np.array([brute_bf16_rne(float(x)) for x in oracle.gelu_f64(v)], np.uint16)
    assert np.array_equal(h, ref)


def test_gelu_bf16_all_patterns_single_rounding_sampled():
    # every finite bf16 input, against scipy's erfc rounded by brute force;
    # the two fp64 evaluations may differ in the last bits, which can flip a
    # bf16 rounding only when the value sits on a midpoint: allow <= 1 ulp.
    import scipy.special
    bits = np.arange(0, 65536, 7, dtype=np.uint32).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]  # finite inputs only
    v = oracle.bf16_to_f32(bits).astype(np.float64)
    fin = np.isfinite(v)
    bits, v = bits[fin], v[fin]
    h = oracle.gelu_bf16(bits)
    ref64 = 0.5 * v * scipy.special.erfc(-v / np.sqrt(2.0))
    sel = np.arange(0, v.size, 5)
    ref = np.array([brute_bf16_rne(float(x)) for x in ref64[sel]], np.uint16)
    got = h[sel]

    def key(b):
        b = b.astype(np.int32)
        return np.where(b & 0x8000, -(b & 0x7FFF), b)
    assert np.max(np.abs(key(got) - key(ref))) <= 1
    assert np.mean(got == ref) > 0.999


# ---------------------------------------------------- composite + golden --
def test_linear_composite_matches_parts_and_digest():
    import hashlib
    import json
    shape = synthetic.CONFIGS["unit"][0]
    st = synthetic.streams(0, shape.config_id, shape.layer_id)
    x = synthetic.bf16_bits(synthetic.activations_bf16(st, shape.M, shape.K))
    w = synthetic.weights_f32(st, shape.N, shape.K)
    b = synthetic.bf16_bits(synthetic.bias_bf16(st, shape.N))
    wq, sw = oracle.quantize_rows_f32(w)
    out = oracle.linear(x, wq, sw, b)
    # int32 range holds and the composite equals its parts
    assert np.abs(out["acc"]).max() <= 16129 * shape.K
    assert np.array_equal(out["acc"], out["q_x"].astype(np.int64) @ wq.astype(np.int64).T)
    with open(os.path.join(GOLDEN, "unit_oracle_digest.json")) as f:
        want = json.load(f)
    got = {k: hashlib.sha256(np.ascontiguousarray(v).tobytes()).hexdigest()
           for k, v in [("x", x), ("wq", wq), ("s_w", sw), ("q_x", out["q_x"]), ("s_x", out["s_x"]),
                        ("acc", out["acc"]), ("y", out["y"])]}
    assert got == want
