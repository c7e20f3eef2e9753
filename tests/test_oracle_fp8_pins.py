"""Pins of the oracle's FP8 (OCP e4m3) variant against things other than itself.

The FP8 layer follows the int8 one with e4m3 codes: scale = absmax / 448,
code = e4m3_rne(clamp(x / scale, -448, 448)), the exact sum of decoded
products, the same epilogue.  Independent references used here: torch's CPU
float8_e4m3fn conversion, a brute-force nearest-code search with Python
fractions, exact fraction sums, hand-worked rows, and numpy fp32 scalars.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

FINITE = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)


def torch_decode(codes: np.ndarray) -> np.ndarray:
    return torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def torch_encode(vals: np.ndarray) -> np.ndarray:
    return torch.from_numpy(vals.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def code_value(c: int) -> Fraction:
    s, e, m = c >> 7, (c >> 3) & 15, c & 7
    v = Fraction(8 + m, 1) * Fraction(2) ** (e - 10) if e else Fraction(m) * Fraction(1, 512)
    return -v if s else v


def nearest_code(v: Fraction) -> int:
    """Brute force: the finite code nearest to v, ties to the even mantissa."""
    best, bd = None, None
    for c in FINITE.tolist():
        if c == 0x80:
            continue  # -0 encodes like +0 except for the sign, handled by the caller
        d = abs(code_value(c) - v)
        if bd is None or d < bd or (d == bd and (c & 1) == 0 and (best & 1) == 1):
            best, bd = c, d
    return best


def test_decode_all_codes_matches_torch():
    c = np.arange(256, dtype=np.uint8)
    a, b = oracle.e4m3_decode(c), torch_decode(c)
    nan = np.isnan(b)
    assert np.array_equal(np.isnan(a), nan) and nan.sum() == 2
    assert np.array_equal(a[~nan], b[~nan])
    assert a[0x7E] == 448.0 and a[0x01] == 2.0 ** -9 and a[0x38] == 1.0


def test_encode_roundtrip_and_ties_match_torch():
    vals = oracle.e4m3_decode(FINITE)
    assert np.array_equal(oracle.e4m3_encode(vals.astype(np.float32)), FINITE)
    # every midpoint between neighbouring magnitudes (exact ties) and values
    # just beside them, both signs
    mags = np.unique(np.abs(vals))
    mids = (mags[:-1] + mags[1:]) / 2
    probe = np.concatenate([mids, np.nextafter(mids.astype(np.float32), np.float32(0)),
                            np.nextafter(mids.astype(np.float32), np.float32(np.inf)), mags])
    probe = np.concatenate([probe, -probe]).astype(np.float32)
    assert np.array_equal(oracle.e4m3_encode(probe), torch_encode(probe))
    rng = np.random.default_rng(0)
    r = (np.exp(rng.uniform(np.log(2.0 ** -12), np.log(460.0), 200000)) *
         rng.choice([-1.0, 1.0], 200000)).astype(np.float32)
    assert np.array_equal(oracle.e4m3_encode(r), torch_encode(r))


def test_encode_brute_force_exact_fractions():
    rng = np.random.default_rng(1)
    vals = np.concatenate([rng.uniform(-448, 448, 300), rng.uniform(-0.05, 0.05, 300)]).astype(np.float32)
    got = oracle.e4m3_encode(vals)
    for v, g in zip(vals.tolist(), got.tolist()):
        c = nearest_code(abs(Fraction(v)))
        if v < 0:
            c |= 0x80
        assert g == c, (v, g, c)


def test_quantize_fp8_worked_rows():
    # hand-worked from the definition: scale = absmax / 448, code = e4m3(x / scale)
    x = np.array([[448.0, 1.0, -224.0, 0.5, 0.0, 1.0625, 1.1875],    # scale 1; 1.0625, 1.1875 are ties
                  [896.0, 3.0, -1.0, 0.0, 0.0, 0.0, 0.0],            # scale 2: 448, 1.5, -0.5
                  [0.0] * 7], np.float32)
    q, s = oracle.quantize_rows_f32_fp8(x)
    assert s.tolist() == [1.0, 2.0, 0.0]
    assert q[0].tolist() == [0x7E, 0x38, 0xF6, 0x30, 0x00, 0x38, 0x3A]
    assert q[1].tolist() == [0x7E, 0x3C, 0xB0, 0, 0, 0, 0]
    assert q[2].tolist() == [0] * 7


def test_quantize_fp8_against_independent_steps_and_clamp():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((64, 96)).astype(np.float32)
    # absmax 2^-140: the fp32 scale rounds to one subnormal quantum, 2^-149,
    # so quotients reach 512 and only the clamp keeps them finite
    x[3] = (np.float32(2.0 ** -140) * rng.uniform(-1, 1, 96)).astype(np.float32)
    x[3, 0] = np.float32(2.0 ** -140)
    q, s = oracle.quantize_rows_f32_fp8(x)
    assert s[3] == np.float32(2.0 ** -149) and q[3, 0] == 0x7E
    amax = np.abs(x).max(axis=1)
    assert np.array_equal(s, (amax / np.float32(448.0)).astype(np.float32))
    t = np.clip(x / s[:, None], np.float32(-448), np.float32(448)).astype(np.float32)
    assert np.array_equal(q, torch_encode(t))
    assert not np.any((q & 0x7F) == 0x7F)
    assert np.all((q & 0x7F).max(axis=1) == 0x7E)
    # bf16 entry point: exact widening, then the same
    xb = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    qb, sb = oracle.quantize_rows_bf16_fp8(xb)
    qf, sf = oracle.quantize_rows_f32_fp8(torch.from_numpy(x).to(torch.bfloat16).float().numpy())
    assert np.array_equal(qb, qf) and np.array_equal(sb, sf)


def test_gemm_fp8_exact_against_fractions():
    rng = np.random.default_rng(3)
    a = rng.choice(FINITE, (5, 37))
    b = rng.choice(FINITE, (4, 37))
    acc = oracle.gemm_fp8(a, b)
    for m in range(5):
        for n in range(4):
            want = sum((code_value(int(a[m, k])) * code_value(int(b[n, k])) for k in range(37)), Fraction(0))
            assert Fraction(acc[m, n]) == want


def test_gemm_fp8_exact_where_fp32_accumulation_is_not():
    # one 448 * 448 product and 4096 products of the smallest subnormals: the
    # exact sum is 200704 + 4096 * 2^-18; summing in fp32 would drop the tail
    K = 4097
    a = np.full((1, K), 0x01, np.uint8)
    b = np.full((1, K), 0x01, np.uint8)
    a[0, 0] = b[0, 0] = 0x7E
    acc = oracle.gemm_fp8(a, b)
    assert acc[0, 0] == 200704.0 + 4096 * 2.0 ** -18
    f32 = np.float32(0)
    for k in range(K):
        f32 = np.float32(f32 + np.float32(oracle.e4m3_decode(a[0, k:k + 1])[0] * oracle.e4m3_decode(b[0, k:k + 1])[0]))
    assert float(f32) != acc[0, 0]
    # closed form: all codes 448 -> 448^2 K
    full = oracle.gemm_fp8(np.full((2, 64), 0x7E, np.uint8), np.full((3, 64), 0xFE, np.uint8))
    assert np.all(full == -448.0 * 448.0 * 64)


def test_epilogue_f64acc_order_numpy_scalars():
    rng = np.random.default_rng(4)
    acc = rng.standard_normal((6, 9)) * 1e4
    sx = rng.uniform(1e-4, 1e-2, 6).astype(np.float32)
    sw = rng.uniform(1e-4, 1e-2, 9).astype(np.float32)
    bias = torch.from_numpy(rng.standard_normal(9).astype(np.float32)).to(torch.bfloat16)
    bb = bias.view(torch.int16).numpy().view(np.uint16)
    y = oracle.epilogue_f64acc(acc, sx, sw, bb)
    bf = bias.float().numpy()
    for m in range(6):
        for n in range(9):
            v = np.float32(np.float32(sx[m] * sw[n]) * np.float32(acc[m, n])) + bf[n]
            want = torch.tensor(np.float32(v)).to(torch.bfloat16).view(torch.int16).item() & 0xFFFF
            assert y[m, n] == want
    y0 = oracle.epilogue_f64acc(acc, sx, sw, None)
    assert y0.shape == (6, 9)
