"""Helpers for the GPU parity tests: moving seeded inputs to the device,
reading results back as raw bits, and the comparison measures the parity bar
uses (bit equality, bf16 ulp distance, cosine, NaN/Inf scan)."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synthetic

DEV = "cuda:0"


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(DEV)


def bits(t: torch.Tensor) -> np.ndarray:
    assert t.dtype == torch.bfloat16
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def ulp_key(b: np.ndarray) -> np.ndarray:
    """Monotone integer line for bf16 patterns (+0 and -0 coincide)."""
    b = b.astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def ulp_dist(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    return np.abs(ulp_key(a) - ulp_key(b))


def cosine(a_bits: np.ndarray, b_bits: np.ndarray) -> float:
    a = oracle.bf16_to_f32(a_bits).astype(np.float64).ravel()
    b = oracle.bf16_to_f32(b_bits).astype(np.float64).ravel()
    na, nb = np.linalg.norm(a), np.linalg.norm(b)
    if na == 0 and nb == 0:
        return 1.0
    return float(a @ b / (na * nb))


def assert_bf16_parity(got: np.ndarray, want: np.ndarray, what: str = ""):
    """The bf16 bar: every element within 1 ulp, cosine >= 0.99999, no NaN/Inf."""
    assert got.shape == want.shape, (got.shape, want.shape)
    finite = (got & 0x7F80) != 0x7F80
    assert finite.all(), f"{what}: {np.count_nonzero(~finite)} NaN/Inf outputs"
    d = ulp_dist(got, want)
    assert d.max(initial=0) <= 1, f"{what}: max ulp distance {d.max()} at {np.unravel_index(d.argmax(), d.shape)}"
    if got.size:
        assert cosine(got, want) >= 0.99999, what
    return int(np.count_nonzero(d))


def shape_inputs(shape: synthetic.GemmShape, seed: int = 0):
    """Seeded host inputs for one linear: x bits, fp32 weights, bias bits."""
    st = synthetic.streams(seed, shape.config_id, shape.layer_id)
    x = synthetic.bf16_bits(synthetic.activations_bf16(st, shape.M, shape.K, shape.outlier_frac))
    w = synthetic.weights_f32(st, shape.N, shape.K)
    b = synthetic.bf16_bits(synthetic.bias_bf16(st, shape.N))
    return x, w, b


def sample_rows(M: int, n: int, seed: int = 0) -> np.ndarray:
    """First, last and a seeded spread of rows (sorted, unique)."""
    rng = np.random.default_rng(seed)
    rows = {0, M - 1, M // 2}
    rows.update(rng.integers(0, M, size=max(0, n - 3)).tolist())
    return np.array(sorted(rows), dtype=np.int64)
