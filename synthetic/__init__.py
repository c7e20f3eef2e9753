"""Seeded synthetic inputs for the W8A8 linear workloads.

This module is shared by the CPU oracle side (tests, the CPU baseline) and the
GPU side (tests, bench, smoke).  It draws random numbers and rounds them to the
storage dtype (bf16 through torch's own CPU conversion); it holds none of the
method's arithmetic: no quantization, no GEMM, no epilogue, no GELU.

Workload shapes are those of a DiT (diffusion transformer) with hidden size
3072 at 768px (48x48 = 2304 patch tokens) and 1024px (64x64 = 4096 tokens),
the model family the pages deploy the fused INT8 GEMM into ("Realizing Native
INT8 Compute for Diffusion Transformers on Consumer GPUs", arXiv 2606.14598,
Abstract).  The pages publish no shapes, prompts or tensors; these inputs are
stand-ins with the value distributions stated below.

Recipe (every tensor row-major, K contiguous):
  * activations X [M, K]: standard normal fp32; optionally a fixed set of
    round(frac * K) columns (a seeded permutation, same columns for every
    token) is multiplied by `outlier_scale` in fp32; then rounded to bf16 (RNE).
  * weights W [N, K]: 0.02 * standard normal, fp32 (quantized per output
    channel by whichever side consumes them).
  * bias [N]: 0.1 * standard normal rounded to bf16.
  * streams: numpy PCG64 seeded by SeedSequence([seed, config_id, layer_id]),
    spawned into four independent streams (x, w, bias, outlier permutation).
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

__all__ = [
    "Streams", "streams", "activations_bf16", "weights_f32", "bias_bf16",
    "bf16_from_f32", "bf16_bits", "GemmShape", "CONFIGS", "BENCH_WORKLOAD",
]


@dataclasses.dataclass
class Streams:
    x: np.random.Generator
    w: np.random.Generator
    bias: np.random.Generator
    perm: np.random.Generator


def streams(seed: int, config_id: int, layer_id: int) -> Streams:
    """Four independent PCG64 streams for one linear layer of one workload."""
    ss = np.random.SeedSequence([int(seed), int(config_id), int(layer_id)])
    kids = ss.spawn(4)
    gens = [np.random.Generator(np.random.PCG64(k)) for k in kids]
    return Streams(*gens)


def bf16_from_f32(a: np.ndarray) -> torch.Tensor:
    """Round an fp32 array to a bf16 CPU tensor with torch's RNE conversion."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """The raw 16-bit patterns of a bf16 CPU tensor, as a uint16 numpy array."""
    assert t.dtype == torch.bfloat16
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def activations_bf16(st: Streams, M: int, K: int, outlier_frac: float = 0.0,
                     outlier_scale: float = 20.0, std: float = 1.0) -> torch.Tensor:
    """X [M, K] bf16: N(0, std^2), with round(outlier_frac*K) outlier columns."""
    x = st.x.standard_normal((M, K), dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    n_out = int(round(outlier_frac * K))
    if n_out > 0:
        cols = st.perm.permutation(K)[:n_out]
        x[:, cols] *= np.float32(outlier_scale)
    return bf16_from_f32(x)


def weights_f32(st: Streams, N: int, K: int, std: float = 0.02) -> np.ndarray:
    """W [N, K] fp32 ~ N(0, std^2)."""
    w = st.w.standard_normal((N, K), dtype=np.float32)
    w *= np.float32(std)
    return w


def bias_bf16(st: Streams, N: int, std: float = 0.1) -> torch.Tensor:
    b = st.bias.standard_normal((N,), dtype=np.float32) * np.float32(std)
    return bf16_from_f32(b)


@dataclasses.dataclass(frozen=True)
class GemmShape:
    """One linear layer: y[M, N] = x[M, K] . W[N, K]^T (+ bias)."""
    name: str
    M: int
    N: int
    K: int
    outlier_frac: float = 0.0
    config_id: int = 0
    layer_id: int = 0


# The five workloads.  config_id numbers them 1..5; layer_id separates the
# linears inside one workload so that each has its own streams.
CONFIGS = {
    "unit": [GemmShape("unit_m64_k256_n128", 64, 128, 256, 0.0, 1, 0)],
    "dit768_attn": [
        GemmShape("attn_proj_m2304_k3072_n3072", 2304, 3072, 3072, 0.01, 2, 0),
        GemmShape("attn_qkv_m2304_k3072_n9216", 2304, 9216, 3072, 0.01, 2, 1),
    ],
    "dit1024_mlp": [
        GemmShape("mlp_up_m4096_k3072_n12288", 4096, 12288, 3072, 0.01, 3, 0),
        # down-proj input: GELU of a random bf16 tensor with outlier columns
        GemmShape("mlp_down_m4096_k12288_n3072", 4096, 3072, 12288, 0.01, 3, 1),
    ],
    "skinny": [
        GemmShape(f"skinny_m{m}_k3072_n{n}", m, n, 3072, 0.0, 4, 10 * i + j)
        for i, m in enumerate((1, 16, 256)) for j, n in enumerate((18432, 3072))
    ],
    "dit1024_chain": [
        GemmShape("chain_qkv_m4608_k3072_n9216", 4608, 9216, 3072, 0.01, 5, 0),
        GemmShape("chain_out_m4608_k3072_n3072", 4608, 3072, 3072, 0.0, 5, 1),
        GemmShape("chain_up_m4608_k3072_n12288", 4608, 12288, 3072, 0.0, 5, 2),
        GemmShape("chain_down_m4608_k12288_n3072", 4608, 3072, 12288, 0.0, 5, 3),
    ],
}

# The timed workload: the 1024px DiT MLP pair (up-proj, GELU + re-quantize of a
# random bf16 tensor, down-proj).  Its up-proj is the headline GEMM shape.
BENCH_WORKLOAD = "dit1024_mlp"
