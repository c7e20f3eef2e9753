"""The drop-in module: W8A8Linear swapped into a small seeded DiT-like block.

Every swapped layer is checked on the input it really received during the
block's forward (captured with a forward hook): its quantized weights and
scales bit-exact against the oracle's per-channel quantization of the
layer's own weights, and its bf16 output bit-exact against the oracle's
linear on that input.  The exported state_dict restores an identical block.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synthetic
import w8a8_int8_quantized_quantize_amd as w8
from gpu_helpers import DEV, bits, cosine, dev_bf16, host

pytestmark = pytest.mark.gpu


class TinyDiTBlock(torch.nn.Module):
    """Linears of one DiT block at a small width: fused QKV, output
    projection of a stand-in attention result, MLP up, GELU, MLP down."""

    def __init__(self, d: int = 256, mlp: int = 1024):
        super().__init__()
        self.qkv = torch.nn.Linear(d, 3 * d)
        self.proj = torch.nn.Linear(d, d)
        self.up = torch.nn.Linear(d, mlp)
        self.act = torch.nn.GELU()
        self.down = torch.nn.Linear(mlp, d)

    def forward(self, x, attn):
        qkv = self.qkv(x)
        h = x + self.proj(attn)
        return qkv, self.down(self.act(self.up(h)))


def make_block(seed: int) -> TinyDiTBlock:
    torch.manual_seed(seed)
    return TinyDiTBlock().to(torch.bfloat16).to(DEV)


def inputs(seed: int, shape=(2, 48, 256)):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape).astype(np.float32)
    a = rng.standard_normal(shape).astype(np.float32)
    return (synthetic.bf16_from_f32(x).to(DEV), synthetic.bf16_from_f32(a).to(DEV))


def test_swapped_block_layers_match_oracle():
    ref = make_block(0)
    blk = make_block(0)
    n = w8.quantize_linears(blk)
    assert n == 4
    assert all(isinstance(getattr(blk, k), w8.W8A8Linear) for k in ("qkv", "proj", "up", "down"))
    seen = {}

    def hook(name):
        def f(mod, args, out):
            seen[name] = (args[0].detach().clone(), out.detach().clone())
        return f

    for k in ("qkv", "proj", "up", "down"):
        getattr(blk, k).register_forward_hook(hook(k))
    x, a = inputs(1)
    with torch.no_grad():
        q8, y8 = blk(x, a)
        qb, yb = ref(x, a)
    for k in ("qkv", "proj", "up", "down"):
        lin, mod = getattr(ref, k), getattr(blk, k)
        wq, sw = oracle.quantize_rows_f32(host(lin.weight.float()))
        assert np.array_equal(host(mod.w_q), wq) and np.array_equal(host(mod.s_w), sw), k
        xin, yout = seen[k]
        assert yout.shape == (*xin.shape[:-1], lin.out_features)
        want = oracle.linear(bits(xin.reshape(-1, xin.shape[-1])), wq, sw, bits(lin.bias))
        assert np.array_equal(bits(yout.reshape(-1, yout.shape[-1])), want["y"]), k
    # against the unquantized bf16 block: the quantization error only
    assert cosine(bits(q8.reshape(-1, q8.shape[-1])), bits(qb.reshape(-1, qb.shape[-1]))) > 0.999
    assert cosine(bits(y8.reshape(-1, y8.shape[-1])), bits(yb.reshape(-1, yb.shape[-1]))) > 0.99


def test_state_dict_round_trip():
    blk = make_block(3)
    w8.quantize_linears(blk)
    sd = {k: v.clone() for k, v in blk.state_dict().items()}
    assert sd["up.w_q"].dtype == torch.int8 and sd["up.s_w"].dtype == torch.float32
    other = make_block(4)  # different float weights
    w8.quantize_linears(other)
    other.load_state_dict(sd)
    x, a = inputs(5)
    with torch.no_grad():
        q1, y1 = blk(x, a)
        q2, y2 = other(x, a)
    assert torch.equal(q1, q2) and torch.equal(y1, y2)


def test_include_filter_and_bias_free_layer():
    blk = make_block(6)
    blk.proj = torch.nn.Linear(256, 256, bias=False).to(torch.bfloat16).to(DEV)
    n = w8.quantize_linears(blk, include=lambda name, lin: name != "qkv")
    assert n == 3 and isinstance(blk.qkv, torch.nn.Linear) and blk.proj.bias is None
    x = inputs(7, (33, 256))[0]
    with torch.no_grad():
        y = blk.proj(x)
    want = oracle.linear(bits(x), host(blk.proj.w_q), host(blk.proj.s_w), None)
    assert np.array_equal(bits(y), want["y"])


def test_fp8_swapped_block_layers_within_bound():
    from test_gpu_fp8 import assert_fp8_gemm_bound
    ref = make_block(8)
    blk = make_block(8)
    assert w8.quantize_linears(blk, fp8=True) == 4
    assert blk.up.fp8 and blk.up.w_q.dtype == torch.uint8
    seen = {}
    for k in ("qkv", "proj", "up", "down"):
        getattr(blk, k).register_forward_hook(
            lambda mod, args, out, k=k: seen.__setitem__(k, (args[0].detach().clone(), out.detach().clone())))
    x, a = inputs(9)
    with torch.no_grad():
        blk(x, a)
    for k in ("qkv", "proj", "up", "down"):
        lin, mod = getattr(ref, k), getattr(blk, k)
        wq, sw = oracle.quantize_rows_f32_fp8(host(lin.weight.float()))
        assert np.array_equal(host(mod.w_q), wq) and np.array_equal(host(mod.s_w), sw), k
        xin, yout = seen[k]
        xb = bits(xin.reshape(-1, xin.shape[-1]))
        qx, sx = oracle.quantize_rows_bf16_fp8(xb)
        assert_fp8_gemm_bound(bits(yout.reshape(-1, yout.shape[-1])), qx, sx, wq, sw, bits(lin.bias), k)
