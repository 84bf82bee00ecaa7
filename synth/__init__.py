"""Seeded synthetic inputs shared by the GPU path's tests/bench and the fp64 oracle.

This module only draws random numbers and changes their storage format; it holds
none of the attention arithmetic.  Both sides of every parity comparison receive
the *same* bits from here.

Recipe (numpy side): ``numpy.random.Generator(PCG64(SeedSequence([seed, layer,
tensor_id])))``, ``standard_normal(dtype=float32)``, then rounding to bfloat16 by
round-to-nearest-even on the integer bits.  tensor_id: Q = 0, K = 1, V = 2,
router weights = 3 (4 for the head).  Large tensors that only the GPU needs are
drawn on the device with torch's Philox generator instead (``torch_normal``);
the host copy the oracle reads is then made from those same device bits.
"""
from __future__ import annotations

import numpy as np

TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_W_ENC, TENSOR_W_HEAD = 0, 1, 2, 3, 4


def rng(seed: int, layer: int = 0, tensor_id: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, layer, tensor_id])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bits to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_f32(shape, seed: int, layer: int = 0, tensor_id: int = 0, std: float = 1.0) -> np.ndarray:
    x = rng(seed, layer, tensor_id).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def normal_bf16_bits(shape, seed: int, layer: int = 0, tensor_id: int = 0) -> np.ndarray:
    """iid N(0,1) drawn in float32 and rounded to bfloat16; returns uint16 bits."""
    return f32_to_bf16_bits(normal_f32(shape, seed, layer, tensor_id))


def qkv_bf16(B, S, Hq, Hkv, d, seed, layer=0):
    """Q [B,S,Hq,d], K/V [B,S,Hkv,d] as bfloat16 bits (uint16)."""
    q = normal_bf16_bits((B, S, Hq, d), seed, layer, TENSOR_Q)
    k = normal_bf16_bits((B, S, Hkv, d), seed, layer, TENSOR_K)
    v = normal_bf16_bits((B, S, Hkv, d), seed, layer, TENSOR_V)
    return q, k, v


def qkv_f32(B, S, Hq, Hkv, d, seed, layer=0):
    """Q/K/V as float32 (no rounding), for the fp32 path."""
    q = normal_f32((B, S, Hq, d), seed, layer, TENSOR_Q)
    k = normal_f32((B, S, Hkv, d), seed, layer, TENSOR_K)
    v = normal_f32((B, S, Hkv, d), seed, layer, TENSOR_V)
    return q, k, v


def router_weights(n_layers, in_features, hidden, seed):
    """Per-layer router weights, N(0, 1/fan_in), float32.

    w_enc [L, hidden, in_features] (row = one hidden unit), b_enc [L, hidden],
    w_head [L, 2, hidden], b_head [L, 2].  Biases are drawn with a small std.
    """
    g = rng(seed, 0, TENSOR_W_ENC)
    w_enc = g.standard_normal((n_layers, hidden, in_features), dtype=np.float32)
    w_enc *= np.float32(1.0 / np.sqrt(in_features))
    b_enc = g.standard_normal((n_layers, hidden), dtype=np.float32) * np.float32(0.1)
    g2 = rng(seed, 0, TENSOR_W_HEAD)
    w_head = g2.standard_normal((n_layers, 2, hidden), dtype=np.float32)
    w_head *= np.float32(1.0 / np.sqrt(hidden))
    b_head = g2.standard_normal((n_layers, 2), dtype=np.float32) * np.float32(0.1)
    return w_enc, b_enc, w_head, b_head


def layer_mode_draw(n_layers: int, n_dense: int, seed: int) -> np.ndarray:
    """Seeded per-layer mode plan: a random permutation, first n_dense layers dense (0), rest sparse (1)."""
    perm = rng(seed, 0, 9).permutation(n_layers)
    modes = np.ones(n_layers, dtype=np.int32)
    modes[perm[:n_dense]] = 0
    return modes


# ---------------------------------------------------------------- torch helpers
def torch_bf16_from_bits(bits: np.ndarray, device="cuda"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(device) if device is not None else t


def torch_normal(shape, seed: int, dtype, device="cuda", chunk_elems: int = 1 << 28):
    """iid N(0,1) drawn on the device with torch's Philox generator, stored as ``dtype``.

    Conversion float32 -> bfloat16 in torch rounds to nearest even.  Drawn in chunks
    so the float32 staging buffer stays small.
    """
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1)
    n = flat.numel()
    for s in range(0, n, chunk_elems):
        e = min(n, s + chunk_elems)
        flat[s:e] = torch.randn(e - s, generator=g, dtype=torch.float32, device=device).to(dtype)
    return out
