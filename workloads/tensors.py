"""Seeded synthetic activations (Q, K, V, dO) for the packed layouts.

Inputs only: iid standard-normal fp32 draws rounded to bfloat16
(round-to-nearest-even), token-major `[tokens, heads, d]`, in the ORIGINAL
packed order.  A caller that needs a permuted order gathers rows itself.

Two generators, both pure draws with no method arithmetic:
  * `toy_qkv` reproduces the NumPy ring tutorial's draws exactly
    (default_rng(0), three standard-normal (16, 8) float32 arrays, Q then K then V).
  * `qkv` draws with a seeded torch generator on the requested device, so the
    large tensors are made directly in GPU memory; the same call on the CPU
    device is used by CPU-only checks.  A per-tensor seed keeps Q, K, V and dO
    independent of one another.
"""
from __future__ import annotations

import numpy as np

TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "do": 3}


def toy_qkv():
    rng = np.random.default_rng(0)
    n, d = 16, 8
    q, k, v = (rng.normal(size=(n, d)).astype(np.float32) for _ in range(3))
    return q, k, v


def _seed(seed: int, tensor: str) -> int:
    return (int(seed) * 1_000_003 + 7919 * TENSOR_IDS[tensor] + 17) & 0x7FFFFFFFFFFF


def randn_bf16(shape, seed: int, tensor: str, device="cpu"):
    """Standard-normal fp32 draws rounded (RNE) to a bfloat16 torch tensor."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(_seed(seed, tensor))
    x = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    return x.to(torch.bfloat16)


def qkv(n: int, hq: int, hkv: int, d: int, seed: int, device="cpu", with_do: bool = False):
    q = randn_bf16((n, hq, d), seed, "q", device)
    k = randn_bf16((n, hkv, d), seed, "k", device)
    v = randn_bf16((n, hkv, d), seed, "v", device)
    if with_do:
        do = randn_bf16((n, hq, d), seed, "do", device)
        return q, k, v, do
    return q, k, v
