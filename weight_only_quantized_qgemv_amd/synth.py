"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

Only random numbers and shapes live here: no quantization, packing or product
arithmetic. Every array comes from numpy's PCG64 generator with an explicit
seed: ``standard_normal`` in fp64, times sigma, rounded to fp32. Rounding of
activations to bf16/fp16 is done by the caller (torch's round-to-nearest-even
conversion).
"""
from __future__ import annotations

import numpy as np


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def normal_f32(shape, sigma: float, seed: int) -> np.ndarray:
    """N(0, sigma^2) samples as fp32, shape `shape`."""
    return (rng(seed).standard_normal(shape) * sigma).astype(np.float32)


def iota_f32(shape) -> np.ndarray:
    """0, 1, 2, ... in row-major order, as fp32."""
    return np.arange(int(np.prod(shape)), dtype=np.float32).reshape(shape)


def moe_ids(n_tokens: int, top_k: int, num_experts: int, seed: int) -> np.ndarray:
    """Expert ids [n_tokens, top_k] (int32): per token, the first top_k entries
    of a seeded permutation of 0..num_experts-1 (uniform, without replacement)."""
    g = rng(seed)
    ids = np.empty((n_tokens, top_k), dtype=np.int32)
    for t in range(n_tokens):
        ids[t] = g.permutation(num_experts)[:top_k]
    return ids


def random_codes(shape, bits: int, seed: int) -> np.ndarray:
    """Uniform integer codes in [0, 2^bits) as uint8."""
    return rng(seed).integers(0, 1 << bits, size=shape, dtype=np.uint8)


def random_ints(shape, lo: int, hi: int, seed: int) -> np.ndarray:
    """Uniform integers in [lo, hi] as int64."""
    return rng(seed).integers(lo, hi + 1, size=shape, dtype=np.int64)
