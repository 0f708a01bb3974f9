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


def edge_weights(n: int, k: int, group_size: int, seed: int) -> np.ndarray:
    """Weights [n, k] fp32 built from the patterns where a folded affine
    product is weakest (row r takes pattern r % 8):

    0. an all-zero row;
    1. constant-zero groups alternating with N(0, 0.02) groups;
    2. one positive spike per group, every other weight exactly 0;
    3. one negative spike per group, every other weight exactly 0;
    4. one spike of either sign per group, the rest N(0, 1e-6);
    5. a single spike in the whole row, everything else exactly 0;
    6. groups entirely below zero (one-sided, negative);
    7. groups of exact zeros with one negative and one positive weight.

    Spike magnitudes are log-uniform in [1e-3, 4]."""
    g = rng(seed)
    w = np.zeros((n, k), dtype=np.float64)
    G = k // group_size

    def spike():
        return float(np.exp(g.uniform(np.log(1e-3), np.log(4.0))))

    for r in range(n):
        p = r % 8
        if p == 1:
            for j in range(1, G, 2):
                w[r, j * group_size:(j + 1) * group_size] = g.standard_normal(group_size) * 0.02
        elif p in (2, 3, 4):
            for j in range(G):
                if p == 4:
                    w[r, j * group_size:(j + 1) * group_size] = g.standard_normal(group_size) * 1e-6
                sign = 1.0 if p == 2 else -1.0 if p == 3 else float(g.choice([-1.0, 1.0]))
                w[r, j * group_size + int(g.integers(0, group_size))] = sign * spike()
        elif p == 5:
            w[r, int(g.integers(0, k))] = float(g.choice([-1.0, 1.0])) * spike()
        elif p == 6:
            w[r] = -np.abs(g.standard_normal(k) * 0.02) - 1e-3
        elif p == 7:
            for j in range(G):
                i0, i1 = g.choice(group_size, 2, replace=False)
                w[r, j * group_size + i0] = -spike()
                w[r, j * group_size + i1] = spike()
    return w.astype(np.float32)


def wide_activations(shape, seed: int, sign: float = 1.0) -> np.ndarray:
    """Activations of one sign with magnitudes log-uniform over e^-8 .. e^2
    (fp32): same-sign, wide-range inputs."""
    g = rng(seed)
    return (sign * np.exp(g.uniform(-8.0, 2.0, size=shape))).astype(np.float32)
