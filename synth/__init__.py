"""Seeded synthetic inputs shared by the oracle-side tests and the GPU path.

This module only draws random numbers and rounds them to bf16 bit patterns.
It holds none of the codec's or the matmul's arithmetic, so both sides of a
parity test can take their inputs from here without sharing method code.

Recipe (the pages publish no weights; these stand in for trained Llama MLP
matrices, whose exponent statistics the Unweight page describes in its
section on the pattern inside BF16 weights):

* weights: ``rng = numpy.random.default_rng(seed)``; float32 N(0,1) * 0.02,
  rounded to bf16 with round-to-nearest-even; then ``round(p*N*K)`` distinct
  positions (``rng.choice(..., replace=False)``) are multiplied by
  ``2**shift`` (exact in bf16 for normal values), which plants rare exponents;
* activations: ``default_rng(xseed)``, float32 N(0,1) rounded to bf16;
  batches are nested, the first M rows of a larger draw.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "weights",
    "activations",
    "all_bf16_patterns",
    "one_hot_activations",
    "CONFIGS",
]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 bit patterns (round to nearest, ties to even).

    Inputs are finite (the generators never produce Inf/NaN).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def weights(rows: int, cols: int, seed: int, outlier_frac: float, outlier_shift: int,
            std: float = 0.02) -> np.ndarray:
    """A [rows, cols] bf16 weight matrix as uint16 bit patterns (row-major)."""
    n = rows * cols
    rng = np.random.default_rng(seed)
    w = rng.standard_normal(n, dtype=np.float32) * np.float32(std)
    bits = f32_to_bf16_bits(w)
    n_out = int(round(outlier_frac * n))
    if n_out:
        idx = rng.choice(n, n_out, replace=False)
        scaled = bf16_bits_to_f32(bits[idx]) * np.float32(2.0 ** outlier_shift)
        bits[idx] = f32_to_bf16_bits(scaled)
    return bits.reshape(rows, cols)


def activations(tokens: int, cols: int, xseed: int = 1, max_tokens: int | None = None) -> np.ndarray:
    """[tokens, cols] bf16 activations N(0,1), nested: the first ``tokens`` rows of a
    ``max_tokens``-row draw (default: exactly ``tokens`` rows)."""
    total = max(tokens, max_tokens or tokens)
    rng = np.random.default_rng(xseed)
    x = rng.standard_normal(total * cols, dtype=np.float32)
    return f32_to_bf16_bits(x).reshape(total, cols)[:tokens].copy()


def one_hot_activations(tokens: int, cols: int, seed: int = 7) -> tuple[np.ndarray, np.ndarray]:
    """X[m, k_m] = 1.0 (bf16 0x3F80), zeros elsewhere; returns (X bits, k_m)."""
    rng = np.random.default_rng(seed)
    ks = rng.integers(0, cols, size=tokens)
    x = np.zeros((tokens, cols), dtype=np.uint16)
    x[np.arange(tokens), ks] = 0x3F80
    return x, ks


def all_bf16_patterns(seed: int = 0) -> np.ndarray:
    """A 256x256 matrix holding each of the 65,536 bf16 bit patterns exactly once
    (random permutation) -- the exhaustive split/reassembly case."""
    rng = np.random.default_rng(seed)
    return rng.permutation(65536).astype(np.uint16).reshape(256, 256)


# The five workloads: name -> dict of shapes and draws.
CONFIGS = {
    "tiny": dict(rows=256, cols=512, seed=0, p=0.001, shift=12, tokens=(1,), xseed=1),
    "gate_8b": dict(rows=14336, cols=4096, seed=0, p=0.0005, shift=10, tokens=(1,), xseed=1),
    "mlp_8b": dict(gate=(14336, 4096, 10), up=(14336, 4096, 11), down=(4096, 14336, 12),
                   p=0.0005, shift=10, tokens=(1, 16, 64), xseed=1),
    "mlp_8b_large": dict(gate=(14336, 4096, 10), up=(14336, 4096, 11), down=(4096, 14336, 12),
                         p=0.0005, shift=10, tokens=(256, 1024), xseed=1),
    "stack_70b": dict(layers=80, gate=(28672, 8192), up=(28672, 8192), down=(8192, 28672),
                      seed_base=1000, p=0.0005, shift=10, tokens=(1, 256), xseed=1),
}
