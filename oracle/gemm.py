"""Oracle: the matmul the decoded weights feed, in fp64 over the original BF16.

TEST INFRASTRUCTURE: imported only by tests/, __graft_entry__.smoke() and
bench.py's cpu_baseline leg.  Shares no code with the HIP library.

The Unweight page's reconstructing matmul (section 七) multiplies activations
by the rebuilt BF16 weights of an MLP projection; the output is the ordinary
``Y = X @ W.T`` of a linear layer with W stored [out, in].  Because the codec
is lossless (section 十), the reference uses the original BF16 W and never
touches the codec.  Each product of two bf16 values is exact in fp64 (8-bit
significands) and the fp64 sum of at most 28,672 such terms is far inside the
1e-3 tolerance of the parity tests.

SwiGLU glue (the page names SwiGLU models in section 十一 and the
gate -> up -> down order in section 八): h = silu(gate) * up, rounded to bf16
(round to nearest even) as the input of the down projection.
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns as float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_rne(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 bit patterns, nearest-even (normal range)."""
    x = np.asarray(x, dtype=np.float64)
    m, ex = np.frexp(x)                      # x = m * 2**ex, 0.5 <= |m| < 1
    q = np.rint(m * 256.0) / 256.0           # 8 significant bits, ties to even
    y = np.ldexp(q, ex).astype(np.float32)   # exact: 8 bits fit in float32
    return (y.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def matmul_fp64(x_bits: np.ndarray, w_bits: np.ndarray) -> np.ndarray:
    """Y[m, n] = sum_k X[m, k] * W[n, k] in float64."""
    return bf16_to_f64(x_bits) @ bf16_to_f64(w_bits).T


def matmul_fp64_rows(x_bits: np.ndarray, w_bits: np.ndarray, rows: np.ndarray) -> np.ndarray:
    """Y[:, rows] only (for sampled checks at full size)."""
    return bf16_to_f64(x_bits) @ bf16_to_f64(np.asarray(w_bits)[rows]).T


def silu_mul_bf16(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """bf16(silu(g) * u) with silu(g) = g / (1 + exp(-g)), computed in float64."""
    g = np.asarray(g, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    return f64_to_bf16_rne(g / (1.0 + np.exp(-g)) * u)


def mlp_layer_fp64(x_bits, gate_bits, up_bits, down_bits):
    """One SwiGLU MLP layer: returns (gate out, up out, h bf16 bits, down out)."""
    g = matmul_fp64(x_bits, gate_bits)
    u = matmul_fp64(x_bits, up_bits)
    h = silu_mul_bf16(g, u)
    return g, u, h, matmul_fp64(h, down_bits)


def rel_err(y: np.ndarray, ref: np.ndarray) -> float:
    """max|y - ref| / max|ref| -- the matmul parity measure."""
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    num = float(np.max(np.abs(np.asarray(y, dtype=np.float64) - ref))) if ref.size else 0.0
    return num / den if den > 0 else num
