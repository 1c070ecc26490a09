"""Pins of the oracle's fp64 matmul and SwiGLU glue (CPU only).

The matmul reference is pinned by exact rational arithmetic (fractions.Fraction)
on sampled outputs and by the one-hot identity; the bf16 rounding by values
worked by hand.  Source: Unweight page, section 七 (the reconstructing matmul
feeds rebuilt BF16 weights to the matrix units) and section 十 (bit-exact).
"""
from fractions import Fraction

import numpy as np

import oracle
import synth


def _exact(bits):
    v = int(bits)
    sign = -1 if v >> 15 else 1
    e = (v >> 7) & 0xFF
    m = v & 0x7F
    assert e != 255
    if e == 0:
        return sign * Fraction(m, 128) * Fraction(2) ** -126
    return sign * (1 + Fraction(m, 128)) * Fraction(2) ** (e - 127)


def test_matmul_fp64_exact_rational_samples():
    w = synth.weights(256, 512, 0, 0.001, 12)
    x = synth.activations(3, 512)
    y = oracle.matmul_fp64(x, w)
    rng = np.random.default_rng(0)
    for m, n in zip(rng.integers(0, 3, 6), rng.integers(0, 256, 6)):
        exact = sum(_exact(x[m, k]) * _exact(w[n, k]) for k in range(512))
        assert abs(Fraction(float(y[m, n])) - exact) <= abs(exact) * Fraction(1, 10 ** 12) + Fraction(1, 10 ** 30)


def test_one_hot_identity():
    w = synth.weights(64, 256, 1, 0.002, 12)
    x, ks = synth.one_hot_activations(5, 256)
    y = oracle.matmul_fp64(x, w)
    for m, k in enumerate(ks):
        assert np.array_equal(y[m], oracle.bf16_to_f64(w[:, k]))


def test_rows_subset_matches_full():
    w = synth.weights(64, 256, 2, 0.0, 0)
    x = synth.activations(4, 256)
    rows = np.array([0, 7, 63])
    assert np.array_equal(oracle.matmul_fp64_rows(x, w, rows), oracle.matmul_fp64(x, w)[:, rows])


def test_bf16_rne_hand_values():
    vals = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -7), 3.0, 2 ** -20, 1 + 2 ** -8 + 2 ** -30])
    got = oracle.f64_to_bf16_rne(vals)
    want = [0x3F80, 0x3F80, 0x3F82, 0xBF81, 0x4040, 0x3580, 0x3F81]
    assert [int(v) for v in got] == want


def test_silu_mul_closed_forms():
    g = np.array([0.0, 1.0, -1.0, 20.0])
    u = np.array([5.0, 2.0, 2.0, 1.0])
    h = oracle.bf16_to_f64(oracle.silu_mul_bf16(g, u))
    s1 = 1.0 / (1.0 + np.exp(-1.0))
    exact = np.array([0.0, 2 * s1, -2 * (1 - s1), 20.0 / (1 + np.exp(-20.0))])
    assert np.all(np.abs(h - exact) <= np.abs(exact) * 2 ** -8)
    assert h[0] == 0.0


def test_rel_err_definition():
    ref = np.array([[1.0, -4.0], [2.0, 0.5]])
    y = ref + np.array([[0.0, 0.002], [-0.004, 0.0]])
    assert abs(oracle.rel_err(y, ref) - 0.001) < 1e-15
