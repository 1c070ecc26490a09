"""Pins of the oracle's length-limited canonical Huffman code (CPU only).

Checked against: Kraft equality, the dyadic closed form, brute-force optimum on
tiny alphabets, an independent dynamic program for the length-limited optimum,
an unlimited heap Huffman as a lower bound, the Shannon bound, brute-force
prefix-freeness, and a hand-worked bitstream (tests/golden/huffman_one_brick.json).
Source: Unweight page, section 四 (Huffman coding of the exponent bytes only).
"""
import heapq
import itertools
import json
import os
from fractions import Fraction
from functools import lru_cache

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _cost(cnt, lengths):
    return int(sum(int(cnt[s]) * int(lengths[s]) for s in range(len(cnt))))


def _brute_force_optimum(counts, lmax):
    """min sum(c*l) over all length vectors with Kraft <= 1 and 1 <= l <= lmax."""
    best = None
    cap = min(lmax, len(counts) - 1)
    for ls in itertools.product(range(1, cap + 1), repeat=len(counts)):
        if sum(Fraction(1, 2 ** l) for l in ls) <= 1:
            c = sum(a * b for a, b in zip(counts, ls))
            best = c if best is None or c < best else best
    return best


def _dp_length_limited_optimum(counts, lmax):
    """Independent optimum: symbols sorted by count descending get non-decreasing
    depths; walk the code tree depth by depth, choosing how many of the
    available nodes become leaves."""
    c = sorted(counts, reverse=True)
    n = len(c)
    prefix = [0]
    for v in c:
        prefix.append(prefix[-1] + v)

    @lru_cache(maxsize=None)
    def best(depth, i, avail):
        if i == n:
            return 0
        if depth > lmax or avail == 0:
            return None
        out = None
        for j in range(0, min(avail, n - i) + 1):
            rest_nodes = min(2 * (avail - j), n - i - j)
            sub = best(depth + 1, i + j, rest_nodes)
            if sub is None:
                continue
            val = depth * (prefix[i + j] - prefix[i]) + sub
            out = val if out is None or val < out else out
        return out
    return best(1, 0, 2)


def _heap_huffman_cost(counts):
    h = list(counts)
    heapq.heapify(h)
    cost = 0
    while len(h) > 1:
        a, b = heapq.heappop(h), heapq.heappop(h)
        cost += a + b
        heapq.heappush(h, a + b)
    return cost


def _lengths_for(counts, lmax):
    cnt = np.zeros(256, np.int64)
    cnt[:len(counts)] = counts
    return cnt, oracle.huffman_lengths(cnt, lmax)


def test_dyadic_closed_form():
    counts = [1, 1, 2, 4, 8, 16, 32]           # p = 2^-l exactly
    cnt, L = _lengths_for(counts, 12)
    assert list(L[:7]) == [6, 6, 5, 4, 3, 2, 1]
    assert oracle.kraft_sum(L) == 1.0


@pytest.mark.parametrize("seed", range(12))
def test_brute_force_optimum_small_alphabets(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(2, 8))
    counts = [int(v) for v in rng.integers(1, 60, size=n)]
    for lmax in sorted({int(np.ceil(np.log2(n))), min(3, n - 1) if n > 2 else 1, 12}):
        if 2 ** lmax < n:
            continue
        cnt, L = _lengths_for(counts, lmax)
        assert L.max() <= lmax
        assert oracle.kraft_sum(L) == 1.0
        assert _cost(cnt, L) == _brute_force_optimum(counts, lmax)


def test_length_limit_binds_and_matches_dp():
    """The tiny config has codes of 17 bits when unlimited; at 12 bits the
    package-merge total must equal the independent DP optimum."""
    w = synth.weights(256, 512, 0, 0.001, 12)
    cnt = oracle.histogram(oracle.split(w)[0])
    present = [int(cnt[s]) for s in range(256) if cnt[s] > 0]
    L = oracle.huffman_lengths(cnt, 12)
    assert L.max() == 12
    assert oracle.kraft_sum(L) == 1.0
    assert _cost(cnt, L) == _dp_length_limited_optimum(present, 12)
    assert _cost(cnt, L) >= _heap_huffman_cost(present)
    L20 = oracle.huffman_lengths(cnt, 20)
    assert _cost(cnt, L20) == _heap_huffman_cost(present)
    assert _dp_length_limited_optimum(present, 20) == _heap_huffman_cost(present)


def test_shannon_bound():
    w = synth.weights(512, 1024, 4, 0.0005, 10)
    cnt = oracle.histogram(oracle.split(w)[0])
    L = oracle.huffman_lengths(cnt, 12)
    H = oracle.entropy_bits(cnt)
    mean = _cost(cnt, L) / cnt.sum()
    assert H <= mean < H + 1


def test_single_symbol_gets_phantom():
    cnt = np.zeros(256, np.int64)
    cnt[0] = 100
    L = oracle.huffman_lengths(cnt)
    assert L[0] == 1 and L[1] == 1 and L.sum() == 2
    w = np.zeros((16, 64), np.uint16)                    # all +0.0: exponent 0 only
    enc = oracle.huffman_encode(w)
    assert enc["total_bits"] == 1024
    assert np.array_equal(oracle.huffman_decode(enc), w)


def test_canonical_hand_example_and_prefix_free():
    L = np.zeros(256, np.int64)
    L[[65, 66, 67, 68]] = [1, 2, 3, 3]
    codes = oracle.canonical_codes(L)
    assert [int(codes[s]) for s in (65, 66, 67, 68)] == [0b0, 0b10, 0b110, 0b111]
    w = synth.weights(256, 512, 0, 0.001, 12)
    cnt = oracle.histogram(oracle.split(w)[0])
    L = oracle.huffman_lengths(cnt)
    codes = oracle.canonical_codes(L)
    words = [format(int(codes[s]), "0%db" % int(L[s])) for s in range(256) if L[s]]
    for a in words:
        for b in words:
            assert a == b or not b.startswith(a)


def test_golden_one_brick_stream():
    g = json.load(open(os.path.join(GOLDEN, "huffman_one_brick.json")))
    w = np.full((16, 64), 120 << 7, dtype=np.uint16)
    w[0, 1] = 121 << 7
    w[0, 2] = 122 << 7
    r, c = np.meshgrid(np.arange(16), np.arange(64), indexing="ij")
    sm = ((r * 64 + c) % 256).astype(np.uint16)
    w = (w | ((sm >> 7) << 15) | (sm & 0x7F)).astype(np.uint16)
    enc = oracle.huffman_encode(w)
    for s, l in g["lengths"].items():
        assert enc["lengths"][int(s)] == l
    for s, cd in g["codes"].items():
        assert enc["codes"][int(s)] == cd
    assert enc["total_bits"] == g["total_bits"]
    assert len(enc["words"]) == g["n_words"]
    assert int(enc["words"][0]) == int(g["word0"], 16)
    assert not enc["words"][1:].any()
    assert list(enc["offsets"]) == g["offsets"]
    assert np.array_equal(oracle.huffman_decode(enc), w)


def test_roundtrip_tiny_and_all_patterns():
    w = synth.weights(256, 512, 0, 0.001, 12)
    enc = oracle.huffman_encode(w)
    assert np.array_equal(oracle.huffman_decode(enc), w)
    w = synth.all_bf16_patterns()
    enc = oracle.huffman_encode(w)
    assert np.array_equal(oracle.huffman_decode(enc), w)
    # 256 equiprobable exponents under a 12-bit limit: every code is 8 bits
    assert set(int(v) for v in enc["lengths"]) == {8}


def test_chunk_offsets_are_independent_entry_points():
    w = synth.weights(64, 512, 9, 0.002, 12)
    enc = oracle.huffman_encode(w)
    e_serial = oracle.to_serial(oracle.split(w)[0])
    rng = np.random.default_rng(0)
    ids = rng.choice(len(enc["offsets"]), 16, replace=False)
    got = oracle.huffman_decode_chunks(enc, ids)
    for c in ids:
        assert np.array_equal(got[int(c)], e_serial[256 * c:256 * c + 256])


def test_bits_per_weight_on_gate_shaped_draw():
    """Section 四's compressed sizes on a gate-shaped synthetic slice: Huffman
    around 10.6-10.8 bits/weight (about a third smaller than 16)."""
    w = synth.weights(1024, 4096, 0, 0.0005, 10)
    enc = oracle.huffman_encode(w)
    assert 10.5 < oracle.huffman_bits_per_weight(enc) < 10.9
