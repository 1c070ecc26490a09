"""Pins of the oracle's split, serial order and palette format (CPU only).

Each test checks the oracle against something other than itself: bit fields
recomputed from float values, loops instead of reshapes, brute-force counts and
hand-worked fixtures (tests/golden/, each citing the Unweight page section it
follows).
"""
import json
import os
from collections import Counter

import numpy as np
import pytest

import oracle
import synth
from oracle import codec

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_split_fields_from_float_values():
    """Section 三: 1 sign, 8 exponent, 7 mantissa bits -- recomputed from each
    pattern's float value with frexp, for every normal bf16 pattern."""
    w = np.arange(65536, dtype=np.uint16)
    e, sm = oracle.split(w)
    vals = synth.bf16_bits_to_f32(w).astype(np.float64)
    normal = np.isfinite(vals) & (np.abs(vals) >= 2.0 ** -126)
    m, ex = np.frexp(np.abs(vals[normal]))          # |x| = m 2^ex, m in [0.5, 1)
    assert np.array_equal(e[normal], (ex + 126).astype(np.uint8))
    mant = np.rint((m * 2 - 1) * 128).astype(np.uint8)
    assert np.array_equal(sm[normal] & 0x7F, mant)
    assert np.array_equal(sm[normal] >> 7, np.signbit(vals[normal]).astype(np.uint8))
    # zeros/subnormals have exponent byte 0, Inf/NaN have 255
    assert np.all(e[~np.isfinite(vals)] == 255)
    assert np.all(e[np.isfinite(vals) & ~normal] == 0)


def test_split_join_exhaustive():
    w = synth.all_bf16_patterns()
    e, sm = oracle.split(w)
    assert np.array_equal(oracle.join(e, sm), w)


def test_serial_index_by_loops():
    rows, cols = 32, 192
    idx = oracle.serial_index(rows, cols)
    assert np.array_equal(np.sort(idx), np.arange(rows * cols))
    n_bcol = cols // 64
    for s in range(rows * cols):
        brick, within = divmod(s, 1024)
        tb, kb = divmod(brick, n_bcol)
        run, j = divmod(within, 16)
        r = tb * 16 + run % 16
        c = kb * 64 + 16 * (run // 16) + j
        assert idx[s] == r * cols + c


def test_serial_roundtrip():
    a = np.arange(48 * 128, dtype=np.int64).reshape(48, 128)
    assert np.array_equal(oracle.from_serial(oracle.to_serial(a), 48, 128), a)


def test_shape_rules():
    with pytest.raises(ValueError):
        oracle.palette_encode(np.zeros((16, 96), np.uint16))
    with pytest.raises(ValueError):
        oracle.huffman_encode(np.zeros((8, 64), np.uint16))


def test_histogram_brute_force():
    w = synth.weights(64, 128, 3, 0.01, 12)
    e, _ = oracle.split(w)
    c = Counter(int(v) for v in e.ravel())
    cnt = oracle.histogram(e)
    assert all(cnt[s] == c.get(s, 0) for s in range(256))


def test_palette_ranking_ties_and_padding():
    cnt = np.zeros(256, np.int64)
    cnt[[10, 20, 30]] = [5, 7, 5]
    pal = oracle.choose_palette(cnt)
    assert list(pal) == [20, 10, 30] + [20] * 13       # fewer than 16: pad with entry 0
    cnt = np.zeros(256, np.int64)
    cnt[0:20] = 3
    cnt[19] = 9
    pal = oracle.choose_palette(cnt)
    assert list(pal) == [19] + list(range(0, 15))     # ties by exponent ascending


def test_raw_flags_brute_force():
    w = synth.weights(32, 256, 5, 0.003, 12)
    e, _ = oracle.split(w)
    pal = oracle.choose_palette(oracle.histogram(e))
    flags = oracle.raw_group_flags(e, pal)
    ps = set(int(p) for p in pal)
    for r in range(32):
        for g in range(4):
            assert flags[r, g] == any(int(v) not in ps for v in e[r, 64 * g:64 * g + 64])


def test_few_exponents_no_raw_groups():
    rng = np.random.default_rng(2)
    e = rng.integers(110, 126, size=(32, 128)).astype(np.uint16)   # 16 distinct values
    w = (e << 7) | rng.integers(0, 128, size=e.shape).astype(np.uint16)
    enc = oracle.palette_encode(w.astype(np.uint16))
    assert enc["n_raw"] == 0 and not enc["flags"].any()
    assert np.array_equal(oracle.palette_decode(enc), w)


def _brick_from_rule(exp_of, rows=16, cols=64):
    r, c = np.meshgrid(np.arange(rows), np.arange(cols), indexing="ij")
    e = exp_of(r, c).astype(np.uint16)
    sm = ((r * 64 + c) % 256).astype(np.uint16)
    return (((sm >> 7) & 1) << 15 | (e << 7) | (sm & 0x7F)).astype(np.uint16)


def test_palette_golden_one_brick():
    g = json.load(open(os.path.join(GOLDEN, "palette_one_brick.json")))

    def rule(r, c):
        e = 100 + (c % 16)
        e[5, 0] = 200
        return e
    w = _brick_from_rule(rule)
    enc = oracle.palette_encode(w)
    assert list(enc["palette"]) == g["palette"]
    assert list(enc["brick_rawmap"]) == g["brick_rawmap"]
    assert list(enc["brick_rawbefore"]) == g["brick_rawbefore"]
    assert enc["n_raw"] == g["n_raw"]
    plain = bytes(int(h, 16) for h in g["plain_run_nibbles"])
    nib = enc["nibbles"].reshape(64, 8)
    for run in range(64):
        want = bytes(8) if run in g["raw_runs"] else plain
        assert bytes(nib[run]) == want, run
    side = enc["side"]
    assert side[0] == 200 and list(side[1:64]) == [100 + (c % 16) for c in range(1, 64)]
    assert np.array_equal(oracle.palette_decode(enc), w)


@pytest.mark.parametrize("name", ["tiny"])
def test_palette_roundtrip_config(name):
    cfg = synth.CONFIGS[name]
    w = synth.weights(cfg["rows"], cfg["cols"], cfg["seed"], cfg["p"], cfg["shift"])
    enc = oracle.palette_encode(w)
    assert np.array_equal(oracle.palette_decode(enc), w)
    # brute-force raw count (the survey computed 92 of 2048 for this draw)
    e, _ = oracle.split(w)
    ps = set(int(p) for p in enc["palette"])
    brute = sum(any(int(v) not in ps for v in e[r, 64 * g:64 * g + 64])
                for r in range(cfg["rows"]) for g in range(cfg["cols"] // 64))
    assert enc["n_raw"] == brute == 92


def test_palette_all_patterns_roundtrip():
    """Every one of the 65,536 patterns survives the palette format (all groups raw)."""
    w = synth.all_bf16_patterns()
    enc = oracle.palette_encode(w)
    assert enc["n_raw"] == 256 * 4
    assert np.array_equal(oracle.palette_decode(enc), w)


def test_pages_exponent_statistics_on_synthetic_weights():
    """Section 三: top-16 exponents cover >99% of a layer's weights and the
    exponent entropy is about 2.6 bits -- the synthetic weights must share this."""
    w = synth.weights(1024, 4096, 0, 0.0005, 10)
    cnt = oracle.histogram(oracle.split(w)[0])
    assert oracle.top_k_coverage(cnt, 16) > 0.99
    assert 2.3 < oracle.entropy_bits(cnt) < 2.9


def _bpw_cases():
    return {
        "tiny": synth.weights(256, 512, 0, 0.001, 12),
        "patterns": synth.all_bf16_patterns(),            # every group raw
        "two_exponents": ((np.arange(64 * 128).reshape(64, 128) % 2) * 0x0080 + 0x3F00).astype(np.uint16),
        "gate_slice": synth.weights(512, 4096, 0, 0.0005, 10),
    }


@pytest.mark.parametrize("name", ["tiny", "patterns", "two_exponents", "gate_slice"])
def test_bits_per_weight_count_the_stored_arrays(name):
    """bits/weight of each form = 8 x the bytes of the arrays its encoder
    returns as the stored form, divided by the weights.  Palette form:
    sign+mantissa bytes, 4-bit codes, raw side table, the two per-brick tables
    and the palette.  Huffman form: sign+mantissa bytes, stream words, chunk
    offsets and the code lengths.  The byte counts come from the arrays
    themselves, so a dropped or miscounted term in either formula fails; the
    side table must also hold 64 bytes for every raw group found by a direct
    scan (section 四: a 64-weight row with an exponent outside the palette is
    stored raw)."""
    w = _bpw_cases()[name]
    enc = oracle.palette_encode(w)
    stored = ("sm", "nibbles", "side", "brick_rawmap", "brick_rawbefore", "palette")
    bits = 8 * sum(np.asarray(enc[k]).nbytes for k in stored)
    assert abs(oracle.palette_bits_per_weight(enc) - bits / w.size) < 1e-12
    e = (w.astype(np.uint32) >> 7) & 0xFF
    in_pal = np.isin(e, np.asarray(enc["palette"]))
    raw_scan = int((~in_pal.reshape(w.shape[0], -1, 64)).any(axis=2).sum())
    assert enc["side"].nbytes == 64 * raw_scan
    he = oracle.huffman_encode(w)
    bits = 8 * sum(np.asarray(he[k]).nbytes for k in ("sm", "words", "offsets", "lengths"))
    assert abs(oracle.huffman_bits_per_weight(he) - bits / w.size) < 1e-12


def test_palette_form_at_least_20_percent_smaller_on_gate_statistics():
    """The size target (>= 20% fewer weight bytes than bf16), from the byte
    counts of the stored arrays on gate-statistics weights; the Huffman form too."""
    w = synth.weights(1024, 4096, 0, 0.0005, 10)
    enc = oracle.palette_encode(w)
    stored = ("sm", "nibbles", "side", "brick_rawmap", "brick_rawbefore", "palette")
    nbytes = sum(np.asarray(enc[k]).nbytes for k in stored)
    assert nbytes <= 0.8 * 2 * w.size
    he = oracle.huffman_encode(w)
    assert sum(np.asarray(he[k]).nbytes for k in ("sm", "words", "offsets", "lengths")) <= 0.8 * 2 * w.size
