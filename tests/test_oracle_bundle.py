"""Pins of oracle/bundle.py (CPU only): the bundle round trip recovers the
weights through the Huffman decoder, the header fields sit where the layout
puts them, and the load-time transcode equals the palette encoding of the
original weights (the Huffman round trip is exact)."""
import struct

import numpy as np
import pytest

import oracle
import synth

CASES = {
    "tiny": lambda: synth.weights(256, 512, 0, 0.001, 12),
    "patterns": lambda: synth.all_bf16_patterns(),
    "one_exponent": lambda: np.full((16, 64), 0x3F80, dtype=np.uint16),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_round_trip(tmp_path, name):
    w = CASES[name]()
    enc = oracle.huffman_encode(w)
    p = tmp_path / "b.uwb"
    oracle.write_bundle(str(p), enc)
    back = oracle.read_bundle(str(p))
    assert np.array_equal(oracle.huffman_decode(back), w)
    assert np.array_equal(back["counts"], enc["counts"])
    n = w.size
    assert p.stat().st_size == 64 + 8 * 256 + 4 * len(enc["offsets"]) + 4 * len(enc["words"]) + n


def test_header_fields(tmp_path):
    w = CASES["tiny"]()
    enc = oracle.huffman_encode(w)
    p = tmp_path / "b.uwb"
    oracle.write_bundle(str(p), enc)
    raw = p.read_bytes()
    assert raw[:8] == b"UWBUNDLE"
    assert struct.unpack_from("<II", raw, 8) == (1, 64)
    assert struct.unpack_from("<qq", raw, 16) == (256, 512)
    # the histogram follows the header and counts every weight once
    counts = np.frombuffer(raw, dtype="<u8", count=256, offset=64)
    assert int(counts.sum()) == w.size
    assert np.array_equal(counts, np.bincount(((w >> 7) & 0xFF).astype(np.int64).ravel(), minlength=256))


def test_reader_rejects_trailing_bytes(tmp_path):
    p = tmp_path / "b.uwb"
    oracle.write_bundle(str(p), oracle.huffman_encode(CASES["tiny"]()))
    p.write_bytes(p.read_bytes() + b"\0")
    with pytest.raises(ValueError):
        oracle.read_bundle(str(p))


@pytest.mark.parametrize("name", ["tiny", "patterns"])
def test_transcode_is_palette_of_original(name):
    w = CASES[name]()
    got = oracle.transcode_bundle(oracle.huffman_encode(w))
    want = oracle.palette_encode(w)
    for k in ("palette", "nibbles", "brick_rawmap", "brick_rawbefore", "side", "sm"):
        assert np.array_equal(got[k], want[k]), k
