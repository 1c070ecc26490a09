"""Distribution bundle files (CPU only).

The oracle's bundle reader/writer against the library's uw_save/uw_load
(two independent implementations of one byte layout), the round trip to the
original weights through the oracle's Huffman decoder, and the documented
error statuses of uw_load.  Palette formats of a loaded bundle are built on
the device; those are tested in test_gpu_bundle.py.
"""
import os
import struct

import numpy as np
import pytest

import decode_gemm_bf16_amd as uw
import oracle
import synth

HOST_HUF = uw.FMT_HUFFMAN | uw.ENC_HOST_ONLY

CASES = {
    "tiny": lambda: synth.weights(256, 512, 0, 0.001, 12),
    "ragged": lambda: synth.weights(272, 576, 3, 0.003, 12),
    "patterns": lambda: synth.all_bf16_patterns(),
    "two_exponents": lambda: np.where(np.arange(16 * 64).reshape(16, 64) % 3 == 0, 0x3F80, 0xBF00).astype(np.uint16),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_library_writer_matches_oracle_writer(tmp_path, name):
    w = CASES[name]()
    m = uw.Matrix(w, HOST_HUF)
    lib_path, orc_path = tmp_path / "lib.uwb", tmp_path / "oracle.uwb"
    m.save(str(lib_path))
    enc = oracle.huffman_encode(w)
    oracle.write_bundle(str(orc_path), enc)
    assert lib_path.read_bytes() == orc_path.read_bytes()
    back = oracle.read_bundle(str(lib_path))
    assert np.array_equal(oracle.huffman_decode(back), w)
    for k in ("words", "offsets", "lengths", "sm"):
        assert np.array_equal(back[k], enc[k]), k
    assert back["total_bits"] == enc["total_bits"]


def test_header_fields(tmp_path):
    w = CASES["tiny"]()
    p = tmp_path / "b.uwb"
    uw.Matrix(w, HOST_HUF).save(str(p))
    raw = p.read_bytes()
    magic, version, hbytes, rows, cols, bits = struct.unpack_from("<8sIIqqQ", raw, 0)
    chunk, lmax, nwords, noff = struct.unpack_from("<IIQQ", raw, 40)
    enc = oracle.huffman_encode(w)
    assert (magic, version, hbytes, rows, cols) == (b"UWBUNDLE", 1, 64, 256, 512)
    assert (bits, chunk, lmax) == (enc["total_bits"], 256, 12)
    assert nwords == (bits + 31) // 32 and noff == 256 * 512 // 256
    assert len(raw) == 64 + 2048 + 4 * noff + 4 * nwords + 256 * 512


@pytest.mark.parametrize("name", sorted(CASES))
def test_host_load_of_oracle_bundle(tmp_path, name):
    w = CASES[name]()
    enc = oracle.huffman_encode(w)
    p = tmp_path / "b.uwb"
    oracle.write_bundle(str(p), enc)
    m = uw.Matrix.load(str(p), HOST_HUF)
    assert (m.rows, m.cols) == w.shape
    assert np.array_equal(m.export(uw.STREAM_WORDS), enc["words"])
    assert np.array_equal(m.export(uw.STREAM_OFFSETS), enc["offsets"])
    assert np.array_equal(m.export(uw.STREAM_LENGTHS), enc["lengths"])
    assert np.array_equal(m.export(uw.STREAM_SM), enc["sm"])
    assert m.info()["stream_bits"] == enc["total_bits"]
    # and it writes back the same file
    q = tmp_path / "c.uwb"
    m.save(str(q))
    assert q.read_bytes() == p.read_bytes()


def _status(fn):
    with pytest.raises(uw.UwError) as e:
        fn()
    return e.value.status


def test_load_errors(tmp_path):
    w = CASES["tiny"]()
    good = tmp_path / "good.uwb"
    uw.Matrix(w, HOST_HUF).save(str(good))
    raw = bytearray(good.read_bytes())

    assert _status(lambda: uw.Matrix.load(str(tmp_path / "missing.uwb"), HOST_HUF)) == uw.ERR_IO
    bad = tmp_path / "bad.uwb"
    bad.write_bytes(b"NOTABNDL" + bytes(raw[8:]))
    assert _status(lambda: uw.Matrix.load(str(bad), HOST_HUF)) == uw.ERR_IO
    bad.write_bytes(bytes(raw[:-1]))  # truncated sign+mantissa bytes
    assert _status(lambda: uw.Matrix.load(str(bad), HOST_HUF)) == uw.ERR_IO
    bad.write_bytes(bytes(raw) + b"\0")  # a byte past the end
    assert _status(lambda: uw.Matrix.load(str(bad), HOST_HUF)) == uw.ERR_FORMAT
    h = bytearray(raw)
    counts = np.frombuffer(bytes(h[64:64 + 2048]), dtype="<u8").copy()
    s = int(np.argmax(counts))
    counts[s] -= 1  # histogram no longer sums to rows*cols
    h[64:64 + 2048] = counts.tobytes()
    bad.write_bytes(bytes(h))
    assert _status(lambda: uw.Matrix.load(str(bad), HOST_HUF)) == uw.ERR_FORMAT
    h = bytearray(raw)
    struct.pack_into("<Q", h, 32, struct.unpack_from("<Q", raw, 32)[0] + 1)  # stream bits off by one
    bad.write_bytes(bytes(h))
    assert _status(lambda: uw.Matrix.load(str(bad), HOST_HUF)) == uw.ERR_FORMAT
    h = bytearray(raw)
    struct.pack_into("<I", h, 8, 2)  # unknown version
    bad.write_bytes(bytes(h))
    assert _status(lambda: uw.Matrix.load(str(bad), HOST_HUF)) == uw.ERR_FORMAT
    h = bytearray(raw)
    struct.pack_into("<q", h, 16, 250)  # rows not a multiple of 16
    bad.write_bytes(bytes(h))
    assert _status(lambda: uw.Matrix.load(str(bad), HOST_HUF)) == uw.ERR_SHAPE
    # palette tables need the device
    assert _status(lambda: uw.Matrix.load(str(good), uw.FMT_PALETTE | uw.ENC_HOST_ONLY)) == uw.ERR_UNSUPPORTED
    assert _status(lambda: uw.Matrix.load(str(good), 0)) == uw.ERR_INVALID_ARG


def test_save_needs_huffman(tmp_path):
    m = uw.Matrix(CASES["tiny"](), uw.FMT_PALETTE | uw.ENC_HOST_ONLY)
    assert _status(lambda: m.save(str(tmp_path / "x.uwb"))) == uw.ERR_UNSUPPORTED
    assert not os.path.exists(tmp_path / "x.uwb")


def test_upload_evict_grouped_host_checks():
    """Host-side argument checks of the expert entry points (no device here)."""
    w = CASES["tiny"]()
    m = uw.Matrix(w, uw.FMT_PALETTE | uw.ENC_HOST_ONLY)
    m.evict()  # host-only: nothing to release
    m2 = uw.Matrix(synth.weights(256, 1024, 1, 0.001, 12), uw.FMT_PALETTE | uw.ENC_HOST_ONLY)
    x = np.zeros((4, 512), dtype=np.uint16)
    y = np.zeros((4, 256), dtype=np.float32)
    assert _status(lambda: uw.grouped_matmul([m, m2], x, y, [0, 2, 4])) == uw.ERR_SHAPE
    assert _status(lambda: uw.grouped_matmul([m, m], x, y, [0, 3, 2])) == uw.ERR_INVALID_ARG
    assert _status(lambda: uw.grouped_matmul([m, m], x, y, [1, 2, 4])) == uw.ERR_INVALID_ARG
    assert _status(lambda: uw.grouped_matmul([m, m], x, y, [0, 2, 4])) == uw.ERR_UNSUPPORTED
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:
        has_gpu = False
    if not has_gpu:
        assert _status(m.upload) == uw.ERR_NO_DEVICE
