"""The C++ host encoder against the oracle, byte for byte (CPU only).

Host-only handles (UW_ENC_HOST_ONLY) run the library's encoder without touching
a device; every stored stream is exported and compared with the oracle's.
Also: every symbol declared in include/uw.h is exported by libuw.so, and the
host-side argument checks return the documented status codes.
"""
import ctypes as C
import os
import re

import numpy as np
import pytest

import decode_gemm_bf16_amd as uw
import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST_ALL = uw.FMT_HUFFMAN | uw.FMT_PALETTE | uw.ENC_HOST_ONLY


def test_header_symbols_exported():
    hdr = open(os.path.join(ROOT, "include", "uw.h")).read()
    declared = set(re.findall(r"\b(uw_[a-z0-9_]+)\s*\(", hdr))
    assert declared, "no declarations found"
    lib = C.CDLL(uw.LIB_PATH)
    for name in sorted(declared):
        assert hasattr(lib, name), name
    assert declared == set(uw.EXPORTED)


def _compare(w, formats=HOST_ALL):
    m = uw.Matrix(w, formats)
    pe = oracle.palette_encode(w)
    he = oracle.huffman_encode(w)
    info = m.info()
    assert np.array_equal(m.export(uw.STREAM_SM), pe["sm"])
    if formats & uw.FMT_PALETTE:
        assert np.array_equal(m.export(uw.STREAM_PALETTE), pe["palette"])
        assert np.array_equal(m.export(uw.STREAM_NIBBLES), pe["nibbles"])
    if formats & (uw.FMT_PALETTE | uw.FMT_RAWAUX):
        assert np.array_equal(m.export(uw.STREAM_RAWMAP), pe["brick_rawmap"])
        assert np.array_equal(m.export(uw.STREAM_RAWBEFORE), pe["brick_rawbefore"])
        assert np.array_equal(m.export(uw.STREAM_SIDE), pe["side"])
        assert info["raw_groups"] == pe["n_raw"]
        assert abs(info["bpw_palette"] - oracle.palette_bits_per_weight(pe)) < 1e-9
    if formats & uw.FMT_HUFFMAN:
        assert np.array_equal(m.export(uw.STREAM_LENGTHS), he["lengths"])
        assert np.array_equal(m.export(uw.STREAM_WORDS), he["words"])
        assert np.array_equal(m.export(uw.STREAM_OFFSETS), he["offsets"])
        assert info["stream_bits"] == he["total_bits"]
        assert abs(info["bpw_huffman"] - oracle.huffman_bits_per_weight(he)) < 1e-9
    m.free()


def test_tiny_config_byte_for_byte():
    c = synth.CONFIGS["tiny"]
    _compare(synth.weights(c["rows"], c["cols"], c["seed"], c["p"], c["shift"]))


def test_all_patterns_byte_for_byte():
    _compare(synth.all_bf16_patterns())


@pytest.mark.parametrize("seed,rows,cols,p,shift", [(3, 48, 192, 0.01, 12), (4, 16, 64, 0.0, 0),
                                                     (5, 160, 320, 0.003, 10), (6, 32, 4096, 0.0005, 10)])
def test_random_shapes_byte_for_byte(seed, rows, cols, p, shift):
    _compare(synth.weights(rows, cols, seed, p, shift))


def test_single_exponent_and_few_exponents():
    _compare(np.zeros((16, 64), np.uint16))                 # one symbol: phantom code
    rng = np.random.default_rng(1)
    e = rng.integers(120, 124, size=(32, 128)).astype(np.uint16)
    _compare(((e << 7) | rng.integers(0, 256, size=e.shape).astype(np.uint16) & 0x807F).astype(np.uint16))


def test_golden_fixture_through_library():
    w = np.full((16, 64), 120 << 7, dtype=np.uint16)
    w[0, 1] = 121 << 7
    w[0, 2] = 122 << 7
    m = uw.Matrix(w, HOST_ALL)
    words = m.export(uw.STREAM_WORDS)
    assert len(words) == 33 and words[0] == 0x58000000 and not words[1:].any()
    assert list(m.export(uw.STREAM_OFFSETS)) == [0, 258, 514, 770]


def test_format_subsets():
    w = synth.weights(64, 256, 8, 0.004, 12)
    _compare(w, uw.FMT_HUFFMAN | uw.ENC_HOST_ONLY)
    _compare(w, uw.FMT_HUFFMAN | uw.FMT_RAWAUX | uw.ENC_HOST_ONLY)
    _compare(w, uw.FMT_PALETTE | uw.ENC_HOST_ONLY)
    m = uw.Matrix(w, uw.FMT_HUFFMAN | uw.ENC_HOST_ONLY)
    with pytest.raises(uw.UwError) as e:
        m.export(uw.STREAM_NIBBLES)
    assert e.value.status == uw.ERR_UNSUPPORTED


def test_bad_shapes_and_args():
    for shape in [(15, 64), (16, 96), (0, 64)]:
        with pytest.raises(uw.UwError) as e:
            uw.Matrix(np.zeros(shape, np.uint16), HOST_ALL)
        assert e.value.status == uw.ERR_SHAPE
    with pytest.raises(uw.UwError) as e:
        uw.Matrix(np.zeros((16, 64), np.uint16), uw.ENC_HOST_ONLY)
    assert e.value.status == uw.ERR_INVALID_ARG
    with pytest.raises(uw.UwError) as e:
        uw.Matrix(np.zeros((16, 64), np.uint16), 0x8 | uw.ENC_HOST_ONLY)
    assert e.value.status == uw.ERR_INVALID_ARG
    h = C.c_void_p()
    assert uw._lib.uw_encode(None, 16, 64, HOST_ALL, C.byref(h)) == uw.ERR_INVALID_ARG
    assert "null" in uw.last_error()


def test_host_only_handle_rejects_device_calls():
    m = uw.Matrix(synth.weights(16, 64, 1, 0.0, 0), HOST_ALL)
    with pytest.raises(uw.UwError) as e:
        uw._check(uw._lib.uw_matmul(m._h, 8, 8, 1, uw.P4_DIRECT_PALETTE))
    assert e.value.status == uw.ERR_UNSUPPORTED
    with pytest.raises(uw.UwError):
        uw._check(uw._lib.uw_decode(m._h, 8))
    with pytest.raises(uw.UwError):
        m.set_plan([(64, 9, 0)])


def test_variant_names():
    assert uw.variant_name(1, 0) == "small:default"
    assert uw.variant_name(1024, 0) == "large:default"
    assert len(uw.variants(1)) > 5 and len(uw.variants(256)) > 5
    assert uw.variant_name(1, 999) is None


def test_variant_in_use_resolution():
    """Which pipeline and kernel shape a call would run (no GPU work): the
    built-in rule, the exponent-form fallback of the LDS-activation shapes,
    an explicit variant and a plan."""
    m = uw.Matrix(synth.weights(2048, 4096, 1, 0.0005, 10), HOST_ALL)
    # two bricks in flight per wave whatever the bricks per wave (8, 16, 28)
    assert m.variant_in_use(1) == (uw.P4_DIRECT_PALETTE, "gemv:w8:d2")
    for cols, name in ((8192, "gemv:w8:d2"), (14336, "gemv:w8:d2")):
        wide = uw.Matrix(synth.weights(2048, cols, 1, 0.0005, 10), HOST_ALL)
        assert wide.variant_in_use(1) == (uw.P4_DIRECT_PALETTE, name), cols
        wide.free()
    assert m.variant_in_use(1, uw.P1_FULL_DECODE)[1] == "hipblaslt"
    assert m.variant_in_use(1024, uw.P5_PALETTE_DECODE) == (uw.P5_PALETTE_DECODE, "hipblaslt")
    # the exponent form has no palette codes: the small kernel runs instead
    p, name = m.variant_in_use(1, uw.P2_EXP_DECODE)
    assert p == uw.P2_EXP_DECODE and name.startswith("small:")
    # 5 tokens x 4096 columns no longer fit the LDS activation buffer
    assert m.variant_in_use(5)[1].startswith("small:")
    assert m.variant_in_use(1024)[1].startswith("large:")
    v = uw.variants(1).index("small:w8:k1:u2")
    m.set_variant(v)
    assert m.variant_in_use(1, uw.P4_DIRECT_PALETTE) == (uw.P4_DIRECT_PALETTE, "small:w8:k1:u2")
    m.set_variant(0)
    # a plan selects pipeline and variant per batch size
    vl = uw.variants(100).index("large:t5(4x32r x128t,32x32):k1")
    m.set_plan([(16, uw.P1_FULL_DECODE, 0), (64, uw.P4_DIRECT_PALETTE, v), (1 << 30, uw.P4_DIRECT_PALETTE, vl)])
    assert m.variant_in_use(1) == (uw.P1_FULL_DECODE, "hipblaslt")
    assert m.variant_in_use(17) == (uw.P4_DIRECT_PALETTE, "small:w8:k1:u2")
    assert m.variant_in_use(100) == (uw.P4_DIRECT_PALETTE, "large:t5(4x32r x128t,32x32):k1")
    # a variant id names a kernel of its batch family (<= 64 tokens or more):
    # an entry tuned above 64 tokens keeps only its pipeline for 17 tokens
    m.set_plan([(1 << 30, uw.P4_DIRECT_PALETTE, vl)])
    assert m.variant_in_use(17) == m.variant_in_use(17, uw.P4_DIRECT_PALETTE)
    with pytest.raises(uw.UwError) as e:
        uw.Matrix(synth.weights(64, 64, 1, 0.0, 0), uw.FMT_PALETTE | uw.ENC_HOST_ONLY).variant_in_use(1, uw.P1_FULL_DECODE)
    assert e.value.status in (uw.ERR_UNSUPPORTED, uw.ERR_INVALID_ARG)


def test_wide_tile_choice():
    """The 128-row x 512-token tile is the built-in choice from 768 tokens
    where its workgroups fill at least 192 CUs; its brick tables live in LDS,
    so for K beyond 256 bricks an explicit request falls back to the
    built-in choice of the shape (no GPU work)."""
    tall = uw.Matrix(synth.weights(14336, 1024, 1, 0.0005, 10), HOST_ALL)  # 112 row blocks of 128
    assert tall.variant_in_use(1024)[1].startswith("large:t22")
    assert tall.variant_in_use(768)[1].startswith("large:t22")
    assert not tall.variant_in_use(512)[1].startswith("large:t22")  # 112 workgroups: half the chip
    tall.free()
    short = uw.Matrix(synth.weights(4096, 1024, 1, 0.0005, 10), HOST_ALL)  # 32 row blocks
    assert not short.variant_in_use(1024)[1].startswith("large:t22")
    short.free()
    longk = uw.Matrix(synth.weights(64, 257 * 64, 1, 0.0005, 10), HOST_ALL)  # K of 257 bricks
    v = uw.variants(1024).index("large:t22(128r x 4x128t,32x32,wide)")
    longk.set_variant(v)
    assert longk.variant_in_use(1024) == (uw.P4_DIRECT_PALETTE, longk.variant_in_use(1024, uw.P4_DIRECT_PALETTE)[1])
    assert not longk.variant_in_use(1024)[1].startswith("large:t22")
    longk.free()


def test_bits_per_weight_on_gate_shaped_slice():
    """North-star size target: >= 20% fewer weight bytes than bf16 in both forms."""
    w = synth.weights(1024, 4096, 0, 0.0005, 10)
    inf = uw.Matrix(w, HOST_ALL).info()
    assert inf["bpw_palette"] < 16 * 0.8 and inf["bpw_huffman"] < 16 * 0.8


def test_max_row_raw_matches_exported_tables():
    """uw_info.max_row_raw (which selects the gemv kernel's LDS copy of the raw
    groups) equals the largest per-brick-row raw count of the exported
    tables; a matrix with no palette tables reports all ones."""
    for rows, cols, p in ((256, 512, 0.003), (272, 1024, 0.02), (64, 4096, 0.0)):
        w = synth.weights(rows, cols, 5, p, 12)
        m = uw.Matrix(w, HOST_ALL)
        rawmap = m.export(uw.STREAM_RAWMAP)
        before = m.export(uw.STREAM_RAWBEFORE)
        kbn = cols // 64
        counts = [int(before[b + kbn - 1]) + bin(int(rawmap[b + kbn - 1])).count("1") - int(before[b])
                  for b in range(0, len(rawmap), kbn)]
        assert m.info()["max_row_raw"] == max(counts)
    h = uw.Matrix(synth.weights(256, 512, 5, 0.003, 12), uw.FMT_HUFFMAN | uw.ENC_HOST_ONLY)
    assert h.info()["max_row_raw"] == 0xFFFFFFFF


def test_scratch_sizes_per_pipeline():
    """uw_info.scratch_bytes: full decodes (pipelines 1 and 5) hold W as bf16,
    256-byte aligned; pipelines 2 and 3 hold 16 exponent bytes / 8 code bytes
    per run, padded to whole groups of 512 chunks of 256 weights; pipeline 4
    needs none."""
    rows, cols = 272, 576
    m = uw.Matrix(synth.weights(rows, cols, 2, 0.003, 12), HOST_ALL)
    sb = m.info()["scratch_bytes"]
    n = rows * cols
    groups = (n // 256 + 511) // 512
    assert sb[1] == sb[5] == (2 * n + 255) // 256 * 256
    assert sb[2] == groups * 512 * 256 and sb[3] == groups * 512 * 128
    assert sb[4] == 0


def test_fused_activation_limit_checked_on_the_host():
    """The fused kernels (pipelines 2-4) address X through a 32-bit buffer
    range: tokens x cols x 2 bytes above 0x7FFFFFF0 is UW_ERR_SHAPE, checked
    before the handle's residency (a host-only handle reaches the check; no
    device memory is touched, the pointers are never dereferenced).  The
    library GEMM of pipelines 1 and 5 has no such limit."""
    m = uw.Matrix(synth.weights(16, 4096, 1, 0.0, 0), HOST_ALL)
    big = 1 << 18  # 2^18 tokens x 4096 columns x 2 bytes = 2^31 bytes
    for p in (2, 3, 4):
        assert uw._lib.uw_matmul(m._h, 8, 8, big, p) == uw.ERR_SHAPE, p
        assert "limit" in uw.last_error()
    for p in (1, 5):
        assert uw._lib.uw_matmul(m._h, 8, 8, big, p) == uw.ERR_UNSUPPORTED, p
    # one token less: 2^31 - 8192 bytes pass the check, then the host-only refusal
    assert uw._lib.uw_matmul(m._h, 8, 8, big - 1, 4) == uw.ERR_UNSUPPORTED
    # the grouped form checks every expert before launching any
    offs = (C.c_int64 * 3)(0, 1, 1 + big)
    hs = (C.c_void_p * 2)(m.handle, m.handle)
    assert uw._lib.uw_grouped_matmul(hs, 2, 8, offs, 8, 4) == uw.ERR_UNSUPPORTED  # host-only first


def test_layer_runner_host_checks():
    """uw_mlp_forward and uw_stack_forward validate shapes, streams and token
    counts of every projection before launching anything (host-only handles:
    the last check standing is the residency one)."""
    mk = lambda seed: uw.Matrix(synth.weights(64, 64, seed, 0.0, 0), HOST_ALL)
    g, u, d = mk(1), mk(2), mk(3)
    p3 = (C.c_int32 * 3)(4, 4, 4)
    ws = uw._lib.uw_mlp_workspace_bytes(2, 64)
    assert uw._lib.uw_mlp_forward(g._h, u._h, d._h, p3, 8, 8, 2, 8, ws) == uw.ERR_UNSUPPORTED
    assert uw._lib.uw_mlp_forward(g._h, u._h, d._h, p3, 8, 8, 0, 8, ws) == uw.ERR_INVALID_ARG
    assert uw._lib.uw_mlp_forward(g._h, u._h, d._h, p3, 8, 8, 2, 8, ws - 1) == uw.ERR_INVALID_ARG
    u.set_streams(main=0x1000)  # never used: the check fails first
    assert uw._lib.uw_mlp_forward(g._h, u._h, d._h, p3, 8, 8, 2, 8, ws) == uw.ERR_INVALID_ARG
    assert "stream" in uw.last_error()
    u.set_streams()
    wide = uw.Matrix(synth.weights(128, 64, 4, 0.0, 0), HOST_ALL)  # a layer of another shape
    hs = (C.c_void_p * 6)(g.handle, u.handle, d.handle, wide.handle, u.handle, d.handle)
    p6 = (C.c_int32 * 6)(4, 4, 4, 4, 4, 4)
    sws = uw._lib.uw_stack_workspace_bytes(2, 64, 64)
    assert uw._lib.uw_stack_forward(hs, p6, 2, 8, 8, 2, 0, 8, sws) == uw.ERR_SHAPE
    assert uw._lib.uw_stack_forward(hs, p6, 2, 8, 8, 0, 0, 8, sws) == uw.ERR_INVALID_ARG
    hs_ok = (C.c_void_p * 6)(g.handle, u.handle, d.handle, g.handle, u.handle, d.handle)
    assert uw._lib.uw_stack_forward(hs_ok, p6, 2, 8, 8, 2, 0, 8, sws) == uw.ERR_UNSUPPORTED


def test_library_bits_per_weight_count_its_exported_streams():
    """uw_info's bits/weight of each form equal 8 x the bytes of the streams
    uw_export hands out for that form (the 8-byte per-brick table counted as
    the two exported 4-byte tables), divided by the weights."""
    for w in (synth.weights(256, 512, 0, 0.001, 12), synth.weights(512, 4096, 0, 0.0005, 10)):
        m = uw.Matrix(w, HOST_ALL)
        info = m.info()
        size = lambda s: m.export(s).nbytes
        pal = sum(size(s) for s in (uw.STREAM_SM, uw.STREAM_NIBBLES, uw.STREAM_SIDE, uw.STREAM_RAWMAP,
                                    uw.STREAM_RAWBEFORE, uw.STREAM_PALETTE))
        huf = sum(size(s) for s in (uw.STREAM_SM, uw.STREAM_WORDS, uw.STREAM_OFFSETS, uw.STREAM_LENGTHS))
        assert abs(info["bpw_palette"] - 8 * pal / w.size) < 1e-12
        assert abs(info["bpw_huffman"] - 8 * huf / w.size) < 1e-12
        m.free()
