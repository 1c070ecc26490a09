"""GPU parity of the load-time transcode: bundle -> palette form on the device.

uw_load builds the direct-palette form (codes, per-brick raw tables, raw
groups' exponents) from a bundle's Huffman form with kernels; every byte must
equal the oracle's palette encoding of the original weights, decoded weights
must be bit-exact, and matmuls on the loaded handle must meet the 1e-3 bar
against the fp64 oracle.
"""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

TOL = 1e-3

CASES = {
    "tiny": lambda: synth.weights(256, 512, 0, 0.001, 12),
    "ragged": lambda: synth.weights(272, 576, 3, 0.003, 12),
    "many_raw": lambda: synth.weights(544, 1728, 5, 0.02, 10),
    "patterns": lambda: synth.all_bf16_patterns(),
    "two_exponents": lambda: np.where(np.arange(32 * 128).reshape(32, 128) % 3 == 0, 0x3F80, 0xBF00).astype(np.uint16),
}


@pytest.fixture(scope="module")
def env():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import decode_gemm_bf16_amd as uw
    return torch, uw


def _bundle(env, w, path):
    torch, uw = env
    m = uw.Matrix(w, uw.FMT_HUFFMAN)
    m.save(str(path))
    m.free()


@pytest.mark.parametrize("name", sorted(CASES))
def test_transcoded_streams_byte_equal(env, tmp_path, name):
    torch, uw = env
    w = CASES[name]()
    p = tmp_path / "b.uwb"
    _bundle(env, w, p)
    print(f"bundle transcode {name} {w.shape}", flush=True)
    m = uw.Matrix.load(str(p), uw.FMT_HUFFMAN | uw.FMT_PALETTE)
    want = oracle.transcode_bundle(oracle.read_bundle(str(p)))
    assert np.array_equal(m.export(uw.STREAM_PALETTE), want["palette"])
    assert np.array_equal(m.export(uw.STREAM_NIBBLES), want["nibbles"])
    assert np.array_equal(m.export(uw.STREAM_RAWMAP), want["brick_rawmap"])
    assert np.array_equal(m.export(uw.STREAM_RAWBEFORE), want["brick_rawbefore"])
    assert np.array_equal(m.export(uw.STREAM_SIDE), want["side"])
    assert np.array_equal(m.export(uw.STREAM_SM), want["sm"])
    assert m.info()["raw_groups"] == want["n_raw"]
    # the largest brick-row raw count, from the oracle's tables
    kbn = w.shape[1] // 64
    rm, rb = want["brick_rawmap"], want["brick_rawbefore"]
    counts = [int(rb[b + kbn - 1]) + bin(int(rm[b + kbn - 1])).count("1") - int(rb[b]) for b in range(0, len(rm), kbn)]
    assert m.info()["max_row_raw"] == max(counts)
    # the palette-only handle decodes through the transcoded tables
    m2 = uw.Matrix.load(str(p), uw.FMT_PALETTE)
    out = torch.empty(w.shape, dtype=torch.int16, device="cuda")
    m2.decode(out)
    torch.cuda.synchronize()
    assert np.array_equal(uw.bits_of(out), w)


@pytest.mark.parametrize("name", ["tiny", "ragged", "many_raw"])
def test_matmul_on_loaded_handles(env, tmp_path, name):
    torch, uw = env
    w = CASES[name]()
    p = tmp_path / "b.uwb"
    _bundle(env, w, p)
    pal = uw.Matrix.load(str(p), uw.FMT_PALETTE)
    aux = uw.Matrix.load(str(p), uw.FMT_HUFFMAN | uw.FMT_RAWAUX)
    for tokens in (1, 16, 100):
        xb = synth.activations(tokens, w.shape[1], xseed=tokens)
        ref = oracle.matmul_fp64(xb, w)
        x = uw.bf16_tensor(xb)
        for m, pipe in ((pal, uw.P4_DIRECT_PALETTE), (aux, uw.P3_PALETTE_TRANSCODE), (aux, uw.P2_EXP_DECODE)):
            print(f"bundle matmul {name} tokens {tokens} P{pipe}", flush=True)
            y = torch.full((tokens, w.shape[0]), float("nan"), device="cuda", dtype=torch.float32)
            m.matmul(x, y, pipeline=pipe)
            torch.cuda.synchronize()
            assert oracle.rel_err(y.cpu().numpy(), ref) <= TOL, (tokens, pipe)


def test_gate_shape_load(env, tmp_path):
    """The 14336 x 4096 gate: the loaded palette form equals the host
    encoder's, and P4 on it gives the same floats as on the encoded handle."""
    torch, uw = env
    c = synth.CONFIGS["gate_8b"]
    w = synth.weights(c["rows"], c["cols"], c["seed"], c["p"], c["shift"])
    p = tmp_path / "gate.uwb"
    _bundle(env, w, p)
    print("bundle gate load", flush=True)
    loaded = uw.Matrix.load(str(p), uw.FMT_PALETTE)
    host = uw.Matrix(w, uw.FMT_PALETTE | uw.ENC_HOST_ONLY)
    for s in (uw.STREAM_PALETTE, uw.STREAM_NIBBLES, uw.STREAM_RAWMAP, uw.STREAM_RAWBEFORE, uw.STREAM_SIDE):
        assert np.array_equal(loaded.export(s), host.export(s)), s
    enc = uw.Matrix(w, uw.FMT_PALETTE)
    xb = synth.activations(1, c["cols"], xseed=1)
    x = uw.bf16_tensor(xb)
    ys = []
    for m in (loaded, enc):
        y = torch.empty((1, c["rows"]), device="cuda", dtype=torch.float32)
        m.matmul(x, y, pipeline=uw.P4_DIRECT_PALETTE)
        torch.cuda.synchronize()
        ys.append(y.cpu().numpy())
    assert np.array_equal(ys[0], ys[1])
    rows = np.arange(0, c["rows"], 997)
    ref = oracle.matmul_fp64_rows(xb, w, rows)
    assert oracle.rel_err(ys[0][:, rows], ref) <= TOL
