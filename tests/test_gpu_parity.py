"""GPU parity: the HIP path (through the C ABI) against the oracle.

Bar (from the method): decoded weights and every intermediate stream
(exponent bytes, 4-bit codes) bit-exact; matmul outputs within
max|gpu - ref| / max|ref| <= 1e-3 of the fp64 oracle; one-hot activations
reproduce weights exactly (an fp32 sum of one exact product).
"""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

TOL = 1e-3


@pytest.fixture(scope="module")
def env():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import decode_gemm_bf16_amd as uw
    return torch, uw


def _dev_x(env, x_bits):
    torch, uw = env
    return uw.bf16_tensor(x_bits)


def _run(env, m, x_bits, pipeline, variant=0):
    torch, uw = env
    x = uw.bf16_tensor(x_bits)
    y = torch.full((x_bits.shape[0], m.rows), float("nan"), device="cuda", dtype=torch.float32)
    m.set_variant(variant)
    m.matmul(x, y, pipeline=pipeline)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _both(env, w):
    torch, uw = env
    return uw.Matrix(w, uw.FMT_HUFFMAN | uw.FMT_PALETTE)


def test_mfma_fragment_layout_one_hot(env):
    """One-hot activations: Y[m, n] == W[n, k_m] exactly for every pipeline and
    small/large batch (checks reconstruction and the MFMA output layout)."""
    torch, uw = env
    w = synth.weights(48, 256, 11, 0.01, 12)
    m = _both(env, w)
    ref_bits = w
    for tokens in (1, 5, 16, 17, 64, 65, 130):
        x, ks = synth.one_hot_activations(tokens, 256, seed=tokens)
        for p in (1, 2, 3, 4, 5):
            y = _run(env, m, x, p)
            want = synth.bf16_bits_to_f32(ref_bits[:, ks].T.copy())
            assert np.array_equal(y, want), (tokens, p)


@pytest.mark.parametrize("name", ["tiny", "patterns", "ragged"])
def test_decode_bit_exact(env, name):
    torch, uw = env
    if name == "tiny":
        c = synth.CONFIGS["tiny"]
        w = synth.weights(c["rows"], c["cols"], c["seed"], c["p"], c["shift"])
    elif name == "patterns":
        w = synth.all_bf16_patterns()
    else:
        w = synth.weights(272, 576, 3, 0.003, 12)
    for fmt in (uw.FMT_HUFFMAN, uw.FMT_PALETTE, uw.FMT_HUFFMAN | uw.FMT_PALETTE):
        m = uw.Matrix(w, fmt)
        out = torch.empty(w.shape, dtype=torch.int16, device="cuda")
        m.decode(out)
        torch.cuda.synchronize()
        assert np.array_equal(uw.bits_of(out), w), fmt


def _serial_from_interleaved(buf, n, run_bytes):
    """Undo the scratch order of pipelines 2/3 (as the header states it): run
    r of chunk c (256 weights, 16 runs) sits at run slot (c//512*16 + r)*512 + c%512."""
    chunks = n // 256
    c = np.arange(chunks)[:, None]
    r = np.arange(16)[None, :]
    slot = (c // 512 * 16 + r) * 512 + c % 512        # [chunk, run]
    runs = buf.reshape(-1, run_bytes)
    return runs[slot.reshape(-1)].reshape(-1)[: n * run_bytes // 16]


@pytest.mark.parametrize("data", ["ragged", "patterns"])
def test_preprocess_streams_bit_exact(env, data):
    """Pipeline 2's exponent bytes and pipeline 3's 4-bit codes equal the
    oracle's -- on low-entropy weights (stream staged in LDS) and on all 65,536
    bit patterns (8 bits per exponent: the stream is read from global memory)."""
    torch, uw = env
    w = synth.weights(272, 576, 5, 0.004, 12) if data == "ragged" else synth.all_bf16_patterns(1)
    m = _both(env, w)
    inf = m.info()
    e_serial = oracle.to_serial(oracle.split(w)[0])
    pe = oracle.palette_encode(w)
    for p, want in ((2, e_serial), (3, pe["nibbles"]), (1, w), (5, w)):
        buf = torch.empty(inf["scratch_bytes"][p], dtype=torch.uint8, device="cuda")
        m.set_scratch(buf)
        m.preprocess(p)
        torch.cuda.synchronize()
        got = buf.cpu().numpy()
        if p in (1, 5):
            got = got[: w.size * 2].view(np.uint16).reshape(w.shape)
        else:
            got = _serial_from_interleaved(got, w.size, 16 if p == 2 else 8)
        assert np.array_equal(got, want), p
    # the resident palette codes uploaded by the encoder, read back from the device
    assert np.array_equal(m.export(uw.STREAM_NIBBLES), pe["nibbles"])


@pytest.mark.parametrize("shape", [(256, 512), (272, 576), (48, 4096)])
@pytest.mark.parametrize("tokens", [1, 3, 16, 33, 64, 65, 129, 300])
def test_matmul_random_all_pipelines(env, shape, tokens):
    torch, uw = env
    rows, cols = shape
    w = synth.weights(rows, cols, 0, 0.001, 12)
    x = synth.activations(tokens, cols, xseed=1)
    ref = oracle.matmul_fp64(x, w)
    m = _both(env, w)
    for p in (1, 2, 3, 4, 5):
        y = _run(env, m, x, p)
        assert np.isfinite(y).all(), p
        assert oracle.rel_err(y, ref) <= TOL, (p, oracle.rel_err(y, ref))


@pytest.mark.parametrize("tokens", [1, 16, 40, 64, 100, 256])
def test_every_variant(env, tokens):
    torch, uw = env
    w = synth.weights(528, 1024, 2, 0.002, 12)
    x = synth.activations(tokens, 1024, xseed=3)
    ref = oracle.matmul_fp64(x, w)
    m = _both(env, w)
    names = uw.variants(tokens)
    for v in range(len(names)):
        for p in (2, 4):
            y = _run(env, m, x, p, variant=v)
            assert oracle.rel_err(y, ref) <= TOL, (names[v], p)


@pytest.mark.parametrize("tokens", [17, 40, 64, 80, 100, 128, 200])
def test_ragged_k_slices_and_ring_tails(env, tokens):
    """K of 27 bricks (1728 columns), 34 brick-rows: the mid kernels split K
    into slices of unequal length (float atomics into a zeroed Y), the ring
    tiles run a step count that is not a multiple of their register ring and
    a last row block with absent brick-rows; every variant, both the exponent
    form (pipeline 2, interleaved scratch) and the direct palette form."""
    torch, uw = env
    w = synth.weights(544, 1728, 5, 0.003, 11)
    x = synth.activations(tokens, 1728, xseed=7)
    ref = oracle.matmul_fp64(x, w)
    m = _both(env, w)
    names = uw.variants(tokens)
    picked = [v for v, n in enumerate(names)
              if n.startswith(("mid", "rowk", "large:t1", "large:t22", "small:default", "large:default"))]
    assert picked
    for v in picked:
        for p in (2, 4):
            y = _run(env, m, x, p, variant=v)
            assert oracle.rel_err(y, ref) <= TOL, (names[v], p, oracle.rel_err(y, ref))


@pytest.mark.parametrize("tokens", [513, 700, 1024])
def test_wide_tile_partial_blocks(env, tokens):
    """The 128-row x 512-token tile (weights rebuilt into LDS once per 512
    tokens) on 34 brick-rows (the last row block has 2 of 8), 27 bricks along
    K (an odd count: the loop runs one brick column past the end) and a last
    token block that is partly or wholly empty; exponent form (pipeline 2),
    runtime transcode (3) and direct palette (4) against fp64."""
    torch, uw = env
    w = synth.weights(544, 1728, 5, 0.003, 11)
    x = synth.activations(tokens, 1728, xseed=11)
    ref = oracle.matmul_fp64(x, w)
    m = _both(env, w)
    names = uw.variants(tokens)
    v = next(i for i, n in enumerate(names) if n.startswith("large:t22"))
    for p in (2, 3, 4):
        y = _run(env, m, x, p, variant=v)
        assert oracle.rel_err(y, ref) <= TOL, (p, oracle.rel_err(y, ref))
        for br in range(w.shape[0] // 16):
            sl = slice(16 * br, 16 * br + 16)
            assert oracle.rel_err(y[:, sl], ref[:, sl]) <= TOL, (p, br)


@pytest.mark.parametrize("tokens", [5, 17, 64])
def test_rowk_fewer_bricks_than_waves(env, tokens):
    """2 bricks along K and 3 brick-rows: most waves of a whole-K workgroup
    own no brick, and the last workgroup has absent brick-rows."""
    torch, uw = env
    w = synth.weights(48, 128, 9, 0.02, 10)
    x = synth.activations(tokens, 128, xseed=5)
    ref = oracle.matmul_fp64(x, w)
    m = _both(env, w)
    names = uw.variants(tokens)
    picked = [v for v, n in enumerate(names) if n.startswith("rowk")]
    assert picked
    for v in picked:
        for p in (2, 4):
            y = _run(env, m, x, p, variant=v)
            assert oracle.rel_err(y, ref) <= TOL, (names[v], p, oracle.rel_err(y, ref))


@pytest.mark.parametrize("tokens", [1, 3, 16])
def test_gemv_odd_brick_count_and_short_waves(env, tokens):
    """The LDS-activation GEMV on 27 bricks along K (an odd count: the
    per-brick table copy is whole 4-byte pieces) and 34 brick-rows, every
    gemv variant (8 or 16 waves: some waves own 1 or 2 bricks, fewer than the
    bricks in flight), direct palette and runtime transcode, against fp64."""
    torch, uw = env
    w = synth.weights(544, 1728, 5, 0.003, 11)
    x = synth.activations(tokens, 1728, xseed=9)
    ref = oracle.matmul_fp64(x, w)
    m = _both(env, w)
    names = uw.variants(tokens)
    picked = [v for v, n in enumerate(names) if n.startswith("gemv")]
    assert picked
    for v in picked:
        for p in (3, 4):
            y = _run(env, m, x, p, variant=v)
            assert oracle.rel_err(y, ref) <= TOL, (names[v], p, oracle.rel_err(y, ref))


def _raw_heavy_weights():
    """4 brick-rows x 4096 columns (1024 groups of 64 per brick-row) with raw
    groups forced by one exponent outside the palette per group (exponents
    20..107 spread so that none enters the palette 108..123): brick-row 0 holds 257 raw
    groups, 1 all 1024, 2 none added, 3 exactly 256 (16 whole bricks)."""
    w = synth.weights(64, 4096, 31, 0.0, 12).copy()
    e = np.clip((w >> 7) & 0xFF, 108, 123)  # every exponent in one 16-value palette: no other raw group
    w = ((w & 0x807F) | (e << 7)).astype(np.uint16)

    def force_raw(row, col, k):
        e = 20 + k % 88
        w[row, col] = (w[row, col] & 0x807F) | (e << 7)

    k = 0
    for g in range(257):  # brick-row 0: bricks 0..16, rows 0..15 (257 = 16 * 16 + 1)
        kb, r = divmod(g, 16)
        force_raw(r, kb * 64 + 5, k); k += 1
    for r in range(16):
        for kb in range(64):
            force_raw(16 + r, kb * 64 + (r * 7 + kb) % 64, k); k += 1
    for r in range(16):
        for kb in range(16):
            force_raw(48 + r, kb * 64 + 63, k); k += 1
    return w


@pytest.mark.parametrize("tokens", [1, 3, 16])
def test_gemv_raw_heavy_brick_rows(env, tokens):
    """The LDS-held activations kernel copies each brick-row's raw-group bytes
    into LDS when no brick-row has more than 256 raw groups (brick-rows 2-3:
    0 and exactly 256), and reads them from global memory otherwise (all four
    brick-rows: 257 and 1024 as well); every gemv variant, direct palette and
    runtime transcode, against fp64 per brick-row."""
    torch, uw = env
    w_all = _raw_heavy_weights()
    x = synth.activations(tokens, 4096, xseed=7)
    names = uw.variants(tokens)
    picked = [v for v, n in enumerate(names) if n.startswith("gemv")]
    assert len(picked) >= 6
    for w, raw in ((w_all, 257 + 1024 + 256), (np.ascontiguousarray(w_all[32:]), 256)):
        m = _both(env, w)
        assert m.info()["raw_groups"] == raw
        ref = oracle.matmul_fp64(x, w)
        for v in picked:
            for p in (3, 4):
                y = _run(env, m, x, p, variant=v)
                assert oracle.rel_err(y, ref) <= TOL, (names[v], p, oracle.rel_err(y, ref))
                # per brick-row as well, so that a wrong group in one
                # brick-row cannot hide behind the magnitude of another
                for br in range(w.shape[0] // 16):
                    sl = slice(16 * br, 16 * br + 16)
                    assert oracle.rel_err(y[:, sl], ref[:, sl]) <= TOL, (names[v], p, br)


@pytest.mark.parametrize("rows,cols", [(1024, 4096), (3584, 18944), (128256, 4096)])
def test_other_projection_shapes(env, rows, cols):
    """Attention k/v (1024 x 4096), a wider MLP's down projection
    (3584 x 18944) and the vocabulary projection (128256 x 4096): direct
    palette with the built-in kernel choice, sampled rows against fp64."""
    torch, uw = env
    w = synth.weights(rows, cols, 21, 0.0005, 10)
    m = uw.Matrix(w, uw.FMT_PALETTE)
    sample = np.random.default_rng(1).choice(rows, min(rows, 384), replace=False)
    for tokens in ((1, 16, 64, 100) if rows * cols < (1 << 28) else (1, 16)):
        print(f"shape {rows}x{cols} tokens {tokens}", flush=True)
        x = synth.activations(tokens, cols, xseed=tokens)
        y = _run(env, m, x, uw.P4_DIRECT_PALETTE)
        assert not np.isnan(y).any()
        ref = oracle.matmul_fp64_rows(x, w, sample)
        assert oracle.rel_err(y[:, sample], ref) <= TOL, (rows, cols, tokens)


def test_gate_full_size_batch1(env):
    """14336x4096 gate, batch 1 (the headline workload): full decode bit-exact,
    resident codes bit-exact, sampled outputs of all pipelines vs fp64."""
    torch, uw = env
    c = synth.CONFIGS["gate_8b"]
    w = synth.weights(c["rows"], c["cols"], c["seed"], c["p"], c["shift"])
    m = _both(env, w)
    out = torch.empty(w.shape, dtype=torch.int16, device="cuda")
    m.decode(out)
    torch.cuda.synchronize()
    assert np.array_equal(uw.bits_of(out), w)
    del out
    x = synth.activations(1, c["cols"], xseed=c["xseed"])
    rows = np.random.default_rng(0).choice(c["rows"], 512, replace=False)
    ref = oracle.matmul_fp64_rows(x, w, rows)
    ys = {}
    for p in (1, 2, 3, 4, 5):
        ys[p] = _run(env, m, x, p)
        assert oracle.rel_err(ys[p][:, rows], ref) <= TOL, p
    for p in (1, 2, 3, 5):
        assert oracle.rel_err(ys[p], ys[4]) <= TOL, p


@pytest.mark.parametrize("proj", ["gate", "up", "down"])
def test_mlp_8b_shapes_every_row(env, proj):
    """8B-shaped projections at 1-1024 tokens, every pipeline with its built-in
    kernel choice: every output element against fp64 (all 896 brick-rows of
    gate/up, so every workgroup's output is compared)."""
    torch, uw = env
    c = synth.CONFIGS["mlp_8b"]
    rows, cols, seed = c[proj]
    w = synth.weights(rows, cols, seed, c["p"], c["shift"])
    m = _both(env, w)
    wt = oracle.bf16_to_f64(w).T.copy()
    xs = synth.activations(1024, cols, xseed=1)
    for tokens in (1, 16, 64, 256, 1024):
        x = xs[:tokens]
        ref = oracle.bf16_to_f64(x) @ wt
        for p in (1, 2, 3, 4, 5):
            print(f"{proj} {rows}x{cols} tokens {tokens} pipeline {p}", flush=True)
            y = _run(env, m, x, p)
            assert oracle.rel_err(y, ref) <= TOL, (tokens, p, oracle.rel_err(y, ref))


@pytest.mark.parametrize("rows,cols", [(28672, 8192), (8192, 28672)])
def test_70b_shapes_every_row(env, rows, cols):
    """70B-shaped gate/up (28672 x 8192) and down (8192 x 28672) projections at
    1, 256 and 1024 tokens -- the shapes and batches the layer stack runs: the
    direct palette and the hard layers' pipelines (runtime transcode, full
    decode) with the built-in kernel choice (at 256 tokens the down projection
    runs the whole-K kernel over 448 bricks; at 1024 the gate runs the wide
    tile in two rounds of 224 workgroups), every output element against fp64."""
    torch, uw = env
    c = synth.CONFIGS["stack_70b"]
    w = synth.weights(rows, cols, c["seed_base"] + (2 if rows < cols else 0), c["p"], c["shift"])
    m = _both(env, w)
    wt = oracle.bf16_to_f64(w).T.copy()
    del w
    xs = synth.activations(1024, cols, xseed=1)
    for tokens in (1, 256, 1024):
        x = xs[:tokens]
        ref = oracle.bf16_to_f64(x) @ wt
        for p in (4, 3, 1):
            print(f"{rows}x{cols} tokens {tokens} pipeline {p} ({m.variant_in_use(tokens, p)[1]})", flush=True)
            y = _run(env, m, x, p)
            assert oracle.rel_err(y, ref) <= TOL, (tokens, p, oracle.rel_err(y, ref))


# the other SwiGLU projection shapes the bench sweeps (seed 100 + index, as there)
OTHER_SWIGLU = [(0, 18944, 3584), (1, 3584, 18944), (2, 14336, 5120), (3, 5120, 14336), (4, 8192, 3072),
                (5, 3072, 8192)]


@pytest.mark.parametrize("idx,rows,cols", OTHER_SWIGLU)
def test_other_swiglu_shapes_every_row(env, idx, rows, cols):
    """Qwen2.5-7B-, Mistral-NeMo-12B- and Llama-3.2-3B-sized gate/up and down
    projections (synthetic weights of the 8B recipe) at 1-1024 tokens with the
    built-in kernel choice: direct palette and runtime transcode at every
    batch, full decode, exponent decode and the palette full decode at 1 and
    256 tokens; every output element against fp64."""
    torch, uw = env
    c = synth.CONFIGS["mlp_8b"]
    w = synth.weights(rows, cols, 100 + idx, c["p"], c["shift"])
    m = _both(env, w)
    wt = oracle.bf16_to_f64(w).T.copy()
    del w
    xs = synth.activations(1024, cols, xseed=1)
    for tokens in (1, 16, 64, 256, 1024):
        x = xs[:tokens]
        ref = oracle.bf16_to_f64(x) @ wt
        for p in ((4, 3, 1, 2, 5) if tokens in (1, 256) else (4, 3)):
            print(f"{rows}x{cols} tokens {tokens} pipeline {p} ({m.variant_in_use(tokens, p)[1]})", flush=True)
            y = _run(env, m, x, p)
            assert oracle.rel_err(y, ref) <= TOL, (tokens, p, oracle.rel_err(y, ref))


@pytest.mark.parametrize("pipes", [(4, 4, 4), (3, 2, 1), (5, 5, 5)])
def test_mlp_layer_8b_shapes(env, pipes):
    """The whole 8B-shaped SwiGLU layer through uw_mlp_forward (gate, up,
    silu*mul to bf16, down) against the fp64 layer, at 1, 64 and 256 tokens."""
    torch, uw = env
    c = synth.CONFIGS["mlp_8b"]
    ws = [synth.weights(*c[p][:2], c[p][2], c["p"], c["shift"]) for p in ("gate", "up", "down")]
    mats = [_both(env, w) for w in ws]
    hidden, inter = ws[0].shape[1], ws[0].shape[0]
    xs = synth.activations(256, hidden, xseed=2)
    work = torch.empty(uw.mlp_workspace_bytes(256, inter), dtype=torch.uint8, device="cuda")
    for tokens in (1, 64, 256):
        print(f"8B layer {pipes} tokens {tokens}", flush=True)
        x = xs[:tokens]
        _, _, _, ref = oracle.mlp_layer_fp64(x, *ws)
        y = torch.empty((tokens, hidden), device="cuda", dtype=torch.float32)
        uw.mlp_forward(*mats, list(pipes), uw.bf16_tensor(x), y, tokens, work)
        torch.cuda.synchronize()
        assert oracle.rel_err(y.cpu().numpy(), ref) <= TOL, (tokens, oracle.rel_err(y.cpu().numpy(), ref))


@pytest.mark.parametrize("gu", [4, 3])
def test_mlp_forward_gate_up_one_launch(env, gu):
    """gate and up take the same gemv or whole-K variant (on the palette
    form, pipeline 4, or on codes decoded into scratch, pipeline 3), so
    uw_mlp_forward sends them out as one launch: the layer must equal, bit for
    bit, the same layer run as separate calls (gate, up, silu*mul, down), and
    the fp64 layer."""
    torch, uw = env
    hidden, inter = 1024, 2048  # 128 brick-rows: the gemv kernels are the default
    ws = [synth.weights(inter, hidden, 60, 0.002, 10), synth.weights(inter, hidden, 61, 0.002, 10),
          synth.weights(hidden, inter, 62, 0.002, 10)]
    mats = [_both(env, w) for w in ws]
    # the down projection (64 brick-rows) would split K with atomic sums by
    # default; variant 1 does not, so both runs add in one order
    mats[2].set_variant(1)
    work = torch.empty(uw.mlp_workspace_bytes(64, inter), dtype=torch.uint8, device="cuda")
    for tokens in (1, 5, 16, 24, 64):
        kind = mats[0].variant_in_use(tokens, gu)[1]
        print(f"gate+up one launch, pipeline {gu}, tokens {tokens}, {kind}", flush=True)
        assert kind.startswith("gemv" if tokens <= 16 else "rowk:r4p4u2d2"), kind
        x = synth.activations(tokens, hidden, xseed=30 + tokens)
        xd = uw.bf16_tensor(x)
        y = torch.empty((tokens, hidden), device="cuda", dtype=torch.float32)
        uw.mlp_forward(*mats, [gu, gu, 4], xd, y, tokens, work)
        g = torch.empty((tokens, inter), device="cuda", dtype=torch.float32)
        u = torch.empty_like(g)
        h = torch.empty((tokens, inter), device="cuda", dtype=torch.int16)
        y2 = torch.empty_like(y)
        mats[0].matmul(xd, g, tokens, gu)
        mats[1].matmul(xd, u, tokens, gu)
        uw.silu_mul(g, u, h)
        mats[2].matmul(h, y2, tokens, 4)
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy(), y2.cpu().numpy()), tokens
        _, _, _, ref = oracle.mlp_layer_fp64(x, *ws)
        assert oracle.rel_err(y.cpu().numpy(), ref) <= TOL, tokens


def test_mlp_forward_shared_scratch_pipeline3(env):
    """gate and up decoded into one shared scratch buffer (pipeline 3): the
    layer must not send their products out as one launch (up's decode would
    overwrite gate's codes first); it runs them one after the other and still
    matches the fp64 layer and the separate calls bit for bit."""
    torch, uw = env
    hidden, inter, tokens = 1024, 2048, 1
    ws = [synth.weights(inter, hidden, 80, 0.002, 10), synth.weights(inter, hidden, 81, 0.002, 10),
          synth.weights(hidden, inter, 82, 0.002, 10)]
    mats = [_both(env, w) for w in ws]
    mats[2].set_variant(1)  # no K split in the down projection: one summation order
    shared = torch.empty(mats[0].info()["scratch_bytes"][3], dtype=torch.uint8, device="cuda")
    mats[0].set_scratch(shared)
    mats[1].set_scratch(shared)
    x = synth.activations(tokens, hidden, xseed=40)
    xd = uw.bf16_tensor(x)
    work = torch.empty(uw.mlp_workspace_bytes(tokens, inter), dtype=torch.uint8, device="cuda")
    y = torch.empty((tokens, hidden), device="cuda", dtype=torch.float32)
    print("shared scratch, pipeline 3 gate/up", flush=True)
    uw.mlp_forward(*mats, [3, 3, 4], xd, y, tokens, work)
    g = torch.empty((tokens, inter), device="cuda", dtype=torch.float32)
    u = torch.empty_like(g)
    h = torch.empty((tokens, inter), device="cuda", dtype=torch.int16)
    y2 = torch.empty_like(y)
    mats[0].matmul(xd, g, tokens, 3)
    mats[1].matmul(xd, u, tokens, 3)
    uw.silu_mul(g, u, h)
    mats[2].matmul(h, y2, tokens, 4)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy(), y2.cpu().numpy())
    _, _, _, ref = oracle.mlp_layer_fp64(x, *ws)
    assert oracle.rel_err(y.cpu().numpy(), ref) <= TOL


@pytest.mark.parametrize("pipes", [[5, 5, 5], [3, 3, 3], [1, 2, 3]])
def test_mlp_forward_side_stream_decodes(env, pipes):
    """With a side stream on the handles, uw_mlp_forward decodes up and down
    there while gate's product runs: the layer must equal, bit for bit, the
    same layer on one stream, and the fp64 layer."""
    torch, uw = env
    hidden, inter, tokens = 1024, 2048, 7
    ws = [synth.weights(inter, hidden, 90, 0.002, 10), synth.weights(inter, hidden, 91, 0.002, 10),
          synth.weights(hidden, inter, 92, 0.002, 10)]
    mats = [_both(env, w) for w in ws]
    mats[2].set_variant(1)  # no K split in the down projection: one summation order
    x = synth.activations(tokens, hidden, xseed=50)
    xd = uw.bf16_tensor(x)
    work = torch.empty(uw.mlp_workspace_bytes(tokens, inter), dtype=torch.uint8, device="cuda")
    main, side = torch.cuda.current_stream(), torch.cuda.Stream()
    outs = []
    for s2 in (main, side):
        for m in mats:
            m.set_streams(main, s2)
        y = torch.empty((tokens, hidden), device="cuda", dtype=torch.float32)
        print(f"layer {pipes}, side stream {s2 is side}", flush=True)
        uw.mlp_forward(*mats, pipes, xd, y, tokens, work)
        torch.cuda.synchronize()
        outs.append(y.cpu().numpy())
    assert np.array_equal(outs[0], outs[1])
    _, _, _, ref = oracle.mlp_layer_fp64(x, *ws)
    assert oracle.rel_err(outs[1], ref) <= TOL


def test_silu_mul(env):
    torch, uw = env
    rng = np.random.default_rng(4)
    g = (rng.standard_normal(10003) * 3).astype(np.float32)
    u = rng.standard_normal(10003).astype(np.float32)
    gd, ud = torch.from_numpy(g).cuda(), torch.from_numpy(u).cuda()
    h = torch.empty(10003, dtype=torch.int16, device="cuda")
    uw.silu_mul(gd, ud, h)
    torch.cuda.synchronize()
    got = oracle.bf16_to_f64(uw.bits_of(h))
    want = oracle.bf16_to_f64(oracle.silu_mul_bf16(g.astype(np.float64), u.astype(np.float64)))
    assert np.all(np.abs(got - want) <= np.abs(want) * 2.0 ** -7 + 1e-30)


def test_mlp_layer_and_stack(env):
    """The SwiGLU layer at the matmul tolerance, and a 4-layer stack of
    alternating hard and easy layers checked layer by layer: layer l's output
    against the fp64 layer fed the same bf16 input the GPU fed it (the bf16
    rounding of layer l-1's GPU output), so each layer meets the tolerance on
    its own; the side-stream overlap must not change a bit."""
    torch, uw = env
    hidden, inter, tokens = 256, 512, 9
    ws = [synth.weights(inter, hidden, 20, 0.002, 10), synth.weights(inter, hidden, 21, 0.002, 10),
          synth.weights(hidden, inter, 22, 0.002, 10)]
    x = synth.activations(tokens, hidden, xseed=5)
    _, _, _, ref = oracle.mlp_layer_fp64(x, *ws)
    mats = [_both(env, w) for w in ws]
    xd = uw.bf16_tensor(x)
    y = torch.empty((tokens, hidden), device="cuda", dtype=torch.float32)
    work = torch.empty(uw.mlp_workspace_bytes(tokens, inter), dtype=torch.uint8, device="cuda")
    for pipes in ([4, 4, 4], [1, 2, 3], [3, 3, 2], [5, 4, 5]):
        uw.mlp_forward(*mats, pipes, xd, y, tokens, work)
        torch.cuda.synchronize()
        assert oracle.rel_err(y.cpu().numpy(), ref) <= TOL, pipes
    # a 4-layer stack, alternating hard (Huffman) and easy (palette) layers
    L = 4
    # std 0.05 and no outliers keep activations of an un-normalised stack in range
    layer_w = [[synth.weights(inter, hidden, 100 + 3 * l, 0.0, 0, std=0.05),
                synth.weights(inter, hidden, 101 + 3 * l, 0.0, 0, std=0.05),
                synth.weights(hidden, inter, 102 + 3 * l, 0.0, 0, std=0.05)] for l in range(L)]
    side = torch.cuda.Stream()
    stack = []
    pipes = []
    scratch = [[torch.empty(2 * inter * hidden, dtype=torch.uint8, device="cuda") for _ in range(3)] for _ in range(2)]
    for l in range(L):
        for j in range(3):
            m = _both(env, layer_w[l][j])
            m.set_streams(torch.cuda.current_stream(), side)
            m.set_scratch(scratch[l % 2][j])
            m.set_variant(1)  # K not split across workgroups: no atomics, runs are bit-reproducible
            stack.append(m)
            pipes.append((3, 4, 5, 4)[l % 4])  # hard layers: runtime transcode, palette full decode
    work = torch.empty(uw.stack_workspace_bytes(tokens, hidden, inter), dtype=torch.uint8, device="cuda")
    # layer l's GPU output: the last output of the stack's first l+1 layers
    ys = []
    for l in range(L):
        yl = torch.empty((tokens, hidden), device="cuda", dtype=torch.float32)
        uw.stack_forward(stack[:3 * (l + 1)], pipes[:3 * (l + 1)], xd, yl, tokens, work, overlap=True)
        torch.cuda.synchronize()
        ys.append(yl.cpu().numpy())
    xin = x
    for l in range(L):
        _, _, _, ref_l = oracle.mlp_layer_fp64(xin, *layer_w[l])
        assert oracle.rel_err(ys[l], ref_l) <= TOL, (l, oracle.rel_err(ys[l], ref_l))
        xin = oracle.f64_to_bf16_rne(ys[l].astype(np.float64))  # what the GPU feeds layer l+1
    outs = []
    for overlap in (False, True, True):
        yo = torch.empty((tokens, hidden), device="cuda", dtype=torch.float32)
        uw.stack_forward(stack, pipes, xd, yo, tokens, work, overlap=overlap)
        torch.cuda.synchronize()
        outs.append(yo.cpu().numpy())
    # overlapped side-stream decode must not change a single bit
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[1], outs[2])
    assert np.array_equal(outs[0], ys[-1])


def test_gemm_baseline_and_copy(env):
    torch, uw = env
    w = synth.weights(512, 1024, 7, 0.0, 0)
    x = synth.activations(37, 1024, xseed=2)
    y = torch.empty((37, 512), device="cuda", dtype=torch.float32)
    uw.gemm_bf16(uw.bf16_tensor(x), uw.bf16_tensor(w), y, 37, 512, 1024)
    torch.cuda.synchronize()
    assert oracle.rel_err(y.cpu().numpy(), oracle.matmul_fp64(x, w)) <= TOL
    src = torch.arange(1 << 20, dtype=torch.int32, device="cuda")
    dst = torch.zeros_like(src)
    uw.device_copy(src, dst, src.numel() * 4)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


def test_device_error_paths(env):
    torch, uw = env
    w = synth.weights(32, 128, 1, 0.0, 0)
    x = uw.bf16_tensor(synth.activations(2, 128))
    y = torch.empty((2, 32), device="cuda", dtype=torch.float32)
    mh = uw.Matrix(w, uw.FMT_HUFFMAN)
    with pytest.raises(uw.UwError) as e:
        mh.matmul(x, y, pipeline=uw.P4_DIRECT_PALETTE)
    assert e.value.status == uw.ERR_UNSUPPORTED
    with pytest.raises(uw.UwError) as e:
        mh.matmul(x, y, pipeline=uw.P3_PALETTE_TRANSCODE)
    assert e.value.status == uw.ERR_UNSUPPORTED
    with pytest.raises(uw.UwError) as e:
        mh.matmul(x, y, pipeline=uw.P5_PALETTE_DECODE)
    assert e.value.status == uw.ERR_UNSUPPORTED
    with pytest.raises(uw.UwError) as e:
        mh.preprocess(uw.P5_PALETTE_DECODE)
    assert e.value.status == uw.ERR_UNSUPPORTED
    with pytest.raises(uw.UwError) as e:
        mh.matmul(x, y, tokens=0)
    assert e.value.status == uw.ERR_INVALID_ARG
    mp = uw.Matrix(w, uw.FMT_PALETTE)
    with pytest.raises(uw.UwError) as e:
        mp.preprocess(uw.P1_FULL_DECODE)
    assert e.value.status == uw.ERR_UNSUPPORTED
    with pytest.raises(uw.UwError) as e:
        mp.preprocess(uw.P4_DIRECT_PALETTE)
    assert e.value.status == uw.ERR_UNSUPPORTED
    with pytest.raises(uw.UwError) as e:
        mh.set_scratch(torch.empty(16, dtype=torch.uint8, device="cuda"))
        mh.matmul(x, y, pipeline=uw.P1_FULL_DECODE)
    assert e.value.status == uw.ERR_INVALID_ARG
    # auto pipeline with a plan
    mb = uw.Matrix(w, uw.FMT_HUFFMAN | uw.FMT_PALETTE)
    mb.set_plan([(1, 1, 0), (64, 4, 0), (1 << 20, 2, 0)])
    for t in (1, 2, 70):
        xt = uw.bf16_tensor(synth.activations(t, 128))
        yt = torch.empty((t, 32), device="cuda", dtype=torch.float32)
        mb.matmul(xt, yt)
        torch.cuda.synchronize()
        assert oracle.rel_err(yt.cpu().numpy(), oracle.matmul_fp64(synth.activations(t, 128), w)) <= TOL


def test_cu_masked_streams(env):
    torch, uw = env
    n = uw.device_cu_count()
    assert n >= 8
    s1 = uw.stream_create(0, n // 4)
    s2 = uw.stream_create(n // 4, n - n // 4)
    w = synth.weights(64, 256, 9, 0.002, 12)
    x = synth.activations(4, 256)
    m = _both(env, w)
    m.set_streams(s2, s1)
    xd = uw.bf16_tensor(x)
    y = torch.empty((4, 64), device="cuda", dtype=torch.float32)
    m.preprocess(3)
    m.matmul(xd, y, pipeline=3)
    torch.cuda.synchronize()
    assert oracle.rel_err(y.cpu().numpy(), oracle.matmul_fp64(x, w)) <= TOL
    m.free()
    uw.stream_destroy(s1)
    uw.stream_destroy(s2)
