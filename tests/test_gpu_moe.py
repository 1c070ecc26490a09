"""Cold experts (Unweight page, section 十一): compressed experts kept on the
host, uploaded on demand, evicted and uploaded again, and the grouped matmul
over experts -- against the fp64 oracle per expert."""
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


def test_upload_evict_reupload(env):
    torch, uw = env
    w = synth.weights(272, 576, 31, 0.003, 11)
    m = uw.Matrix(w, uw.FMT_HUFFMAN | uw.FMT_PALETTE | uw.ENC_HOST_ONLY)
    host_nib = m.export(uw.STREAM_NIBBLES)
    m.upload()
    assert m.info()["resident_bytes"] > 0
    assert np.array_equal(m.export(uw.STREAM_NIBBLES), host_nib)  # read back from the device
    x = uw.bf16_tensor(synth.activations(5, 576, xseed=2))
    outs = []
    for rep in range(2):
        ys = {}
        for p in (2, 3, 4):
            y = torch.full((5, 272), float("nan"), device="cuda", dtype=torch.float32)
            m.matmul(x, y, pipeline=p)
            torch.cuda.synchronize()
            ys[p] = y.cpu().numpy()
            assert oracle.rel_err(ys[p], oracle.matmul_fp64(synth.activations(5, 576, xseed=2), w)) <= TOL, p
        outs.append(ys)
        m.evict()
        with pytest.raises(uw.UwError) as e:
            m.matmul(x, torch.empty((5, 272), device="cuda"), pipeline=4)
        assert e.value.status == uw.ERR_UNSUPPORTED
        m.upload()
    # the same streams give the same result up to the order of the K-split
    # workgroups' atomic additions (this 17-brick-row matrix splits K)
    for p in (2, 3, 4):
        assert oracle.rel_err(outs[0][p], outs[1][p]) <= 1e-6, p
    # a handle encoded on the device has no host copy to return to
    d = uw.Matrix(w, uw.FMT_PALETTE)
    with pytest.raises(uw.UwError) as e:
        d.evict()
    assert e.value.status == uw.ERR_UNSUPPORTED


@pytest.mark.parametrize("pipeline", [4, 3, 1])
def test_grouped_matmul(env, pipeline):
    torch, uw = env
    rows, cols, n = 528, 1024, 4
    ws = [synth.weights(rows, cols, 40 + e, 0.002, 12) for e in range(n)]
    experts = [uw.Matrix(w, uw.FMT_HUFFMAN | uw.FMT_PALETTE | uw.ENC_HOST_ONLY) for w in ws]
    for m in experts:
        m.upload()
    offs = [0, 3, 3, 70, 74]  # expert 1 gets no rows, expert 2 more than 64
    xb = synth.activations(offs[-1], cols, xseed=9)
    x = uw.bf16_tensor(xb)
    y = torch.full((offs[-1], rows), float("nan"), device="cuda", dtype=torch.float32)
    print(f"grouped matmul pipeline {pipeline}", flush=True)
    uw.grouped_matmul(experts, x, y, offs, pipeline)
    torch.cuda.synchronize()
    yh = y.cpu().numpy()
    for e in range(n):
        if offs[e + 1] == offs[e]:
            continue
        ref = oracle.matmul_fp64(xb[offs[e]:offs[e + 1]], ws[e])
        assert oracle.rel_err(yh[offs[e]:offs[e + 1]], ref) <= TOL, e


def test_grouped_gemv_launch(env):
    """More active experts than one grouped gemv launch holds, with short
    matrices (17 brick-rows, 9 bricks of K): the experts that fit the gemv
    kernels share launches, the one with 20 tokens runs alone.  Each expert is
    checked against fp64 and, bit for bit, against a single-matrix call forced
    to the same gemv variant (same kernel body, same summation order)."""
    torch, uw = env
    rows, cols, n = 272, 576, 22
    ws = [synth.weights(rows, cols, 300 + e, 0.003, 11) for e in range(n)]
    experts = [uw.Matrix(w, uw.FMT_PALETTE | uw.ENC_HOST_ONLY) for w in ws]
    for m in experts:
        m.upload()
    counts = [1, 2, 0, 1, 3, 1, 1, 16, 1, 0, 2, 1, 1, 1, 20, 1, 4, 1, 1, 2, 1, 1]
    assert len(counts) == n
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    xb = synth.activations(int(offs[-1]), cols, xseed=17)
    x = uw.bf16_tensor(xb)
    y = torch.full((int(offs[-1]), rows), float("nan"), device="cuda", dtype=torch.float32)
    print("grouped gemv: 22 experts", flush=True)
    uw.grouped_matmul(experts, x, y, offs, 4)
    torch.cuda.synchronize()
    yh = y.cpu().numpy()
    for e in range(n):
        a, b = int(offs[e]), int(offs[e + 1])
        if a == b:
            continue
        ref = oracle.matmul_fp64(xb[a:b], ws[e])
        assert oracle.rel_err(yh[a:b], ref) <= TOL, e
        if counts[e] > 16:
            continue
        names = uw.variants(counts[e])
        experts[e].set_variant(names.index("gemv:w8:d2"))
        ys = torch.full((b - a, rows), float("nan"), device="cuda", dtype=torch.float32)
        experts[e].matmul(x[a:b], ys, pipeline=4)
        torch.cuda.synchronize()
        experts[e].set_variant(0)
        assert np.array_equal(ys.cpu().numpy(), yh[a:b]), e
    for m in experts:
        m.free()
