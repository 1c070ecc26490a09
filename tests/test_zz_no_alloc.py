"""The allocation-free SwiGLU layer (uw_mlp_forward_noalloc), through the C
ABI, against uw_mlp_forward with a caller-provided workspace: two calls in a
row on 8B-shaped projections, the second with fewer tokens (the fixed device
array keeps the first call's contents), each within the matmul tolerance of
the workspace entry point; the device's free memory does not change across
either call."""
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


def test_noalloc_layer_matches_workspace_layer(env):
    torch, uw = env
    c = synth.CONFIGS["mlp_8b"]
    ws = [synth.weights(*c[p][:2], c[p][2], c["p"], c["shift"]) for p in ("gate", "up", "down")]
    mats = [uw.Matrix(w, uw.FMT_PALETTE) for w in ws]
    hidden, inter = ws[0].shape[1], ws[0].shape[0]
    xs = synth.activations(64, hidden, xseed=3)
    pipes = [uw.P4_DIRECT_PALETTE] * 3
    first = 64
    xd = uw.bf16_tensor(xs)
    work = torch.empty(uw.mlp_workspace_bytes(first, inter), dtype=torch.uint8, device="cuda")
    outs = {t: (torch.full((t, hidden), float("nan"), device="cuda"), torch.full((t, hidden), float("nan"), device="cuda"))
            for t in (first, 5)}
    # a first call of the entry point on this device: the HIP runtime places
    # the fixed array when it loads the library's code object, and the entry
    # point looks up the array's device address once
    y1 = torch.empty((1, hidden), device="cuda")
    uw.mlp_forward_noalloc(*mats, pipes, xd, y1, 1)
    torch.cuda.synchronize()
    for tokens in (first, 5):  # the second call is smaller than the first
        print(f"noalloc layer, {tokens} tokens", flush=True)
        y_ws, y_na = outs[tokens]
        # the workspace entry point first: it also loads the code objects of
        # the kernels this token count runs
        uw.mlp_forward(*mats, pipes, xd, y_ws, tokens, work)
        torch.cuda.synchronize()
        free_before = torch.cuda.mem_get_info()[0]
        uw.mlp_forward_noalloc(*mats, pipes, xd, y_na, tokens)
        torch.cuda.synchronize()
        assert torch.cuda.mem_get_info()[0] == free_before, tokens
        a, b = y_ws.cpu().numpy(), y_na.cpu().numpy()
        assert np.isfinite(b).all(), tokens
        assert oracle.rel_err(b, a) <= TOL, (tokens, oracle.rel_err(b, a))


def test_noalloc_layer_rejections(env):
    torch, uw = env
    hidden, inter = 256, 512
    ws = [synth.weights(inter, hidden, 20, 0.002, 10), synth.weights(inter, hidden, 21, 0.002, 10),
          synth.weights(hidden, inter, 22, 0.002, 10)]
    mats = [uw.Matrix(w, uw.FMT_HUFFMAN | uw.FMT_PALETTE) for w in ws]
    x = uw.bf16_tensor(synth.activations(4, hidden, xseed=5))
    y = torch.empty((4, hidden), device="cuda", dtype=torch.float32)
    # a projection whose pipeline needs preprocessing scratch
    with pytest.raises(uw.UwError) as e:
        uw.mlp_forward_noalloc(*mats, [4, 3, 4], x, y, 4)
    assert e.value.status == uw.ERR_UNSUPPORTED
    # more tokens than the fixed array holds (checked before any launch)
    too_many = uw.STATIC_WORKSPACE_BYTES // (10 * inter) + 1
    assert uw.mlp_workspace_bytes(too_many, inter) > uw.STATIC_WORKSPACE_BYTES
    with pytest.raises(uw.UwError) as e:
        uw.mlp_forward_noalloc(*mats, [4, 4, 4], x, y, too_many)
    assert e.value.status == uw.ERR_SHAPE
    # and a small layer against the fp64 oracle
    uw.mlp_forward_noalloc(*mats, [4, 4, 4], x, y, 4)
    torch.cuda.synchronize()
    _, _, _, ref = oracle.mlp_layer_fp64(synth.activations(4, hidden, xseed=5), *ws)
    assert oracle.rel_err(y.cpu().numpy(), ref) <= TOL
