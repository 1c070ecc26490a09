"""GPU tests of the autotuner and the CU-split search (Unweight page, section 九).

The tuner's output is a plan; what must hold is that the plan is well formed,
that installing it changes nothing in the results (every pipeline computes the
same product), and that the layer it was tuned on still matches the oracle.
"""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    assert torch.cuda.is_available()
    import decode_gemm_bf16_amd as uw
    from decode_gemm_bf16_amd import tune
    return torch, uw, tune


def test_tune_mlp_plan_and_parity(env):
    torch, uw, tune = env
    hidden, inter = 256, 512
    ws = {"gate": synth.weights(inter, hidden, 30, 0.002, 10), "up": synth.weights(inter, hidden, 31, 0.002, 10),
          "down": synth.weights(hidden, inter, 32, 0.002, 10)}
    stream = torch.cuda.Stream()
    layer = {}
    for proj, w in ws.items():
        m = uw.Matrix(w, uw.FMT_HUFFMAN | uw.FMT_PALETTE)
        layer[proj] = [m, m.clone()]
        for mm in layer[proj]:
            mm.set_streams(stream)
    plan = tune.tune_mlp(torch, layer, [1, 70], stream, steps=3, keep=2, log=lambda s: None)
    assert set(plan["batches"]) == {"1", "70"}
    for t, e in plan["batches"].items():
        for proj in ("gate", "up", "down"):
            p, v = e[proj]
            assert 1 <= p <= 4 and 0 <= v < len(uw.variants(int(t)))
        assert e["layer_us"] > 0
    tune.apply_plan(plan, layer)
    for tokens in (1, 5, 70, 100):
        x = synth.activations(tokens, hidden, xseed=tokens)
        _, _, _, ref = oracle.mlp_layer_fp64(x, ws["gate"], ws["up"], ws["down"])
        y = torch.empty((tokens, hidden), device="cuda", dtype=torch.float32)
        work = torch.empty(uw.mlp_workspace_bytes(tokens, inter), dtype=torch.uint8, device="cuda")
        with torch.cuda.stream(stream):
            uw.mlp_forward(layer["gate"][1], layer["up"][1], layer["down"][1], [0, 0, 0], uw.bf16_tensor(x), y,
                           tokens, work)
        torch.cuda.synchronize()
        assert oracle.rel_err(y.cpu().numpy(), ref) <= 1e-3, tokens


def test_tune_split_stack(env):
    torch, uw, tune = env
    hidden, inter, tokens, L = 256, 512, 4, 4
    ws = [[synth.weights(inter, hidden, 200 + 3 * l, 0.0, 0, std=0.05),
           synth.weights(inter, hidden, 201 + 3 * l, 0.0, 0, std=0.05),
           synth.weights(hidden, inter, 202 + 3 * l, 0.0, 0, std=0.05)] for l in range(L)]
    stack, pipes = [], []
    for l in range(L):
        for j in range(3):
            hard = l % 2 == 0
            m = uw.Matrix(ws[l][j], (uw.FMT_HUFFMAN | uw.FMT_RAWAUX) if hard else uw.FMT_PALETTE)
            stack.append(m)
            pipes.append(3 if hard else 4)
    x = synth.activations(tokens, hidden, xseed=9)
    res = tune.tune_split(torch, stack, pipes, uw.bf16_tensor(x), tokens, [0, 32, 128], steps=2, log=lambda s: None)
    assert sorted(n for _, n in res) == [0, 32, 128]
    assert all(ms > 0 for ms, _ in res)
    # after the search the handles are back on the null stream; each layer of
    # the stack still matches the fp64 layer fed the bf16 input the GPU fed it
    work = torch.empty(uw.stack_workspace_bytes(tokens, hidden, inter), dtype=torch.uint8, device="cuda")
    xin = x
    for l in range(L):
        y = torch.empty((tokens, hidden), device="cuda", dtype=torch.float32)
        uw.stack_forward(stack[:3 * (l + 1)], pipes[:3 * (l + 1)], uw.bf16_tensor(x), y, tokens, work, overlap=True)
        torch.cuda.synchronize()
        yl = y.cpu().numpy()
        _, _, _, ref = oracle.mlp_layer_fp64(xin, *ws[l])
        assert oracle.rel_err(yl, ref) <= 1e-3, (l, oracle.rel_err(yl, ref))
        xin = oracle.f64_to_bf16_rne(yl.astype(np.float64))
