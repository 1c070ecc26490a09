"""Autotuner: per projection and batch size, choose the pipeline and the fused
kernel variant by measurement (Unweight page, section 九).

The page's tuner measures end-to-end throughput on the target hardware,
sweeps the gate, up and down projections in turn and repeats until nothing
improves, and writes a per-model configuration (pipeline, kernel variant and
decode/compute split per projection and batch size).  Here:

1. each projection is first timed alone for every (pipeline, variant) pair and
   the few fastest pairs are kept as its candidates;
2. the SwiGLU layer (gate, up, silu*mul, down through ``uw_mlp_forward``) is
   then timed as a whole while the projections are optimised one at a time,
   gate -> up -> down, round after round, until a round gains less than 1%;
3. the decode/compute CU split of the side-stream layer pipeline is chosen by
   timing a short stack of alternating hard and easy layers (``tune_split``).

Timing: HIP graph replay of repeated calls on one stream, bracketed by HIP
events; weight copies at distinct addresses are rotated so that at least
1 GiB is touched between reuses and the 256 MB Infinity Cache cannot serve
them.  The plan is JSON: {"batches": {M: {"gate": [pipeline, variant], ...}}}.
"""
from __future__ import annotations

import json
import math
import sys
import time

from . import (FMT_HUFFMAN, FMT_PALETTE, Matrix, mlp_forward, mlp_workspace_bytes, variants,
               stack_forward, stack_workspace_bytes, stream_create, stream_destroy, device_cu_count, bf16_tensor,
               gemm_bf16, silu_mul)

PROJECTIONS = ("gate", "up", "down")


def time_graph(torch, fn, steps: int, warmup: int, stream, use_graph: bool = True, lead_in=None) -> float:
    """Average milliseconds per call of fn() on `stream`, from HIP events
    around `steps` calls replayed from a HIP graph (eager launches if capture
    is not possible).  With lead_in, an untimed run of the same steps and
    then lead_in() are enqueued just before the start event, without a host
    wait: the device is busy (and at the workload's clocks) while the host
    submits the timed graph, so neither the submission latency nor a clock
    ramp lands inside the timed region (both matter when `steps` is small);
    lead_in should evict the caches (a large read)."""
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            fn()
    torch.cuda.synchronize()
    graph = None
    if use_graph:
        try:
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=stream):
                for _ in range(steps):
                    fn()
            with torch.cuda.stream(stream):
                graph.replay()
            torch.cuda.synchronize()
        except Exception as e:  # noqa: BLE001 -- fall back to eager timing
            print(f"graph capture unavailable ({e}); timing eager launches", file=sys.stderr)
            graph = None
            torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        if lead_in is not None:
            # the same steps once more, untimed and without a host wait, so the
            # timed steps start at the clocks the workload runs at
            if graph is not None:
                graph.replay()
            else:
                for _ in range(steps):
                    fn()
            lead_in()
        start.record(stream)
        if graph is not None:
            graph.replay()
        else:
            for _ in range(steps):
                fn()
        end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def copies_for(mat: Matrix, min_bytes: int = 1 << 30) -> list[Matrix]:
    """mat plus enough device clones that cycling them touches >= min_bytes."""
    n = max(2, math.ceil(min_bytes / max(1, mat.info()["resident_bytes"])))
    return [mat] + [mat.clone() for _ in range(n - 1)]


def share_scratch(torch, mats: list[Matrix]):
    """Bind one scratch buffer, large enough for every pipeline, to all copies
    (so that no copy allocates lazily inside a captured graph).  Returns it."""
    need = max(m.info()["scratch_bytes"][1] for m in mats)
    buf = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    for m in mats:
        m.set_scratch(buf)
    return buf


def candidates(mat: Matrix) -> list[int]:
    p = []
    if mat.formats & FMT_HUFFMAN:
        p += [1, 2]
        if mat.formats & (FMT_PALETTE | 0x4):
            p.append(3)
    if mat.formats & FMT_PALETTE:
        p += [4, 5]
    return p


def time_projection(torch, mats, x, y, tokens: int, pipeline: int, variant: int, stream, steps=20) -> float:
    """Milliseconds per call of one projection, rotating copies."""
    for m in mats:
        m.set_variant(variant)
    i = [0]

    def fn():
        mats[i[0] % len(mats)].matmul(x, y, tokens, pipeline)
        i[0] += 1
    return time_graph(torch, fn, steps, 3, stream)


def effective_name(mat: Matrix, tokens: int, pipeline: int, variant: int) -> str:
    """The kernel that (pipeline, variant) launches for this shape (variants
    that do not apply fall back to their family's default; pipeline 1 is the
    library GEMM whatever the variant)."""
    mat.set_variant(variant)
    name = mat.variant_in_use(tokens, pipeline)[1]
    mat.set_variant(0)
    return name


def rank_projection(torch, mats, x, y, tokens: int, stream, keep: int = 4, steps: int = 20) -> list[tuple]:
    """All distinct (pipeline, kernel) choices of one projection, fastest
    first, as (ms, pipeline, variant id)."""
    res = []
    seen = set()
    for p in candidates(mats[0]):
        for v in range(len(variants(tokens))):
            key = (p, effective_name(mats[0], tokens, p, v))
            if key in seen:  # the same kernel under another id
                continue
            seen.add(key)
            ms = time_projection(torch, mats, x, y, tokens, p, v, stream, steps)
            res.append((ms, p, v))
    res.sort()
    for m in mats:
        m.set_variant(0)
    return res[:keep]


def tune_mlp(torch, layer: dict, tokens_list, stream, steps: int = 10, keep: int = 4, log=print) -> dict:
    """layer: {"gate": [copies], "up": [copies], "down": [copies]} (equal copy
    counts).  Returns the plan and the measured layer times."""
    gate0 = layer["gate"][0]
    inter, hidden = gate0.rows, gate0.cols
    ncopy = min(len(layer[p]) for p in PROJECTIONS)
    plan = {"batches": {}}
    max_t = max(tokens_list)
    xs = torch.randn(max_t, max(hidden, inter), device="cuda").to(torch.bfloat16)
    scratch = {proj: share_scratch(torch, layer[proj]) for proj in PROJECTIONS}  # noqa: F841 (kept alive)
    for tokens in tokens_list:
        t0 = time.perf_counter()
        x = xs[:tokens, :hidden].contiguous()
        # 1. per-projection candidates
        cands = {}
        for proj in PROJECTIONS:
            m0 = layer[proj][0]
            xp = xs[:tokens, :m0.cols].contiguous()
            yp = torch.empty((tokens, m0.rows), device="cuda", dtype=torch.float32)
            cands[proj] = [(p, v) for _, p, v in rank_projection(torch, layer[proj], xp, yp, tokens, stream, keep)]
        # 2. coordinate descent on the whole layer
        choice = {proj: cands[proj][0] for proj in PROJECTIONS}
        work = torch.empty(mlp_workspace_bytes(tokens, inter), dtype=torch.uint8, device="cuda")
        y = torch.empty((tokens, hidden), device="cuda", dtype=torch.float32)

        def layer_ms(ch):
            for proj in PROJECTIONS:
                for m in layer[proj]:
                    m.set_variant(ch[proj][1])
            pipes = [ch[p][0] for p in PROJECTIONS]
            i = [0]

            def fn():
                k = i[0] % ncopy
                mlp_forward(layer["gate"][k], layer["up"][k], layer["down"][k], pipes, x, y, tokens, work)
                i[0] += 1
            return time_graph(torch, fn, steps, 2, stream)

        best = layer_ms(choice)
        rounds = 0
        while True:
            rounds += 1
            start_best = best
            for proj in PROJECTIONS:
                for cand in cands[proj]:
                    if cand == choice[proj]:
                        continue
                    trial = dict(choice)
                    trial[proj] = cand
                    ms = layer_ms(trial)
                    if ms < best:
                        best, choice = ms, trial
            if best > start_best * 0.99 or rounds >= 4:
                break
        for proj in PROJECTIONS:
            for m in layer[proj]:
                m.set_variant(0)
        entry = {proj: list(choice[proj]) for proj in PROJECTIONS}
        entry["layer_us"] = round(best * 1e3, 2)
        entry["variant_names"] = {proj: effective_name(layer[proj][0], tokens, *choice[proj]) for proj in PROJECTIONS}
        entry["rounds"] = rounds
        plan["batches"][str(tokens)] = entry
        log(f"tokens {tokens}: {json.dumps(entry)} ({time.perf_counter() - t0:.1f} s)")
    return plan


def apply_plan(plan: dict, mats_by_proj: dict) -> None:
    """Install a tuned plan on matrices: {"gate": [Matrix...], ...}.  A batch
    size between two tuned sizes uses the next larger tuned entry."""
    sizes = sorted(int(t) for t in plan["batches"])
    for proj, mats in mats_by_proj.items():
        entries = []
        for i, t in enumerate(sizes):
            p, v = plan["batches"][str(t)][proj]
            bound = t if i + 1 < len(sizes) else (1 << 30)
            entries.append((bound, p, v))
        for m in mats:
            m.set_plan(entries)


def tune_split(torch, stack: list[Matrix], pipes: list[int], x, tokens: int, splits, steps: int = 3, log=print):
    """Time the layer stack with the side stream limited to `n` CUs (the rest
    to the main stream) for each n in splits (0 = no overlap, one stream).
    Returns [(ms, n)], fastest first."""
    ncu = device_cu_count()
    inter, hidden = stack[0].rows, stack[0].cols
    work = torch.empty(stack_workspace_bytes(tokens, hidden, inter), dtype=torch.uint8, device="cuda")
    y = torch.empty((tokens, hidden), device="cuda", dtype=torch.float32)
    out = []
    for n in splits:
        if n <= 0:
            main = torch.cuda.Stream()
            streams = []
            for m in stack:
                m.set_streams(main, main)
            overlap = False
            main_ptr = main
        else:
            s_side = stream_create(0, n)
            s_main = stream_create(n, ncu - n) if n < ncu else stream_create(0, ncu)
            streams = [s_side, s_main]
            for m in stack:
                m.set_streams(s_main, s_side)
            overlap = True
            main_ptr = torch.cuda.ExternalStream(s_main)
        fn = lambda: stack_forward(stack, pipes, x, y, tokens, work, overlap=overlap)  # noqa: E731
        with torch.cuda.stream(main_ptr):
            fn()
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(main_ptr):
            start.record()
            for _ in range(steps):
                fn()
            end.record()
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / steps
        out.append((ms, n))
        log(f"split side={n} CUs: {ms * 1e3:.1f} us per stack pass")
        for m in stack:
            m.set_streams(None, None)
        for s in streams:
            stream_destroy(s)
    out.sort()
    return out


def layer_baselines(torch, layer: dict, weights: dict, tokens_list, stream, steps: int = 10) -> dict:
    """Layer times (us) next to a tuned plan: the built-in choice on the
    palette form (pipeline 4 for all three projections, variant 0) and the
    uncompressed layer (hipBLASLt gate, up and down on bf16 copies, silu*mul
    between), both on rotated copies."""
    gate0 = layer["gate"][0]
    inter, hidden = gate0.rows, gate0.cols
    ncopy = min(len(layer[p]) for p in PROJECTIONS)
    nbf = max(2, math.ceil((1 << 30) / (2 * 3 * inter * hidden)))
    wd = [{p: bf16_tensor(weights[p]) for p in PROJECTIONS} for _ in range(nbf)]
    out = {}
    for tokens in tokens_list:
        x = torch.randn(tokens, hidden, device="cuda").to(torch.bfloat16)
        y = torch.empty((tokens, hidden), device="cuda", dtype=torch.float32)
        work = torch.empty(mlp_workspace_bytes(tokens, inter), dtype=torch.uint8, device="cuda")
        i = [0]

        def fused():
            k = i[0] % ncopy
            mlp_forward(layer["gate"][k], layer["up"][k], layer["down"][k], [4, 4, 4], x, y, tokens, work)
            i[0] += 1
        g = torch.empty((tokens, inter), device="cuda", dtype=torch.float32)
        u = torch.empty_like(g)
        h = torch.empty((tokens, inter), device="cuda", dtype=torch.int16)
        j = [0]

        def plain():
            w = wd[j[0] % nbf]
            gemm_bf16(x, w["gate"], g, tokens, inter, hidden, stream)
            gemm_bf16(x, w["up"], u, tokens, inter, hidden, stream)
            silu_mul(g, u, h, stream)
            gemm_bf16(h, w["down"], y, tokens, hidden, inter, stream)
            j[0] += 1
        plain()  # the library's candidate timing of each shape, once
        torch.cuda.synchronize()
        out[str(tokens)] = {"builtin_P4_us": round(time_graph(torch, fused, steps, 2, stream) * 1e3, 2),
                            "bf16_hipblaslt_us": round(time_graph(torch, plain, steps, 2, stream) * 1e3, 2)}
    del wd
    return out


# hidden and intermediate sizes of the SwiGLU layers tuned by main(), by model family
MODEL_SHAPES = {
    "8b": (4096, 14336, "Llama-3.1-8B"),
    "qwen7b": (3584, 18944, "Qwen2.5-7B"),
    "nemo12b": (5120, 14336, "Mistral-NeMo-12B"),
    "llama3b": (3072, 8192, "Llama-3.2-3B"),
}


def main(argv=None) -> int:
    import argparse
    import os
    import torch
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    sys.path.insert(0, root)
    import synth

    ap = argparse.ArgumentParser(description="tune pipelines and kernel variants of a SwiGLU MLP layer")
    ap.add_argument("--batches", default="1,16,64,256,1024")
    ap.add_argument("--model", default="8b", choices=sorted(MODEL_SHAPES),
                    help="layer shape: hidden x intermediate of a model family (synthetic weights)")
    ap.add_argument("--baselines", action="store_true",
                    help="also time the built-in choice and the uncompressed hipBLASLt layer")
    ap.add_argument("--out", default="")
    ap.add_argument("--keep", type=int, default=3)
    args = ap.parse_args(argv)
    torch.cuda.set_device(0)
    c = synth.CONFIGS["mlp_8b"]
    hidden, inter, label = MODEL_SHAPES[args.model]
    shapes = {"gate": (inter, hidden), "up": (inter, hidden), "down": (hidden, inter)}
    stream = torch.cuda.Stream()
    layer = {}
    weights = {}
    for proj in PROJECTIONS:
        rows, cols = shapes[proj]
        seed = c[proj][2] if args.model == "8b" else 200 + PROJECTIONS.index(proj)
        weights[proj] = synth.weights(rows, cols, seed, c["p"], c["shift"])
        m = Matrix(weights[proj], FMT_HUFFMAN | FMT_PALETTE)
        m.set_streams(stream)
        layer[proj] = copies_for(m, 1 << 30)
        for mm in layer[proj]:
            mm.set_streams(stream)
    n = min(len(v) for v in layer.values())
    for proj in PROJECTIONS:
        layer[proj] = layer[proj][:n]
    plan = tune_mlp(torch, layer, [int(t) for t in args.batches.split(",")], stream, keep=args.keep,
                    log=lambda s: print(s, file=sys.stderr, flush=True))
    if args.baselines:
        plan["baselines"] = layer_baselines(torch, layer, weights, [int(t) for t in args.batches.split(",")],
                                            stream)
        print(f"baselines: {json.dumps(plan['baselines'])}", file=sys.stderr, flush=True)
    plan["model"] = (f"{label}-shaped SwiGLU MLP (gate/up {inter}x{hidden}, down {hidden}x{inter}), "
                     "synthetic weights")
    plan["device"] = torch.cuda.get_device_name(0)
    text = json.dumps(plan, indent=1)
    if args.out:
        with open(args.out, "w") as f:
            f.write(text + "\n")
    print(text)
    return 0


if __name__ == "__main__":
    sys.exit(main())
