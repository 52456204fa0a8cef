"""The layer captured in a HIP graph (as bench.py times it) gives the eager
results bit for bit on every replay.

Each case captures three layer calls on different tokens into one graph and
replays it four times, with eager layer calls and synchronisations between
the replays (the library records no memset node: every buffer it clears is
written by its own kernels).
"""
import numpy as np
import pytest
import torch

import mixture_experts_router_amd as moe
import moe_inputs as mi
from gpu_util import Dev, host_bits

pytestmark = pytest.mark.gpu

GRAPH_CASES = {
    "decode_gemv": ("decode_b1", dict(T=6, H=1024, E=16, I=704), 1, {}),
    "decode_gemv_opts": ("decode_b1", dict(T=6, H=1024, E=16, I=704), 2, dict(groups=4, capacity=1, alpha=0.5)),
    "batched_mfma": ("batched_decode", dict(T=96, H=512, E=8, I=320), 32, {}),
    "entropy_two_pass": ("entropy", dict(T=192, H=512, E=16, I=192, bits=4, segment=2), 64, {}),
    "prefill_opts": ("prefill", dict(T=600, H=512, E=16, I=192), 200, dict(groups=4, capacity=96, alpha=0.5)),
    "decode_f4": ("decode_b1", dict(T=6, H=1024, E=16, I=704, fmt="nvfp4"), 1, {}),
    "batched_f4": ("prefill", dict(T=300, H=512, E=16, I=192, fmt="nvfp4"), 96, {}),
}


@pytest.mark.parametrize("name", list(GRAPH_CASES))
def test_graph_replays_match_eager(name):
    recipe, kw, tpc, opt = GRAPH_CASES[name]
    inp = mi.make_inputs(recipe, **kw)
    dev = Dev(inp)
    extra = {}
    if "alpha" in opt:
        extra["health"] = torch.from_numpy(mi.load_index(3, inp.E)).cuda()
        extra["alpha"] = opt["alpha"]
    for key in ("groups", "capacity"):
        if key in opt:
            extra[key] = opt[key]
    n_calls = inp.T // tpc
    xs = [dev.x[i * tpc:(i + 1) * tpc] for i in range(n_calls)][:3]
    ws = torch.empty(moe.layer_workspace_size(tpc, inp.H, inp.E, inp.k, inp.I, 0), dtype=torch.uint8, device="cuda")
    ys = [torch.empty((tpc, inp.H), dtype=dev.x.dtype, device="cuda") for _ in xs]
    print("case", name, "calls", len(xs), "tokens per call", tpc, flush=True)

    def calls():
        for x, y in zip(xs, ys):
            moe.layer_forward(x, dev.wr, inp.k, dev.down, gate_up=dev.gate_up, out=y, workspace=ws, **extra)

    calls()
    torch.cuda.synchronize()
    eager = [host_bits(y) for y in ys]
    # warm the capture stream, then capture
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        calls()
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    torch.cuda.synchronize()
    other = torch.empty_like(ys[0])
    for rep in range(4):
        for y in ys:
            y.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, y in enumerate(ys):
            assert np.array_equal(host_bits(y), eager[i]), "%s replay %d call %d" % (name, rep, i)
        # eager work between replays reuses the same workspace
        moe.layer_forward(xs[-1], dev.wr, inp.k, dev.down, gate_up=dev.gate_up, out=other, workspace=ws, **extra)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(other), eager[-1])
