"""moe_layer_forward_noalloc (no workspace argument, no allocation) against
moe_layer_forward_ex with a caller workspace: the same kernels on the same
inputs, so the outputs must be bit-identical.  Two calls in a row share the
library's scratch array, the second with a smaller input, so stale contents
from the first call must not leak into the second."""
import numpy as np
import pytest
import torch

import mixture_experts_router_amd as moe
import moe_inputs as mi
from gpu_util import Dev, host_bits

pytestmark = pytest.mark.gpu


def _both(dev, x, flags=0, **opts):
    inp = dev.inp
    T = x.shape[0]
    taps_a = moe.make_taps(T, inp.E, inp.k, inp.I, "cuda", names=("topk_idx", "topk_w", "k_used", "perm"))
    taps_b = moe.make_taps(T, inp.E, inp.k, inp.I, "cuda", names=("topk_idx", "topk_w", "k_used", "perm"))
    y_ref = moe.layer_forward(x, dev.wr, inp.k, dev.down, gate_up=dev.gate_up, flags=flags, taps=taps_a, **opts)
    y = torch.full_like(x, float("nan"))
    moe.layer_forward_noalloc(x, dev.wr, inp.k, dev.down, gate_up=dev.gate_up, flags=flags, taps=taps_b, out=y,
                              **opts)
    torch.cuda.synchronize()
    for n in taps_a:
        assert torch.equal(taps_a[n], taps_b[n]), n
    return host_bits(y_ref), host_bits(y), moe.last_plan()


@pytest.mark.parametrize("recipe,kw,flags", [
    # batched path (sort, MFMA GEMMs, combine), then the first 40 tokens
    ("prefill", dict(T=300, H=512, E=16, I=192), moe.FLAG_FORCE_MFMA),
    # entropy-adaptive k on the batched path (two-pass selection)
    ("entropy", dict(T=96, H=512, E=16, I=192, bits=4, segment=2), 0),
    # decode path (three launches), a ragged batch then one token
    ("decode_b1", dict(T=3, H=1024, E=16, I=704), 0),
])
def test_noalloc_matches_workspace_entry_point(recipe, kw, flags):
    inp = mi.make_inputs(recipe, **kw)
    dev = Dev(inp)
    print("case", recipe, kw, flush=True)
    first = dev.x
    second = dev.x[: max(1, inp.T // 7)].contiguous()  # a smaller second call
    for x in (first, second):
        ref, got, plan = _both(dev, x, flags)
        assert np.array_equal(ref, got), (recipe, x.shape[0], plan)


def test_noalloc_with_routing_options_and_capacity():
    inp = mi.make_inputs("prefill", T=300, H=512, E=16, I=192)
    dev = Dev(inp)
    health = torch.from_numpy(mi.load_index(5, inp.E)).cuda()
    opts = dict(health=health, alpha=0.5, groups=4, capacity=48)
    for x in (dev.x, dev.x[:64].contiguous()):
        ref, got, _ = _both(dev, x, **opts)
        assert np.array_equal(ref, got)


def test_noalloc_refuses_what_does_not_fit_and_enqueues_nothing():
    # T*kcap*H*2 bytes of down outputs alone exceed the scratch array here
    inp = mi.make_inputs("tiny", T=4096, H=4096, E=8, k=2, I=128)
    dev = Dev(inp)
    y = torch.full_like(dev.x, 7.0)
    with pytest.raises(moe.MoeError) as ei:
        moe.layer_forward_noalloc(dev.x, dev.wr, inp.k, dev.down, gate_up=dev.gate_up, out=y)
    assert ei.value.name == "MOE_ERR_SCRATCH"
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)
