"""Routing options on the GPU against the oracle, through the C ABI: the
load-aware logit correction, group-limited selection, and the expert load
statistics.

Bars as elsewhere: logits bit-exact where the inputs make every partial sum
exact; indices bit-exact on identical logits; weights within 1e-6; layer
output max-abs <= 2e-2 and rel-L2 <= 5e-3 against the oracle under the
verified routing; fused == unfused bit-exact; statistics: least-used expert
exact and the standard deviation within one fp32 ulp of the oracle's.
"""
import numpy as np
import pytest
import torch

import mixture_experts_router_amd as moe
import moe_inputs as mi
import oracle
from gpu_util import Dev, assert_within_tolerance, batched_path_takes, dev_half, host_bits

pytestmark = pytest.mark.gpu


def _health(E, seed=5):
    return mi.load_index(seed, E)


# ---------------------------------------------------------- correction --

@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("T,E,k,groups", [(1, 64, 4, 0), (7, 8, 2, 0), (300, 64, 4, 4), (33, 32, -1, 0),
                                          (200, 64, 4, 0), (129, 256, 8, 8), (64, 32, -1, 8)])
def test_corrected_logits_and_selection_exact(dtype, T, E, k, groups):
    x, wr = mi.exact_router_inputs(9, T, 1024, E, dtype)
    hv = _health(E)
    alpha = 0.375
    print("route T=%d E=%d k=%d groups=%d %s" % (T, E, k, groups, dtype), flush=True)
    r = moe.route(dev_half(x, dtype), dev_half(wr, dtype), k, want_logits=True,
                  health=torch.from_numpy(hv).cuda(), alpha=alpha, groups=groups)
    torch.cuda.synchronize()
    idx_o, w_o, ku_o, hm_o, lo = oracle.route(x, wr, dtype, k, want_logits=True, health=hv, alpha=alpha,
                                              groups=groups)
    assert np.array_equal(r["logits"].cpu().numpy(), lo), "corrected logits differ"
    assert int(r["k_used"].item()) == ku_o
    assert np.array_equal(r["idx"].cpu().numpy(), idx_o)
    assert np.max(np.abs(r["w"].cpu().numpy() - w_o)) <= 1e-6


def test_correction_with_zero_alpha_is_plain_routing():
    x, wr = mi.exact_router_inputs(10, 40, 512, 16, "f16")
    a = moe.route(dev_half(x, "f16"), dev_half(wr, "f16"), 2, want_logits=True)
    b = moe.route(dev_half(x, "f16"), dev_half(wr, "f16"), 2, want_logits=True,
                  health=torch.from_numpy(_health(16)).cuda(), alpha=0.0)
    torch.cuda.synchronize()
    for n in ("logits", "idx", "w"):
        assert torch.equal(a[n], b[n]), n


# ------------------------------------------------------------- groups --

@pytest.mark.parametrize("E,G,k", [(64, 4, 4), (64, 4, 2), (64, 8, 3), (256, 32, 8), (12, 3, 3), (32, 8, -1),
                                   (16, 16, 5)])
def test_grouped_topk_from_identical_logits(E, G, k):
    rng = np.random.default_rng(E * 100 + G)
    logits = (rng.standard_normal((200, E)) * 1.5).astype(np.float32)
    logits[:40, 3] = logits[:40, 1]          # ties inside a group
    logits[40:60, E // G] = logits[40:60, 0]  # ties across groups
    logits[60:70] = 0.25                      # all equal
    r = moe.topk_from_logits(torch.from_numpy(logits).cuda(), k, groups=G)
    torch.cuda.synchronize()
    ku = int(r["k_used"].item())
    kcap = k if k > 0 else 3
    if k < 0:
        assert ku == oracle.entropy_k(oracle.batch_entropy(logits))
    oi, ow = oracle.select_topk(logits, ku, kcap, groups=G)
    assert np.array_equal(r["idx"].cpu().numpy(), oi)
    assert np.max(np.abs(r["w"].cpu().numpy() - ow)) <= 1e-6


# ------------------------------------------------------- whole layer --

LAYER_CASES = {
    "decode_small": ("decode_b1", dict(T=1, H=1024, E=16, I=704), 4),
    "decode_t3": ("decode_b1", dict(T=3, H=512, E=16, I=320), 4),
    "batched_small": ("batched_decode", dict(T=40, H=512, E=8, I=320), 2),
    "prefill_small": ("prefill", dict(T=300, H=512, E=16, I=192), 4),
    "entropy_q4": ("entropy", dict(T=96, H=512, E=16, I=192, bits=4, segment=2), 4),
    "decode_q5": ("decode_b1", dict(T=3, H=512, E=16, I=320, bits=5), 4),
    "decode_q6": ("decode_b1", dict(T=2, H=1024, E=16, I=704, bits=6), 4),
    "batched_q5": ("prefill", dict(T=200, H=512, E=16, I=256, bits=5), 4),
    "decode_f4": ("decode_b1", dict(T=3, H=512, E=16, I=320, fmt="nvfp4"), 4),
    "batched_f4": ("prefill", dict(T=200, H=512, E=16, I=256, fmt="nvfp4"), 4),
}


def _option_paths(inp):
    """Both paths where the weights allow (5-bit codes on the batched path:
    hidden and inter multiples of 128)."""
    P = inp.T * inp.kcap
    paths = [("mfma", moe.FLAG_FORCE_MFMA)] if batched_path_takes(inp) else []
    return paths + ([("gemv", moe.FLAG_FORCE_GEMV)] if P <= 128 else [])


@pytest.mark.parametrize("name", list(LAYER_CASES))
def test_layer_with_options_matches_oracle(name):
    recipe, kw, groups = LAYER_CASES[name]
    inp = mi.make_inputs(recipe, **kw)
    dev = Dev(inp)
    gu_np = oracle.fuse_gate_up(inp.gate, inp.up)
    hv = _health(inp.E, seed=7)
    hd = torch.from_numpy(hv).cuda()
    alpha = 0.5
    paths = _option_paths(inp)
    print("case", name, "T=%d E=%d k=%d groups=%d" % (inp.T, inp.E, inp.k, groups), flush=True)
    for pname, pflag in paths:
        outs = []
        for extra in (0, moe.FLAG_UNFUSED):
            taps = moe.make_taps(inp.T, inp.E, inp.k, inp.I, "cuda")
            y = moe.layer_forward(dev.x, dev.wr, inp.k, dev.down, gate_up=dev.gate_up, flags=pflag | extra,
                                  taps=taps, health=hd, alpha=alpha, groups=groups)
            torch.cuda.synchronize()
            outs.append((host_bits(y), {n: v.cpu().numpy() for n, v in taps.items()}))
        (y, t), (y_u, t_u) = outs
        assert np.array_equal(y, y_u), "%s/%s fused vs unfused" % (name, pname)
        ku = int(t["k_used"][0])
        # the corrected logits: the oracle's correction of the GPU's raw logits
        raw = moe.route(dev.x, dev.wr, inp.k, want_logits=True)["logits"].cpu().numpy()
        assert np.array_equal(t["logits"], oracle.correct_logits(raw, hv, alpha))
        # selection on identical (corrected) logits
        oi, ow = oracle.select_topk(t["logits"], ku, inp.kcap, groups=groups)
        assert np.array_equal(t["topk_idx"], oi), "%s/%s selection" % (name, pname)
        assert np.max(np.abs(t["topk_w"] - ow)) <= 1e-6
        # the oracle's own routing agrees except at near-ties of its logits
        io, wo, kuo, _, lo = oracle.route(inp.x, inp.wr, inp.dtype, inp.k, want_logits=True, health=hv,
                                          alpha=alpha, groups=groups)
        assert kuo == ku
        assert np.max(np.abs(lo - t["logits"])) <= 1e-4 * max(1.0, float(np.max(np.abs(lo))))
        ref = oracle.tokens_forward(inp.x, inp.dtype, np.arange(inp.T), t["topk_idx"], t["topk_w"], ku, gu_np,
                                    inp.down)
        assert_within_tolerance(y, ref, inp.dtype, "%s/%s" % (name, pname))
        # the load figures of this call's counts
        lu, sd = moe.expert_load_stats(torch.from_numpy(t["counts"]).cuda())
        olu, osd = oracle.load_stats(t["counts"])
        assert int(lu.item()) == olu
        assert abs(float(sd.item()) - osd) <= np.spacing(np.float32(osd))


# --------------------------------------------------------- load stats --

@pytest.mark.parametrize("E", [1, 7, 32, 64, 65, 256])
def test_load_stats_matches_oracle(E):
    rng = np.random.default_rng(E)
    cases = [np.zeros(E, np.int32), np.full(E, 5, np.int32), rng.integers(0, 1000, E).astype(np.int32),
             rng.integers(0, 1 << 30, E).astype(np.int32), (rng.integers(0, 3, E) * 7).astype(np.int32)]
    one = np.zeros(E, np.int32)
    one[E // 2] = 1 << 20
    cases.append(one)
    for c in cases:
        lu, sd = moe.expert_load_stats(torch.from_numpy(c).cuda())
        torch.cuda.synchronize()
        olu, osd = oracle.load_stats(c)
        assert int(lu.item()) == olu, (E, c[:8])
        assert abs(float(sd.item()) - osd) <= np.spacing(np.float32(osd)), (E, float(sd.item()), osd)


# ----------------------------------------------------------- capacity --

CAP_CASES = {
    "decode_t3": ("decode_b1", dict(T=3, H=512, E=16, I=320), [1, 2]),
    "decode_t4_e4": ("decode_b1", dict(T=4, H=512, E=4, k=2, I=320), [1, 3]),
    "batched_small": ("batched_decode", dict(T=40, H=512, E=8, I=320), [3, 8]),
    "prefill_small": ("prefill", dict(T=300, H=512, E=16, I=192), [20, 64]),
    "entropy_q4": ("entropy", dict(T=96, H=512, E=16, I=192, bits=4, segment=2), [5]),
    "decode_q5": ("decode_b1", dict(T=4, H=512, E=4, k=2, I=320, bits=5), [1, 3]),
    "decode_q6": ("decode_b1", dict(T=4, H=512, E=4, k=2, I=320, bits=6), [1, 3]),
    "decode_f4": ("decode_b1", dict(T=4, H=512, E=4, k=2, I=320, fmt="nvfp4"), [1, 3]),
    "prefill_f4": ("prefill", dict(T=300, H=512, E=16, I=192, fmt="nvfp4"), [20, 64]),
    # more than 64 experts: the sort's workgroups take two and four experts each
    "batched_e96": ("prefill", dict(T=300, H=256, E=96, k=4, I=128), [4, 12]),
    "batched_e256": ("prefill", dict(T=400, H=256, E=256, k=8, I=128), [3, 10]),
}


@pytest.mark.parametrize("name", list(CAP_CASES))
def test_layer_with_capacity_matches_oracle(name):
    recipe, kw, caps = CAP_CASES[name]
    inp = mi.make_inputs(recipe, **kw)
    dev = Dev(inp)
    gu_np = oracle.fuse_gate_up(inp.gate, inp.up)
    paths = _option_paths(inp)
    for pname, pflag in paths:
        base_t = moe.make_taps(inp.T, inp.E, inp.k, inp.I, "cuda")
        y0 = host_bits(moe.layer_forward(dev.x, dev.wr, inp.k, dev.down, gate_up=dev.gate_up, flags=pflag,
                                         taps=base_t))
        torch.cuda.synchronize()
        idx = base_t["topk_idx"].cpu().numpy()
        w = base_t["topk_w"].cpu().numpy()
        ku = int(base_t["k_used"].item())
        routed = np.bincount(idx[:, :ku].ravel(), minlength=inp.E)
        for C in caps + [int(routed.max())]:
            print("case", name, pname, "capacity", C, "max routed", int(routed.max()), flush=True)
            outs = []
            for extra in (0, moe.FLAG_UNFUSED):
                taps = moe.make_taps(inp.T, inp.E, inp.k, inp.I, "cuda")
                y = moe.layer_forward(dev.x, dev.wr, inp.k, dev.down, gate_up=dev.gate_up, flags=pflag | extra,
                                      taps=taps, capacity=C)
                torch.cuda.synchronize()
                outs.append((host_bits(y), {n: v.cpu().numpy() for n, v in taps.items()}))
            (y, t), (y_u, _) = outs
            assert np.array_equal(y, y_u), "fused vs unfused"
            assert np.array_equal(t["topk_idx"], idx)  # routing unchanged
            # the dispatch lists exactly the oracle's kept pairs
            c, o, p_, _ = oracle.sort_pairs(idx, ku, inp.E, capacity=C)
            assert np.array_equal(t["counts"], c) and np.array_equal(t["offsets"], o)
            assert np.array_equal(t["perm"], p_)
            keep = oracle.capacity_keep(idx, ku, inp.E, C)
            if C >= routed.max():
                assert keep[:, :ku].all()
                assert np.array_equal(y, y0), "a capacity above every count changes nothing"
            idx_kept = np.where(keep, idx, -1).astype(np.int32)
            ref = oracle.tokens_forward(inp.x, inp.dtype, np.arange(inp.T), idx_kept, w, ku, gu_np, inp.down)
            assert_within_tolerance(y, ref, inp.dtype, "%s/%s C=%d (dropped %d)" % (name, pname, C,
                                                                                   int((~keep[:, :ku]).sum())))
