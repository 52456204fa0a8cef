"""Full-size workloads on the GPU, in the launch configuration the benchmark
times, checked against the oracle on sampled tokens (the oracle computes each
token's output independently), plus the properties that hold at any size:
bit-exact routing on identical logits, exact sort, fused == unfused.
"""
import time

import numpy as np
import pytest
import torch

import mixture_experts_router_amd as moe
import moe_inputs as mi
import oracle
from gpu_util import Dev, assert_within_tolerance, check_routing_identical_logits, host_bits, reference_outputs

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _gen(recipe, **kw):
    t = time.time()
    inp = mi.make_inputs(recipe, **kw)
    gu_np = oracle.fuse_gate_up(inp.gate, inp.up)
    dev = Dev(inp)
    torch.cuda.synchronize()
    _say("generated %s %s in %.1fs" % (recipe, kw, time.time() - t))
    return inp, gu_np, dev


def _forward(dev, flags=0):
    inp = dev.inp
    taps = moe.make_taps(inp.T, inp.E, inp.k, inp.I, "cuda", names=("logits", "topk_idx", "topk_w", "k_used",
                                                                      "counts", "offsets", "perm"))
    y = dev.forward(flags=flags, taps=taps)
    return host_bits(y), {k: v.cpu().numpy() for k, v in taps.items()}, moe.last_plan()


def _check(inp, gu_np, y, taps, tokens, label):
    ku = int(taps["k_used"][0])
    check_routing_identical_logits(taps["logits"], taps["topk_idx"], taps["topk_w"], ku)
    ref, flips = reference_outputs(inp, gu_np, tokens, taps["topk_idx"], taps["topk_w"], ku)
    assert_within_tolerance(y[tokens], ref, inp.dtype, "%s (tokens %d, near-tie flips %d)" % (label, len(tokens),
                                                                                             flips))
    if "perm" in taps:
        counts, offsets, perm, _ = oracle.sort_pairs(taps["topk_idx"], ku, inp.E)
        assert np.array_equal(taps["counts"], counts) and np.array_equal(taps["perm"], perm)


def _assert_packed_same(dev, y):
    """The benchmark loads its weights with pack_sb: same bits as the per-call repack."""
    if dev.inp.bits == 16:
        return
    gu, dn = moe.pack_sb(dev.gate_up), moe.pack_sb(dev.down)
    yp = host_bits(moe.layer_forward(dev.x, dev.wr, dev.inp.k, dn, gate_up=gu))
    assert np.array_equal(yp, y), "prepacked scales vs per-call repack"


def test_decode_b1_full_size():
    _decode_one_token_calls(*_gen("decode_b1", T=6), "decode_b1")


@pytest.mark.parametrize("bits", [5, 6])
def test_decode_b1_full_size_5_and_6_bit(bits):
    # the benchmark's 5- and 6-bit decode shape: H 4096, E 64, top-4, I 2816
    _decode_one_token_calls(*_gen("decode_b1", T=4, I=2816, bits=bits), "decode_b1 %d-bit" % bits)


def _decode_one_token_calls(inp, gu_np, dev, label):
    for t in range(inp.T):
        # one token per call, as the benchmark runs it
        x1 = dev.x[t:t + 1]
        taps = moe.make_taps(1, inp.E, inp.k, inp.I, "cuda", names=("logits", "topk_idx", "topk_w", "k_used"))
        y = host_bits(moe.layer_forward(x1, dev.wr, inp.k, dev.down, gate_up=dev.gate_up, taps=taps))
        plan = moe.last_plan()
        y_u = host_bits(moe.layer_forward(x1, dev.wr, inp.k, dev.down, gate_up=dev.gate_up, flags=moe.FLAG_UNFUSED))
        assert np.array_equal(y, y_u), "decode fused vs unfused"
        assert "gemv_gate_up_swiglu" in plan, plan
        tp = {k: v.cpu().numpy() for k, v in taps.items()}
        import dataclasses
        sub = dataclasses.replace(inp, T=1, x=np.ascontiguousarray(inp.x[t:t + 1]))
        _check(sub, gu_np, y, tp, np.array([0]), "%s token %d" % (label, t))


def test_decode_b1_full_size_mfma_path():
    inp, gu_np, dev = _gen("decode_b1", T=2)
    y, taps, plan = _forward(dev, moe.FLAG_FORCE_MFMA)
    assert "gemm_gate_up_swiglu" in plan
    _check(inp, gu_np, y, taps, np.arange(inp.T), "decode_b1/mfma")


def test_batched_decode_full_size():
    inp, gu_np, dev = _gen("batched_decode")
    y, taps, plan = _forward(dev)
    _say("plan", plan, "counts", taps["counts"].tolist())
    _check(inp, gu_np, y, taps, np.arange(inp.T), "batched_decode")
    y_u, _, _ = _forward(dev, moe.FLAG_UNFUSED)
    assert np.array_equal(y, y_u)
    _assert_packed_same(dev, y)


def test_prefill_full_size():
    _prefill_full_size(*_gen("prefill"), "prefill")


@pytest.mark.parametrize("bits", [5, 6])
def test_prefill_full_size_5_and_6_bit(bits):
    # the prefill shape with 5- and 6-bit codes on the batched path (40- and
    # 48-byte group rows staged through LDS)
    _prefill_full_size(*_gen("prefill", bits=bits), "prefill %d-bit" % bits)


def test_decode_b1_full_size_6_bit_inter_11008():
    # the decode shape itself with 6-bit codes: 11 chunks per lane in a down
    # row, four waves per slot
    _decode_one_token_calls(*_gen("decode_b1", T=3, bits=6), "decode_b1 6-bit I 11008")


def test_decode_b1_full_size_nvfp4():
    # the decode shape with NVFP4 weights: H 4096 (two chunks per lane),
    # I 11008 (six chunks per down row, two waves per slot)
    _decode_one_token_calls(*_gen("decode_b1", T=3, fmt="nvfp4"), "decode_b1 NVFP4")


def test_prefill_full_size_nvfp4():
    _prefill_full_size(*_gen("prefill", fmt="nvfp4"), "prefill NVFP4")


def _prefill_full_size(inp, gu_np, dev, label):
    y, taps, plan = _forward(dev)
    assert "gemm_gate_up_swiglu" in plan, plan
    counts = taps["counts"]
    _say("plan", plan, "hot expert %d tokens, mean %.1f" % (counts.max(), counts.mean()))
    assert counts.max() >= 10 * counts.mean()
    # sampled tokens: the first few, some of the hot expert's, and a spread
    hot = int(np.argmax(counts))
    hot_tokens = np.where((taps["topk_idx"] == hot).any(axis=1))[0]
    rng = np.random.default_rng(0)
    tokens = np.unique(np.concatenate([np.arange(4), hot_tokens[:6], hot_tokens[-4:],
                                       rng.choice(inp.T, 14, replace=False), [inp.T - 1]]))
    _check(inp, gu_np, y, taps, tokens, label)
    y_u, _, _ = _forward(dev, moe.FLAG_UNFUSED)
    assert np.array_equal(y, y_u)
    _assert_packed_same(dev, y)


@pytest.mark.parametrize("bits", [16, 4])
def test_entropy_full_size(bits):
    import dataclasses
    from gpu_util import dev_half
    inp0, gu_np, dev = _gen("entropy", bits=bits, segment=0)
    for seg, k_expect in enumerate((1, 2, 3, 3)):
        # same expert weights; each segment has its own tokens and router temperature
        x, wr, _ = mi.make_router_inputs("entropy", segment=seg)
        inp = dataclasses.replace(inp0, x=x, wr=wr, segment=seg)
        dev.inp, dev.x, dev.wr = inp, dev_half(x, "f16"), dev_half(wr, "f16")
        y, taps, plan = _forward(dev)
        assert int(taps["k_used"][0]) == k_expect
        rng = np.random.default_rng(seg)
        tokens = np.unique(np.concatenate([[0, inp.T - 1], rng.choice(inp.T, 10, replace=False)]))
        _check(inp, gu_np, y, taps, tokens, "entropy bits=%d segment %d (k=%d)" % (bits, seg, k_expect))
        y_u, _, _ = _forward(dev, moe.FLAG_UNFUSED)
        assert np.array_equal(y, y_u)
        _assert_packed_same(dev, y)


# ------------------------------------------ routing options, full size --

def _opt_check(inp, gu_np, dev, tokens, label, flags=0, **opt):
    """Layer with routing options vs the oracle on sampled tokens: corrected
    logits, selection on identical logits, capped sort, outputs under the kept
    pairs, fused == unfused."""
    health = opt.pop("health", None)
    extra = dict(opt)
    if health is not None:
        extra["health"] = torch.from_numpy(health).cuda()
    outs, plans = [], []
    for f in (flags, flags | moe.FLAG_UNFUSED):
        taps = moe.make_taps(inp.T, inp.E, inp.k, inp.I, "cuda",
                             names=("logits", "topk_idx", "topk_w", "k_used", "counts", "offsets", "perm"))
        y = host_bits(moe.layer_forward(dev.x, dev.wr, inp.k, dev.down, gate_up=dev.gate_up, flags=f, taps=taps,
                                        **extra))
        plans.append(moe.last_plan())
        outs.append((y, {k: v.cpu().numpy() for k, v in taps.items()}))
    (y, t), (y_u, _) = outs
    assert np.array_equal(y, y_u), label + " fused vs unfused"
    ku = int(t["k_used"][0])
    groups, cap = opt.get("groups", 0), opt.get("capacity", 0)
    if health is not None:
        raw = moe.route(dev.x, dev.wr, inp.k, want_logits=True)["logits"].cpu().numpy()
        assert np.array_equal(t["logits"], oracle.correct_logits(raw, health, opt["alpha"]))
    oi, ow = oracle.select_topk(t["logits"], ku, inp.kcap, groups=groups)
    assert np.array_equal(t["topk_idx"], oi), label + " selection"
    assert np.max(np.abs(t["topk_w"] - ow)) <= 1e-6
    c, o, p, _ = oracle.sort_pairs(t["topk_idx"], ku, inp.E, capacity=cap)
    assert np.array_equal(t["counts"], c) and np.array_equal(t["offsets"], o) and np.array_equal(t["perm"], p)
    keep = oracle.capacity_keep(t["topk_idx"], ku, inp.E, cap)
    idx_kept = np.where(keep, t["topk_idx"], -1).astype(np.int32)
    ref = oracle.tokens_forward(inp.x, inp.dtype, tokens, idx_kept, t["topk_w"], ku, gu_np, inp.down)
    assert_within_tolerance(y[tokens], ref, inp.dtype, "%s (tokens %d, dropped pairs %d)" % (
        label, len(tokens), int((~keep[:, :ku]).sum())))
    return t, keep, plans[0]


def test_decode_b1_full_size_with_options():
    inp, gu_np, dev = _gen("decode_b1", T=4)
    hv = mi.load_index(5, inp.E)
    # the decode path (four tokens, 16 pairs) with correction and groups, and
    # a capacity that drops pairs two tokens share
    _, _, plan = _opt_check(inp, gu_np, dev, np.arange(inp.T), "decode_b1 opts", flags=moe.FLAG_FORCE_GEMV,
                            health=hv, alpha=0.5, groups=4, capacity=1)
    assert "gemv_gate_up_swiglu" in plan, plan


def test_prefill_full_size_with_options():
    inp, gu_np, dev = _gen("prefill")
    hv = mi.load_index(5, inp.E)
    rng = np.random.default_rng(3)
    tokens = np.unique(np.concatenate([np.arange(3), rng.choice(inp.T, 12, replace=False), [inp.T - 1]]))
    _opt_check(inp, gu_np, dev, tokens, "prefill correction+groups", health=hv, alpha=0.5, groups=4)
    # capacity 512 (twice the mean) caps the hot experts; sample dropped tokens too
    cap = 512
    base = moe.make_taps(inp.T, inp.E, inp.k, inp.I, "cuda", names=("topk_idx", "k_used"))
    dev.forward(taps=base)
    bidx = base["topk_idx"].cpu().numpy()
    bkeep = oracle.capacity_keep(bidx, inp.k, inp.E, cap)
    dropped = np.where(~bkeep.all(axis=1))[0]
    _say("capacity %d drops %d pairs of %d tokens" % (cap, int((~bkeep).sum()), dropped.size))
    assert dropped.size > 0
    tokens = np.unique(np.concatenate([tokens, dropped[:6], dropped[-4:]]))
    _opt_check(inp, gu_np, dev, tokens, "prefill capacity", capacity=cap)
