"""HIP path vs the CPU oracle, through the C ABI, at sizes the oracle finishes
in seconds that still span several tiles and a ragged tail.

Bars: expert indices and sort results bit-exact (on identical logits);
GPU fused == GPU unfused bit-exact; layer output max-abs <= 2e-2 and rel-L2
<= 5e-3 against the oracle's fp32 result.
"""
import numpy as np
import pytest
import torch

import mixture_experts_router_amd as moe
import moe_inputs as mi
import oracle
from ref64 import half64
from gpu_util import (Dev, assert_within_tolerance, batched_path_takes, check_routing_identical_logits, dev_half,
                      host_bits, reference_outputs)

pytestmark = pytest.mark.gpu

# (recipe, overrides) — scaled-down shapes of the five workloads plus edge cases
CASES = {
    "tiny": ("tiny", dict()),
    "tiny_q8_bf16": ("tiny", dict(bits=8, dtype="bf16")),
    "tiny_fp16w": ("tiny", dict(bits=16)),
    "decode_small": ("decode_b1", dict(T=1, H=1024, E=16, I=704)),
    "decode_t3": ("decode_b1", dict(T=3, H=512, E=16, I=320)),
    "batched_small": ("batched_decode", dict(T=40, H=512, E=8, I=320)),
    "prefill_small": ("prefill", dict(T=300, H=512, E=16, I=192)),
    "prefill_bm128": ("prefill", dict(T=2304, H=256, E=8, I=384)),
    "entropy_fp16w": ("entropy", dict(T=96, H=512, E=16, I=192, bits=16)),
    "entropy_q4": ("entropy", dict(T=96, H=512, E=16, I=192, bits=4, segment=2)),
    "one_expert": ("tiny", dict(E=1, k=1, T=5)),
    "dense_k_eq_e": ("tiny", dict(k=8, T=6)),
    "k8_e256": ("tiny", dict(E=256, k=8, T=12, H=128, I=64)),
    "ragged_shapes": ("tiny", dict(T=37, H=192, E=12, k=3, I=320)),
    # bf16 batches that end inside a sort-and-convert workgroup (four tokens
    # each): 8-bit and 4-bit weights
    "batched_bf16_ragged": ("batched_decode", dict(T=37, H=512, E=8, I=320)),
    "prefill_bf16_ragged": ("prefill", dict(T=301, H=512, E=16, I=192)),
    # 256 experts over 4800 pairs: four experts per sort workgroup
    "batched_e256": ("prefill", dict(T=600, H=256, E=256, k=8, I=128)),
    # more than 16384 logits with H not a multiple of 256: the four-wave MFMA router
    "ragged_mfma_router": ("tiny", dict(T=200, H=192, E=96, k=3, I=128)),
    # decode shapes with long down rows (two waves per slot), one per
    # weight format
    "decode_1l_q4": ("decode_b1", dict(T=2, H=1024, E=8, I=8192)),
    "decode_1l_q8": ("decode_b1", dict(T=1, H=2048, E=8, I=6144, bits=8)),
    "decode_1l_fp16": ("decode_b1", dict(T=1, H=1024, E=8, I=3072, bits=16)),
    # 6-bit codes (decode path only): a ragged batch, three chunks per lane,
    # and the longest down row the decode kernels take (six chunks per lane)
    "decode_q6": ("decode_b1", dict(T=3, H=1024, E=16, I=704, bits=6)),
    "decode_q6_h4096": ("decode_b1", dict(T=1, H=4096, E=8, I=2816, bits=6)),
    "decode_q6_long": ("decode_b1", dict(T=2, H=1024, E=8, I=6144, bits=6)),
    # 5-bit codes (decode path only): one, two and (two waves per slot, a
    # ragged last round) three chunks per lane
    "decode_q5": ("decode_b1", dict(T=3, H=1024, E=16, I=704, bits=5)),
    "decode_q5_h4096": ("decode_b1", dict(T=1, H=4096, E=8, I=2816, bits=5)),
    "decode_q5_long": ("decode_b1", dict(T=2, H=1024, E=8, I=11008, bits=5)),
    "decode_q5_bf16": ("decode_b1", dict(T=2, H=512, E=8, I=320, bits=5, dtype="bf16")),
    # entropy-adaptive k on the decode path (kcap 3, 12 pairs)
    "entropy_q6": ("entropy", dict(T=4, H=512, E=16, I=192, bits=6, segment=2)),
    # 5- and 6-bit codes on the batched path: 64-row tiles (5-bit two-group
    # stages, 6-bit one-group stages with an odd group count), 32-row tiles,
    # 128-row tiles, and bf16 activations
    "batched_q5": ("prefill", dict(T=300, H=512, E=16, I=256, bits=5)),
    "batched_q6": ("prefill", dict(T=300, H=512, E=16, I=320, bits=6)),
    "batched_q5_bm32": ("batched_decode", dict(T=40, H=512, E=8, I=256, bits=5)),
    "batched_q6_bm32": ("batched_decode", dict(T=40, H=384, E=8, I=192, bits=6)),
    "prefill_q5_bm128": ("prefill", dict(T=2304, H=256, E=8, I=384, bits=5)),
    "prefill_q6_bm128": ("prefill", dict(T=2304, H=256, E=8, I=384, bits=6)),
    "entropy_q5": ("entropy", dict(T=96, H=512, E=16, I=256, bits=5, segment=2)),
    # a small batch over long rows (bf16 activations; 8- and 4-bit weights)
    "batched_long_k": ("batched_decode", dict(T=16, H=2048, E=16, I=1024)),
    "batched_long_k_q4": ("prefill", dict(T=8, H=2048, E=16, I=1024)),
    # NVFP4 weights (E2M1 codes, E4M3 block scales, tensor scale): decode
    # (one and two chunks per lane, long down rows), the batched tiles of 32,
    # 64 and 128 rows with an odd group count on the down GEMM, bf16
    # activations, and entropy-adaptive k
    "decode_f4": ("decode_b1", dict(T=3, H=1024, E=16, I=704, fmt="nvfp4")),
    "decode_f4_h4096": ("decode_b1", dict(T=1, H=4096, E=8, I=2816, fmt="nvfp4")),
    "decode_f4_long": ("decode_b1", dict(T=2, H=1024, E=8, I=11008, fmt="nvfp4")),
    "batched_f4": ("prefill", dict(T=300, H=512, E=16, I=192, fmt="nvfp4")),
    "batched_f4_bm32": ("batched_decode", dict(T=40, H=512, E=8, I=320, fmt="nvfp4")),
    "prefill_f4_bm128": ("prefill", dict(T=2304, H=256, E=8, I=384, fmt="nvfp4")),
    "entropy_f4": ("entropy", dict(T=96, H=512, E=16, I=192, fmt="nvfp4", segment=2)),
    "batched_long_k_f4": ("batched_decode", dict(T=16, H=2048, E=16, I=1024, fmt="nvfp4")),
}


@pytest.fixture(scope="module")
def built():
    cache = {}

    def get(name):
        if name not in cache:
            recipe, kw = CASES[name]
            inp = mi.make_inputs(recipe, **kw)
            gu_np = oracle.fuse_gate_up(inp.gate, inp.up)
            cache[name] = (inp, gu_np, Dev(inp))
        return cache[name]

    return get


def _run(dev, flags, fused_tensor=True):
    inp = dev.inp
    taps = moe.make_taps(inp.T, inp.E, inp.k, inp.I, "cuda")
    y = dev.forward(flags=flags, fused_tensor=fused_tensor, taps=taps)
    return host_bits(y), {k: v.cpu().numpy() for k, v in taps.items()}


def _paths(inp):
    P = inp.T * inp.kcap
    paths = [("mfma", moe.FLAG_FORCE_MFMA)] if batched_path_takes(inp) else []
    if P <= 128:
        paths.append(("gemv", moe.FLAG_FORCE_GEMV))
    return paths


@pytest.mark.parametrize("name", list(CASES))
def test_layer_matches_oracle(name, built):
    inp, gu_np, dev = built(name)
    print("case", name, "T=%d H=%d E=%d I=%d k=%d bits=%d %s %s" % (inp.T, inp.H, inp.E, inp.I, inp.k, inp.bits,
                                                                    inp.fmt, inp.dtype), flush=True)
    for pname, pflag in _paths(inp):
        y, taps = _run(dev, pflag)
        ku = int(taps["k_used"][0])
        check_routing_identical_logits(taps["logits"], taps["topk_idx"], taps["topk_w"], ku)
        ref, flips = reference_outputs(inp, gu_np, np.arange(inp.T), taps["topk_idx"], taps["topk_w"], ku)
        assert_within_tolerance(y, ref, inp.dtype, "%s/%s (near-tie flips %d)" % (name, pname, flips))


@pytest.mark.parametrize("name", list(CASES))
def test_fused_and_unfused_are_bit_identical(name, built):
    inp, _, dev = built(name)
    for pname, pflag in _paths(inp):
        y_f, t_f = _run(dev, pflag)
        y_u, t_u = _run(dev, pflag | moe.FLAG_UNFUSED)
        y_s, t_s = _run(dev, pflag, fused_tensor=False)  # separate gate/up tensors
        ku = int(t_f["k_used"][0])
        valid = (np.arange(inp.T * inp.kcap) % inp.kcap) < ku
        assert np.array_equal(y_f, y_u), "%s/%s fused vs unfused y" % (name, pname)
        assert np.array_equal(y_f, y_s), "%s/%s fused tensor vs separate tensors y" % (name, pname)
        hf = t_f["h"].view(np.uint16)[valid]
        assert np.array_equal(hf, t_u["h"].view(np.uint16)[valid]), "%s/%s SwiGLU rows" % (name, pname)
        assert np.array_equal(hf, t_s["h"].view(np.uint16)[valid])
        # the fp32 gate+up sums themselves, before SwiGLU and its fp16 rounding
        # (oMLX gate/up page, how correctness is verified: fused == separate)
        pf = t_f["gate_up_preact"].view(np.uint32)[valid]
        assert np.array_equal(pf, t_u["gate_up_preact"].view(np.uint32)[valid]), "%s/%s gate_up preact" % (name,
                                                                                                         pname)
        assert np.array_equal(pf, t_s["gate_up_preact"].view(np.uint32)[valid])
        # the tap holds the values the SwiGLU rows were formed from
        g = t_f["gate_up_preact"][valid][:, :inp.I].astype(np.float64)
        u = t_f["gate_up_preact"][valid][:, inp.I:].astype(np.float64)
        with np.errstate(over="ignore"):
            h_host = (g / (1.0 + np.exp(-g)) * u).astype(np.float16).astype(np.float64)
        h_gpu = t_f["h"][valid].astype(np.float64)
        ulp = np.spacing(np.abs(h_host).astype(np.float16)).astype(np.float64)
        assert np.all(np.abs(h_gpu - h_host) <= ulp + 1e-7), "%s/%s preact vs h" % (name, pname)


@pytest.mark.parametrize("name", ["tiny", "prefill_small", "batched_small", "entropy_q4", "ragged_shapes",
                                  "prefill_bm128", "k8_e256", "ragged_mfma_router", "batched_e256"])
def test_sort_matches_oracle_exactly(name, built):
    inp, _, dev = built(name)
    _, taps = _run(dev, moe.FLAG_FORCE_MFMA)
    ku = int(taps["k_used"][0])
    counts, offsets, perm, pos = oracle.sort_pairs(taps["topk_idx"], ku, inp.E)
    assert np.array_equal(taps["counts"], counts)
    assert np.array_equal(taps["offsets"], offsets)
    assert np.array_equal(taps["perm"], perm)


# (row tile, K groups per stage, N subtiles per wave, waves per column block,
# workgroups per CU): every launch shape of one k split accumulates each
# output over K in the same order, so the shapes of a split give identical
# bits; the two splits are compared with each other within the layer tolerance
GEMM_SHAPES = [(32, 2, 2, 1, 2), (32, 2, 2, 1, 1), (32, 2, 2, 2, 1), (32, 1, 2, 2, 1), (64, 1, 2, 1, 2), (64, 1, 2, 1, 3), (64, 2, 2, 1, 1), (64, 2, 2, 2, 2),
               (64, 1, 2, 2, 2), (128, 1, 2, 1, 2), (128, 2, 2, 1, 2), (128, 2, 4, 1, 2), (128, 1, 2, 2, 2),
               (128, 2, 2, 2, 2)]
DEFAULT_TUNING = {2: 1 << 30, 3: 1, 4: 2, 5: 2, 6: 1, 7: 8}


@pytest.mark.parametrize("name", ["prefill_bm128", "prefill_small", "tiny_q8_bf16", "tiny_fp16w", "batched_long_k",
                                  "prefill_f4_bm128"])
def test_gemm_launch_shapes_are_bit_identical(name, built):
    from ref64 import half64
    inp, _, dev = built(name)
    first = {}
    # the same weights with packed codes (and scales): every shape gives the same bits
    gu_p = moe.pack_q(dev.gate_up)
    dn_p = moe.pack_q(dev.down)
    if inp.bits != 16:
        gu_p, dn_p = moe.pack_sb(gu_p), moe.pack_sb(dn_p)
    try:
        for bm, kg, nsub, ks, wpc in GEMM_SHAPES:
            print("case", name, "bm", bm, "kg", kg, "nsub", nsub, "ksplit", ks, "wpc", wpc, flush=True)
            moe.debug_set_tuning(7, wpc)
            moe.debug_set_tuning(3, bm)
            moe.debug_set_tuning(4, kg)
            moe.debug_set_tuning(5, nsub)
            moe.debug_set_tuning(6, ks)
            moe.debug_set_tuning(2, 2)  # short row groups: exercises the grouped tile order
            y, _ = _run(dev, moe.FLAG_FORCE_MFMA)
            yp = host_bits(moe.layer_forward(dev.x, dev.wr, inp.k, dn_p, gate_up=gu_p, flags=moe.FLAG_FORCE_MFMA))
            torch.cuda.synchronize()
            assert np.array_equal(yp, y), "packed codes, bm %d kg %d nsub %d ksplit %d" % (bm, kg, nsub, ks)
            split = ks
            if split in first:
                assert np.array_equal(y, first[split]), "%s bm %d kg %d nsub %d ksplit %d" % (name, bm, kg, nsub, ks)
            else:
                first[split] = y
    finally:
        for key, v in DEFAULT_TUNING.items():
            moe.debug_set_tuning(key, v)
    # the two k splits differ only in fp32 summation order
    a, b = half64(first[1], inp.dtype), half64(first[2], inp.dtype)
    assert np.max(np.abs(a - b)) <= 2e-2
    assert np.linalg.norm(a - b) <= 5e-3 * np.linalg.norm(a)


def _packed_reference(w):
    """packed_sb layout written out with numpy from the host copies."""
    if w.fmt == "nvfp4":
        # the four block-scale bytes of groups 2p and 2p+1 (0 if none), as words
        E, N, nb = w.scales.shape
        ng = nb // 4
        words = np.ascontiguousarray(w.scales).view(np.uint32)  # [E, N, ng]
        if ng % 2:
            words = np.concatenate([words, np.zeros((E, N, 1), np.uint32)], axis=2)
        out = np.zeros((E, (ng + 1) // 2, N, 2), np.uint32)
        out[..., 0] = words[:, :, 0::2].transpose(0, 2, 1)
        out[..., 1] = words[:, :, 1::2].transpose(0, 2, 1)
        return out.view(np.uint16)
    E, N, ng = w.scales.shape
    NP = (ng + 1) // 2
    pad = lambda a: np.concatenate([a, np.zeros((E, N, 1), np.uint16)], axis=2) if ng % 2 else a
    s, b = pad(w.scales), pad(w.biases)
    out = np.zeros((E, NP, N, 4), np.uint16)
    out[..., 0] = s[:, :, 0::2].transpose(0, 2, 1)
    out[..., 1] = s[:, :, 1::2].transpose(0, 2, 1)
    out[..., 2] = b[:, :, 0::2].transpose(0, 2, 1)
    out[..., 3] = b[:, :, 1::2].transpose(0, 2, 1)
    return out


@pytest.mark.parametrize("name", ["prefill_small", "tiny_q8_bf16", "ragged_shapes", "entropy_q4", "batched_q5",
                                  "batched_q6", "batched_f4", "entropy_f4"])
def test_packed_sb_layout_and_bit_identity(name, built):
    inp, gu_np, dev = built(name)
    down = moe.pack_sb(dev.down)
    gate_up = moe.pack_sb(dev.gate_up)
    torch.cuda.synchronize()
    E, N, ng = inp.down.scales.shape
    if inp.fmt == "nvfp4":
        ng //= 4  # four block scales per group
    got = down.packed_sb.cpu().numpy().view(np.uint16).reshape(E, (ng + 1) // 2, N, 4)
    assert np.array_equal(got, _packed_reference(inp.down))
    got = gate_up.packed_sb.cpu().numpy().view(np.uint16).reshape(E, -1, 2 * inp.I, 4)
    assert np.array_equal(got, _packed_reference(gu_np))
    # the batched path gives the same bits whether it repacks per call or not
    for flags in (moe.FLAG_FORCE_MFMA, moe.FLAG_FORCE_MFMA | moe.FLAG_UNFUSED):
        y0 = host_bits(dev.forward(flags=flags))
        y1 = moe.layer_forward(dev.x, dev.wr, inp.k, down, gate_up=gate_up, flags=flags)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(y1), y0), flags


def _packed_q_reference(w):
    """packed_q layout written out with numpy from the host copies: [E, NB, NU, 32, PB] bytes."""
    q = np.ascontiguousarray(w.q).view(np.uint8).reshape(w.E, w.N, -1)
    ug = 1 if w.bits in (6, 16) else 2  # groups per unit
    pb = 8 * w.bits * ug
    nu = (w.K + 64 * ug - 1) // (64 * ug)
    padded = np.zeros((w.E, w.N, nu * pb), np.uint8)
    padded[:, :, :q.shape[2]] = q
    return padded.reshape(w.E, w.N // 32, 32, nu, pb).transpose(0, 1, 3, 2, 4)


@pytest.mark.parametrize("name", ["prefill_small", "tiny_q8_bf16", "tiny_fp16w", "batched_q5", "batched_q6",
                                  "batched_f4", "entropy_q4", "batched_small", "entropy_fp16w", "prefill_q6_bm128"])
def test_packed_q_layout_and_bit_identity(name, built):
    inp, gu_np, dev = built(name)
    down = moe.pack_q(dev.down)
    gate_up = moe.pack_q(dev.gate_up)
    torch.cuda.synchronize()
    got = down.packed_q.cpu().numpy().reshape(_packed_q_reference(inp.down).shape)
    assert np.array_equal(got, _packed_q_reference(inp.down))
    got = gate_up.packed_q.cpu().numpy().reshape(_packed_q_reference(gu_np).shape)
    assert np.array_equal(got, _packed_q_reference(gu_np))
    # separate gate and up tensors, each with its own packed codes
    gate, up = moe.pack_q(dev.gate), moe.pack_q(dev.up)
    for flags in (moe.FLAG_FORCE_MFMA, moe.FLAG_FORCE_MFMA | moe.FLAG_UNFUSED):
        y0 = host_bits(dev.forward(flags=flags))
        y1 = host_bits(moe.layer_forward(dev.x, dev.wr, inp.k, down, gate_up=gate_up, flags=flags))
        y2 = host_bits(moe.layer_forward(dev.x, dev.wr, inp.k, down, gate=gate, up=up, flags=flags))
        torch.cuda.synchronize()
        assert np.array_equal(y1, y0), flags
        assert np.array_equal(y2, y0), flags


def test_five_bit_batched_path_needs_multiples_of_128(built):
    # two-group (80-byte) stages: inter 704 is 11 groups
    inp, _, dev = built("decode_q5")
    with pytest.raises(moe.MoeError) as e:
        dev.forward(flags=moe.FLAG_FORCE_MFMA)
    assert e.value.name == "MOE_ERR_QUANT"
    # 5-bit rows longer than the decode kernels take, and 8256 columns: refused
    inp = mi.make_inputs("decode_b1", T=1, H=8256, E=4, k=2, I=128, bits=5)
    with pytest.raises(moe.MoeError) as e:
        Dev(inp).forward(flags=moe.FLAG_FORCE_GEMV)
    assert e.value.name == "MOE_ERR_QUANT"


@pytest.mark.parametrize("bits,H,I,k,plan", [
    (6, 8192, 128, 2, "gemm_gate_up_swiglu"),     # hidden beyond the decode layout: the batched path
    (5, 8320, 256, 2, "gemm_gate_up_swiglu"),
    (6, 256, 6208, 2, "gemv_down_combine"),       # down rows of 7 chunks per lane: four waves per slot
    (5, 256, 12352, 4, "gemv_down_combine"),
    (6, 1024, 11008, 4, "gemv_down_combine"),     # the decode shape's inter with 6-bit codes
    (8, 512, 11008, 4, "gemv_down_combine"),
])
def test_long_rows_take_the_path_that_holds_them(bits, H, I, k, plan):
    inp = mi.make_inputs("decode_b1", T=1, H=H, E=4 if k == 2 else 8, k=k, I=I, bits=bits)
    print("case bits=%d H=%d I=%d k=%d" % (bits, H, I, k), flush=True)
    dev = Dev(inp)
    gu_np = oracle.fuse_gate_up(inp.gate, inp.up)
    taps = moe.make_taps(inp.T, inp.E, inp.k, inp.I, "cuda")
    y = host_bits(dev.forward(taps=taps))
    assert plan in moe.last_plan()
    t = {n: v.cpu().numpy() for n, v in taps.items()}
    ku = int(t["k_used"][0])
    check_routing_identical_logits(t["logits"], t["topk_idx"], t["topk_w"], ku)
    ref, flips = reference_outputs(inp, gu_np, np.arange(inp.T), t["topk_idx"], t["topk_w"], ku)
    assert_within_tolerance(y, ref, inp.dtype, "bits %d H %d I %d" % (bits, H, I))
    y_u = host_bits(dev.forward(flags=moe.FLAG_UNFUSED))
    assert np.array_equal(y, y_u)


def test_runs_are_deterministic(built):
    inp, _, dev = built("prefill_small")
    a, _ = _run(dev, 0)
    b, _ = _run(dev, 0)
    c, _ = _run(dev, moe.FLAG_UNFUSED)
    assert np.array_equal(a, b) and np.array_equal(a, c)


def test_token_permutation_equivariance(built):
    inp, _, dev = built("prefill_small")
    y, _ = _run(dev, 0)
    perm = np.random.default_rng(4).permutation(inp.T)
    xp = dev.x[torch.from_numpy(perm).cuda()].contiguous()
    y2 = host_bits(dev.forward(x=xp))
    assert np.array_equal(y2, y[perm])


def test_fuse_gate_up_matches_oracle_concatenation(built):
    for name in ("tiny", "tiny_q8_bf16", "tiny_fp16w", "decode_f4"):
        inp, gu_np, dev = built(name)
        if inp.bits == 16:
            assert np.array_equal(host_bits(dev.gate_up.q), gu_np.q)
        elif inp.fmt == "nvfp4":
            assert np.array_equal(dev.gate_up.q.cpu().numpy(), gu_np.q)
            assert np.array_equal(dev.gate_up.scales.cpu().numpy(), gu_np.scales)
            assert dev.gate_up.biases is None and dev.gate_up.tensor_scale == gu_np.tensor_scale
        else:
            assert np.array_equal(dev.gate_up.q.cpu().numpy(), gu_np.q)
            assert np.array_equal(host_bits(dev.gate_up.scales), gu_np.scales)
            assert np.array_equal(host_bits(dev.gate_up.biases), gu_np.biases)


# ------------------------------------------------------------------ router --

@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("T,E,k", [(1, 64, 4), (7, 8, 2), (300, 64, 4), (64, 256, 8), (33, 32, -1),
                                   (300, 32, -1), (200, 8, 2), (129, 256, 8), (300, 20, 2), (90, 45, 3),
                                   (400, 40, 2), (4096, 64, 4)])
def test_router_exact_inputs_with_planted_ties(dtype, T, E, k):
    # H = 1024 takes the sixteen-wave MFMA router above 128 tokens and 16384
    # logits (H = 2048: one whole round of eight k-steps per wave); H = 320
    # (not a multiple of 256) the four-wave one, as do 256 tiles or more
    # (4096 tokens x 64 experts); H = 8192 runs
    # the small-batch router's four-slice rounds (partial sums stay exact:
    # multiples of 2^-14 below 2^9).  The small-batch router takes 1, 2, 4 or 8
    # experts per workgroup as T*E grows (E = 20, 45 and 40: a partial last
    # block)
    for H in (1024, 320) + ((8192,) if T <= 128 else (2048,)):
        _router_exact_case(dtype, T, E, k, H)


def _router_exact_case(dtype, T, E, k, H):
    x, wr = mi.exact_router_inputs(7, T, H, E, dtype)
    wr = wr.copy()
    wr[E - 1] = wr[0]  # duplicated rows: identical logits, lower index must win
    wr[E // 2] = wr[1]
    r = moe.route(dev_half(x, dtype), dev_half(wr, dtype), k, want_logits=True)
    torch.cuda.synchronize()
    logits = r["logits"].cpu().numpy()
    assert np.array_equal(logits, oracle.router_logits(x, wr, dtype)), "exact-arithmetic logits differ"
    idx_o, w_o, ku_o, hm_o = oracle.route(x, wr, dtype, k)
    assert int(r["k_used"].item()) == ku_o
    assert np.array_equal(r["idx"].cpu().numpy(), idx_o)
    assert np.max(np.abs(r["w"].cpu().numpy() - w_o)) <= 1e-6


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("T,E,H", [(512, 32, 4096), (130, 64, 1024), (401, 40, 2048), (97, 100, 512)])
def test_router_tokens_per_workgroup_bit_identical(dtype, T, E, H):
    # the small-batch router at eight experts per workgroup, with one, two or
    # four tokens per workgroup: each logit is summed in the same order, so the
    # bits agree (T not a multiple of 4 and E not of 8: partial last blocks),
    # with and without the load-aware correction
    rng = np.random.default_rng(T * E)
    xs = (rng.standard_normal((T, H))).astype(np.float32)
    ws = (rng.standard_normal((E, H)) * 0.02).astype(np.float32)
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    xd, wd = torch.from_numpy(xs).to(tdt).cuda(), torch.from_numpy(ws).to(tdt).cuda()
    hv = torch.from_numpy(rng.random(E).astype(np.float32)).cuda()
    try:
        for health in (None, hv):
            got = {}
            for tb in (1, 2, 4):
                moe.debug_set_tuning(9, tb)
                r = moe.route(xd, wd, 4, want_logits=True, health=health, alpha=0.5 if health is not None else 0.0)
                torch.cuda.synchronize()
                got[tb] = r["logits"].cpu().numpy().view(np.uint32)
            assert np.array_equal(got[1], got[2]) and np.array_equal(got[1], got[4])
    finally:
        moe.debug_set_tuning(9, 2)


@pytest.mark.parametrize("E,k", [(8, 1), (64, 4), (256, 8), (32, -1)])
def test_topk_from_identical_logits(E, k):
    rng = np.random.default_rng(E)
    logits = (rng.standard_normal((200, E)) * 1.5).astype(np.float32)
    logits[:50, 3] = logits[:50, 1]  # ties
    logits[50:60] = 0.25  # all equal
    r = moe.topk_from_logits(torch.from_numpy(logits).cuda(), k)
    torch.cuda.synchronize()
    ku = int(r["k_used"].item())
    if k > 0:
        assert ku == k
    else:
        assert ku == oracle.entropy_k(oracle.batch_entropy(logits))
    check_routing_identical_logits(logits, r["idx"].cpu().numpy(), r["w"].cpu().numpy(), ku)


@pytest.mark.parametrize("m,k", [(1, 1), (3, 1), (4, 2), (12, 2), (13, 3), (32, 3)])
def test_entropy_closed_form_on_gpu(m, k):
    l = np.full((64, 32), -40.0, np.float32)
    l[:, :m] = 0.5
    for t in range(64):
        l[t] = np.roll(l[t], t)
    r = moe.topk_from_logits(torch.from_numpy(l).cuda(), moe.MOE_K_ENTROPY)
    torch.cuda.synchronize()
    assert int(r["k_used"].item()) == k
    assert abs(float(r["entropy"].item()) - np.log(m)) < 1e-5
    idx = r["idx"].cpu().numpy()
    assert np.all(idx[:, k:] == -1)
    assert np.all(r["w"].cpu().numpy()[:, k:] == 0)


def test_router_realistic_logits_within_bound():
    inp = mi.make_inputs("prefill", T=512, E=64, H=4096, I=64)
    r = moe.route(dev_half(inp.x, "bf16"), dev_half(inp.wr, "bf16"), 4, want_logits=True)
    torch.cuda.synchronize()
    got = r["logits"].cpu().numpy().astype(np.float64)
    from ref64 import half64
    x64, w64 = half64(inp.x, "bf16"), half64(inp.wr, "bf16")
    want = x64 @ w64.T
    n = 4096
    gamma = n * 2.0 ** -24 / (1 - n * 2.0 ** -24)
    assert np.all(np.abs(got - want) <= gamma * (np.abs(x64) @ np.abs(w64).T))
    check_routing_identical_logits(got.astype(np.float32), r["idx"].cpu().numpy(), r["w"].cpu().numpy(), 4)


def test_zero_tokens_and_errors_on_gpu():
    inp = mi.make_inputs("tiny")
    dev = Dev(inp)
    y = moe.layer_forward(dev.x[:0], dev.wr, 2, dev.down, gate_up=dev.gate_up)
    assert y.shape[0] == 0
    with pytest.raises(moe.MoeError) as e:
        moe.layer_forward(dev.x, dev.wr, 9, dev.down, gate_up=dev.gate_up)
    assert e.value.name == "MOE_ERR_K"



def _token_exponent(x_bits_row: np.ndarray) -> int:
    """The scale exponent a_t the library takes for a bf16 token: the smallest
    a >= 0 with max|x| * 2^-a < 64 (include/moe.h, Arithmetic)."""
    e = int((np.max(x_bits_row & 0x7FFF) >> 7))
    return max(0, e - 132)


@pytest.mark.parametrize("nbytes", [16, 4096, 8 << 20, (37 << 20) + 48])
def test_stream_read_reads_every_word_once(nbytes):
    # the measurement reference's sink XORs fold to the XOR of the buffer
    g = torch.Generator().manual_seed(nbytes % 1000003)
    src = torch.randint(-2 ** 31, 2 ** 31 - 1, (nbytes // 4,), dtype=torch.int32, generator=g)
    sink = moe.debug_stream_read(src.cuda())
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(src.numpy().view(np.uint32))
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == want


@pytest.mark.parametrize("recipe,kw,flag", [
    ("batched_decode", dict(T=40, H=512, E=8, I=320), moe.FLAG_FORCE_MFMA),   # 8-bit, batched path
    ("prefill", dict(T=300, H=512, E=16, I=192), moe.FLAG_FORCE_MFMA),        # 4-bit, batched path
    ("batched_decode", dict(T=6, H=512, E=8, I=320), moe.FLAG_FORCE_GEMV),    # 8-bit, decode path
    ("prefill", dict(T=4, H=512, E=16, I=192), moe.FLAG_FORCE_GEMV),          # 4-bit, decode path
    ("prefill", dict(T=300, H=512, E=16, I=192, fmt="nvfp4"), moe.FLAG_FORCE_MFMA),  # NVFP4, batched path
    ("prefill", dict(T=4, H=512, E=16, I=192, fmt="nvfp4"), moe.FLAG_FORCE_GEMV),    # NVFP4, decode path
])
def test_bf16_activations_beyond_fp16_range(recipe, kw, flag):
    # rows of bf16 activations scaled near 1e5 (beyond fp16's 65504) and one
    # row with a single element of 2e5: the layer keeps bf16's range
    inp = mi.make_inputs(recipe, dtype="bf16", **kw)
    x = half64(inp.x, "bf16")
    big = {1: 1e5, 3: 3e4}
    for t, c in big.items():
        x[t] *= c
    x[2, 7] = 2e5
    import dataclasses
    inp = dataclasses.replace(inp, x=mi.round_half(x, "bf16"))
    a = np.array([_token_exponent(inp.x[t]) for t in range(inp.T)])
    print("token exponents", a[:6].tolist(), flush=True)
    assert a[1] > 0 and a[3] > 0 and a[2] > 0 and a[0] == 0
    dev = Dev(inp)
    gu_np = oracle.fuse_gate_up(inp.gate, inp.up)
    taps = moe.make_taps(inp.T, inp.E, inp.k, inp.I, "cuda")
    yb = host_bits(dev.forward(flags=flag, taps=taps))
    t = {n: v.cpu().numpy() for n, v in taps.items()}
    ku = int(t["k_used"][0])
    check_routing_identical_logits(t["logits"], t["topk_idx"], t["topk_w"], ku)
    ref, _ = reference_outputs(inp, gu_np, np.arange(inp.T), t["topk_idx"], t["topk_w"], ku)
    y = half64(yb, "bf16")
    assert np.all(np.isfinite(y)), "non-finite output"
    assert np.all(np.isfinite(t["h"].astype(np.float64)))
    normal = a == 0
    # tokens at unit scale: the usual bars
    assert_within_tolerance(yb[normal], ref[normal], "bf16", "bf16 unscaled tokens")
    # scaled tokens: the same bars on the output in units of its rms
    for tk in np.where(~normal)[0]:
        r = ref[tk].astype(np.float64)
        rms = float(np.sqrt(np.mean(r * r)))
        d = (y[tk] - r) / rms
        rel = float(np.linalg.norm(y[tk] - r) / np.linalg.norm(r))
        print("token %d a=%d rms %.3g: max_abs/rms %.3g rel_l2 %.3g" % (tk, a[tk], rms, np.max(np.abs(d)), rel),
              flush=True)
        assert np.max(np.abs(d)) <= 2e-2 and rel <= 5e-3, tk
    # fused == unfused still holds bit for bit
    y_u = host_bits(dev.forward(flags=flag | moe.FLAG_UNFUSED))
    assert np.array_equal(yb, y_u)
