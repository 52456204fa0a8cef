"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test ties one oracle function to something other than itself: hand-worked
values (tests/golden), closed forms, fp64 brute force, library routines on
special cases, or invariants.  Together they are chosen so that a plausible
slip (a dropped term, a wrong sign, a swapped operand, the wrong nibble, the
wrong tie-break, the wrong logarithm) fails at least one.
"""
import math

import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from conftest import golden_path
from ref64 import dense_layer64, dequant64, e4m3_64, entropy64, half64, rel_l2, select64, silu64

U = 2.0 ** -24  # unit roundoff of fp32


# ------------------------------------------------------------ rounding --

def test_half_encode_matches_numpy_and_torch():
    rng = np.random.default_rng(0)
    vals = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * 3,
        (rng.standard_normal(5000) * 1e-6).astype(np.float32),  # fp16 subnormals
        np.float32([0.0, -0.0, 65504, 65519.99, 65520, 1e6, -1e6, 2 ** -24, 2 ** -25, 3 * 2 ** -26,
                    1 + 2 ** -11, 1 + 3 * 2 ** -11, 1 + 2 ** -8, 1 + 3 * 2 ** -8]),
    ]).astype(np.float32)
    with np.errstate(over="ignore"):
        want16 = vals.astype(np.float16).view(np.uint16)
    want_bf = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got16 = np.array([oracle.float_to_half(v, "f16") for v in vals], np.uint16)
    gotbf = np.array([oracle.float_to_half(v, "bf16") for v in vals], np.uint16)
    assert np.array_equal(got16, want16)
    assert np.array_equal(gotbf, want_bf)


def test_half_decode_matches_numpy():
    allbits = np.arange(0, 65536, 7, dtype=np.uint16)
    finite = np.isfinite(allbits.view(np.float16))
    got = np.array([oracle.half_to_float(b, "f16") for b in allbits[finite]], np.float64)
    assert np.array_equal(got, allbits[finite].view(np.float16).astype(np.float64))
    got_bf = np.array([oracle.half_to_float(b, "bf16") for b in allbits[:2000]], np.float64)
    assert np.array_equal(got_bf, half64(allbits[:2000], "bf16"))


def test_round_output_matches_numpy():
    y = (np.random.default_rng(1).standard_normal(4096) * 5).astype(np.float32)
    assert np.array_equal(oracle.round_output(y, "f16"), y.astype(np.float16).view(np.uint16))
    bf = torch.from_numpy(y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.round_output(y, "bf16"), bf)


# ------------------------------------------------------------- dequant --

def _read_dequant_cases():
    cases, cur = [], None
    for line in open(golden_path("dequant_groups.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        tag, *rest = line.split()
        if tag == "case":
            cur = dict(name=rest[0], bits=int(rest[1]), s=int(rest[2], 16), b=int(rest[3], 16))
            cases.append(cur)
        elif tag == "codes":
            cur["codes"] = [int(v) for v in rest]
        elif tag == "expect":
            cur["expect"] = [float(v) for v in rest]
    return cases


@pytest.mark.parametrize("case", _read_dequant_cases(), ids=lambda c: c["name"])
def test_dequant_golden(case):
    codes = np.array(case["codes"], np.uint8)
    if case["bits"] == 4:
        q = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)  # even column -> low nibble
    elif case["bits"] in (5, 6):
        # the bits of each code, least significant first, as one little-endian stream
        nb = case["bits"]
        stream = ((codes[:, None].astype(np.int64) >> np.arange(nb)) & 1).astype(np.uint8).ravel()
        q = np.packbits(stream, bitorder="little")
    else:
        q = codes
    got = oracle.dequant_row(q, np.array([case["s"]], np.uint16), np.array([case["b"]], np.uint16), 64,
                             case["bits"])
    assert np.array_equal(got, np.array(case["expect"], np.float32))


@pytest.mark.parametrize("bits", [4, 5, 6, 8])
def test_dequant_requantize_returns_same_codes(bits):
    w = mi.quant_weights(77, 2, 2, 8, 256, bits)
    deq = oracle.dequant(w)  # fp32
    q2, s2, b2 = mi.quantize_rows(deq.reshape(-1, 256).astype(np.float64), bits)
    assert np.array_equal(q2.reshape(w.q.shape), w.q)
    assert np.array_equal(s2.reshape(w.scales.shape), w.scales)
    assert np.array_equal(b2.reshape(w.biases.shape), w.biases)


@pytest.mark.parametrize("bits", [4, 5, 6, 8, 16])
def test_dequant_matches_fp64_statement(bits):
    w = mi.quant_weights(5, 3, 2, 16, 192, bits)
    got = oracle.dequant(w).astype(np.float64)
    want = dequant64(w)
    # two fp32 roundings of s*q + b
    assert np.all(np.abs(got - want) <= 2 * U * (np.abs(want) + 1e-3))


# --------------------------------------------------------------- NVFP4 --

def test_e4m3_decode_matches_torch_float8_e4m3fn():
    got = np.array([oracle.e4m3_to_float(b) for b in range(256)], np.float64)
    want = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2  # 0x7F and 0xFF
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def test_e2m1_decode_is_the_published_table():
    # NVFP4 element values, NVIDIA's format definition: codes 0..7 are
    # 0, 0.5, 1, 1.5, 2, 3, 4, 6; bit 3 is the sign
    table = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]
    got = [oracle.e2m1_to_float(c) for c in range(16)]
    assert got == table
    assert [math.copysign(1, g) for g in got] == [math.copysign(1, v) for v in table]


def _read_nvfp4_cases():
    cases, cur = [], None
    for line in open(golden_path("nvfp4_blocks.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        tag, *rest = line.split()
        if tag == "case":
            cur = dict(name=rest[0], ts=float(rest[1]), s=[int(v, 16) for v in rest[2:6]])
            cases.append(cur)
        elif tag == "codes":
            cur["codes"] = [int(v, 16) for v in rest]
        elif tag == "expect":
            cur["expect"] = [float(v) for v in rest]
    return cases


@pytest.mark.parametrize("case", _read_nvfp4_cases(), ids=lambda c: c["name"])
def test_nvfp4_dequant_golden(case):
    codes = np.array(case["codes"], np.uint8)
    q = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)  # even column -> low nibble
    got = oracle.dequant_row(q, np.array(case["s"], np.uint8), None, 64, oracle.NVFP4, 16, case["ts"])
    assert np.array_equal(got, np.array(case["expect"], np.float32))


def test_nvfp4_requantize_returns_same_codes():
    w = mi.nvfp4_weights(77, 2, 2, 8, 256)
    deq = oracle.dequant(w)
    q2, s2, ts = mi.quantize_rows_nvfp4(deq.reshape(-1, 256).astype(np.float64), ts=w.tensor_scale)
    assert np.array_equal(q2.reshape(w.q.shape), w.q)
    assert np.array_equal(s2.reshape(w.scales.shape), w.scales)


def test_nvfp4_dequant_matches_fp64_statement():
    w = mi.nvfp4_weights(5, 3, 2, 16, 192)
    got = oracle.dequant(w).astype(np.float64)
    want = dequant64(w)
    # two fp32 roundings: ts * s, then times the E2M1 value
    assert np.all(np.abs(got - want) <= 2 * U * np.abs(want))
    # every block uses its own scale: the largest code of a block is +-6
    assert np.all(np.abs(want).reshape(2, 16, 12, 16).max(-1) > 0)


def test_nvfp4_quantiser_error_within_half_a_step():
    # the generator's quantiser rounds to the nearest E2M1 value of each
    # block's grid: the error is at most half the largest gap (2 steps)
    rng = np.random.default_rng(4)
    w64 = rng.standard_normal((6, 128)) * 0.02
    q, s, ts = mi.quantize_rows_nvfp4(w64)
    back = np.stack([oracle.dequant_row(q[r], s[r], None, 128, oracle.NVFP4, 16, ts) for r in range(6)])
    step = ts * np.repeat(e4m3_64(s), 16, axis=-1)
    assert np.all(np.abs(back - w64) <= step * 1.0 + 1e-9)


# -------------------------------------------------------------- router --

def test_router_logits_within_higham_bound():
    x = mi.normal_half(9, 0, 16 * 1024, 1.0, "f16").reshape(16, 1024)
    wr = mi.normal_half(9, 1, 24 * 1024, 0.02, "f16").reshape(24, 1024)
    got = oracle.router_logits(x, wr, "f16").astype(np.float64)
    x64, w64 = half64(x, "f16"), half64(wr, "f16")
    want = x64 @ w64.T
    n = 1024
    gamma = n * U / (1 - n * U)
    bound = gamma * (np.abs(x64) @ np.abs(w64).T)
    assert np.all(np.abs(got - want) <= bound)
    assert np.max(np.abs(got - want)) > 0  # the bound is not vacuous


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_router_logits_exact_on_exact_inputs(dtype):
    x, wr = mi.exact_router_inputs(3, 8, 2048, 16, dtype)
    got = oracle.router_logits(x, wr, dtype)
    want = half64(x, dtype) @ half64(wr, dtype).T
    assert np.array_equal(got.astype(np.float64), want)


def _read_router_worked():
    d = {"wr": []}
    for line in open(golden_path("router_worked.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        tag, *rest = line.split()
        vals = [float(v) for v in rest]
        if tag == "wr":
            d["wr"].append(vals)
        else:
            d[tag] = vals
    return d


def test_router_worked_example():
    d = _read_router_worked()
    x = mi.round_half(np.array([d["x"]]), "f16")
    wr = mi.round_half(np.array(d["wr"]), "f16")
    idx, w, ku, _, logits = oracle.route(x, wr, "f16", 2, want_logits=True)
    assert np.array_equal(logits[0], np.float32(d["logits"]))
    assert idx[0].tolist() == [int(v) for v in d["idx"]]
    assert np.allclose(w[0], d["w"], rtol=0, atol=2e-7)
    assert ku == 2


# ------------------------------------------------------------ selection --

@pytest.mark.parametrize("E,k", [(8, 1), (8, 2), (32, 2), (32, 3), (64, 4), (64, 8), (256, 8)])
def test_selection_brute_force(E, k):
    rng = np.random.default_rng(E * 10 + k)
    logits = (rng.standard_normal((64, E)) * 1.3).astype(np.float32)
    # planted ties: duplicate some logits inside rows
    logits[:16, 1] = logits[:16, 0]
    logits[16:32, E - 1] = logits[16:32, 2]
    idx, w = oracle.select_topk(logits, k)
    for t in range(64):
        order = sorted(range(E), key=lambda e: (-float(logits[t, e]), e))
        assert idx[t].tolist() == order[:k]


def test_selection_matches_torch_topk_without_ties():
    rng = np.random.default_rng(5)
    logits = rng.permutation(np.arange(64 * 64, dtype=np.float32)).reshape(64, 64) / 97.0
    idx, _ = oracle.select_topk(logits, 4)
    tv, ti = torch.topk(torch.softmax(torch.from_numpy(logits).double(), -1), 4, dim=-1)
    assert np.array_equal(idx, ti.numpy().astype(np.int32))


def test_ties_go_to_lower_index():
    logits = np.zeros((3, 8), np.float32)
    logits[1, [5, 2, 7]] = 1.0
    logits[2, :] = [0, 3, 3, 1, 3, 0, 0, 3]
    idx, w = oracle.select_topk(logits, 3)
    assert idx.tolist() == [[0, 1, 2], [2, 5, 7], [1, 2, 4]]
    assert np.all(w[0] == np.float32(1 / 3)) or np.allclose(w[0], 1 / 3, atol=1e-7)


# -------------------------------------------------------------- weights --

def test_weights_sum_to_one_and_closed_forms():
    rng = np.random.default_rng(11)
    for k in (1, 2, 3, 4, 8):
        logits = (rng.standard_normal((256, 64)) * 2).astype(np.float32)
        _, w = oracle.select_topk(logits, k)
        s = w.astype(np.float64).sum(axis=1)
        assert np.all(np.abs(s - 1) <= (k + 2) * 2 ** -23)
        if k == 1:
            assert np.all(w == 1.0)
    # equal logits -> 1/k
    _, w = oracle.select_topk(np.full((1, 16), 0.75, np.float32), 4)
    assert np.allclose(w, 0.25, atol=1e-7)
    # two experts: w1 = 1/(1 + e^(l2 - l1))
    l = np.array([[0.3, 1.7, -2.0, -5.0]], np.float32)
    idx, w = oracle.select_topk(l, 2)
    assert idx[0].tolist() == [1, 0]
    want = 1.0 / (1.0 + math.exp(float(l[0, 0]) - float(l[0, 1])))
    assert abs(float(w[0, 0]) - want) < 3e-7
    assert abs(float(w[0, 1]) - (1 - want)) < 3e-7


def test_weights_match_fp64_renormalised_softmax():
    rng = np.random.default_rng(12)
    logits = (rng.standard_normal((128, 32)) * 1.5).astype(np.float32)
    idx, w = oracle.select_topk(logits, 3)
    i64, w64 = select64(logits.astype(np.float64), 3)
    assert np.array_equal(idx, i64)
    assert np.max(np.abs(w - w64)) < 1e-6


# -------------------------------------------------------------- entropy --

def _read_entropy_bands():
    rows = []
    for line in open(golden_path("entropy_bands.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        E, m, h, k = line.split()
        rows.append((int(E), int(m), float(h), int(k)))
    return rows


@pytest.mark.parametrize("E,m,h,k", _read_entropy_bands())
def test_entropy_closed_form_bands(E, m, h, k):
    l = np.full((4, E), -40.0, np.float32)
    l[:, :m] = 0.0
    l[1] = np.roll(l[1], 3)
    l += np.float32(1.25)  # a common shift changes nothing
    tol = 4 * E * U * max(1.0, h) + 1e-6  # fp32 sums over E terms
    assert abs(oracle.token_entropy(l[0]) - h) < tol
    hm = oracle.batch_entropy(l)
    assert abs(hm - h) < tol
    assert oracle.entropy_k(hm) == k


def test_entropy_thresholds_inclusive_as_printed():
    assert oracle.entropy_k(np.nextafter(np.float32(1.2), np.float32(0))) == 1
    assert oracle.entropy_k(1.2) == 2
    assert oracle.entropy_k(np.nextafter(np.float32(2.5), np.float32(0))) == 2
    assert oracle.entropy_k(2.5) == 3


def test_entropy_matches_fp64_and_is_natural_log():
    rng = np.random.default_rng(13)
    l = (rng.standard_normal((64, 32)) * 1.7).astype(np.float32)
    want = entropy64(l.astype(np.float64))
    got = np.array([oracle.token_entropy(r) for r in l])
    assert np.max(np.abs(got - want)) < 1e-5
    # uniform distribution: ln E, not log2 E
    assert abs(oracle.token_entropy(np.zeros(32, np.float32)) - math.log(32)) < 2e-6


def test_entropy_route_truncates_to_k_used():
    # logits with 3 dominant experts per token -> H = ln 3 < 1.2 -> k = 1
    E, H = 8, 64
    x = mi.round_half(np.eye(4, H) * 4.0, "f16")
    wr64 = np.zeros((E, H))
    for t in range(4):
        for e in range(3):
            wr64[(t + e) % E, t] = 10.0
    wr = mi.round_half(wr64, "f16")
    idx, w, ku, hm = oracle.route(x, wr, "f16", -1)
    assert ku == 1 and abs(hm - math.log(3)) < 1e-5
    assert np.all(idx[:, 1:] == -1) and np.all(w[:, 1:] == 0) and np.all(w[:, 0] == 1)


# ----------------------------------------------------------------- sort --

@pytest.mark.parametrize("T,kcap,ku,E", [(1, 4, 4, 64), (37, 2, 2, 8), (128, 3, 2, 32), (513, 4, 4, 64),
                                         (64, 3, 1, 32), (16, 8, 8, 256)])
def test_sort_pairs_is_stable_counting_sort(T, kcap, ku, E):
    rng = np.random.default_rng(T + E)
    idx = rng.integers(0, E, size=(T, kcap)).astype(np.int32)
    idx[:, ku:] = -1
    counts, offsets, perm, pos = oracle.sort_pairs(idx, ku, E)
    pairs = [p for p in range(T * kcap) if p % kcap < ku]
    want = sorted(pairs, key=lambda p: (idx.flat[p], p))  # Python's sort is stable
    assert perm[:len(want)].tolist() == want
    assert np.all(perm[len(want):] == -1)
    assert counts.sum() == len(pairs)
    assert np.array_equal(np.bincount(idx[:, :ku].ravel(), minlength=E), counts)
    assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts)
    for i, p in enumerate(want):
        assert pos[p] == i
    assert all(pos[p] == -1 for p in range(T * kcap) if p % kcap >= ku)


# ------------------------------------------------------------------ FFN --

@pytest.mark.parametrize("bits", [4, 8, 16, "nvfp4"])
def test_fused_gate_up_bit_identical_to_separate(bits):
    inp = mi.make_inputs("tiny", fmt="nvfp4") if bits == "nvfp4" else mi.make_inputs("tiny", bits=bits)
    gu = oracle.fuse_gate_up(inp.gate, inp.up)
    assert gu.q.shape[1] == 2 * inp.I
    assert np.array_equal(gu.q[:, :inp.I], inp.gate.q) and np.array_equal(gu.q[:, inp.I:], inp.up.q)
    x = half64(inp.x, "f16").astype(np.float32)
    for e in range(inp.E):
        for t in range(inp.T):
            h1, o1 = oracle.expert_ffn(x[t], gu, inp.down, e)
            h2, o2 = oracle.expert_ffn_unfused(x[t], inp.gate, inp.up, inp.down, e)
            assert np.array_equal(h1.view(np.uint32), h2.view(np.uint32))
            assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32))


def _read_layer_worked():
    d = {}
    for line in open(golden_path("layer_worked.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split()
            d[k] = float(v)
    return d


def test_layer_worked_example():
    d = _read_layer_worked()
    H = I = 64

    def w_const(N, K, bias):
        q = np.zeros((1, N, K // 2), np.uint8)
        s = np.full((1, N, K // 64), 0x3800, np.uint16)
        b = np.full((1, N, K // 64), mi.round_half(np.array([bias]), "f16")[0], np.uint16)
        return mi.Weights(q, s, b, 1, N, K, 4)

    gate, up, down = w_const(I, H, 1 / 64), w_const(I, H, 2 / 64), w_const(H, I, 1 / 64)
    gu = oracle.fuse_gate_up(gate, up)
    x = mi.round_half(np.ones((1, H)), "f16")
    wr = mi.round_half(np.ones((1, H)) * 0.01, "f16")
    res = oracle.layer_forward(x, wr, "f16", 1, gu, down)
    y, hvec = oracle.tokens_forward(x, "f16", [0], res["idx"], res["w"], 1, gu, down, want_h=True)
    assert np.allclose(hvec[0, 0], d["h"], rtol=2e-7, atol=0)
    assert np.all(res["y"].view(np.float16).astype(np.float64) == d["y"])
    assert float(res["w"][0, 0]) == 1.0


def test_single_expert_is_the_textbook_swiglu_mlp():
    inp = mi.make_inputs("tiny", E=1, k=1, T=6)
    gu = oracle.fuse_gate_up(inp.gate, inp.up)
    res = oracle.layer_forward(inp.x, inp.wr, "f16", 1, gu, inp.down)
    x = half64(inp.x, "f16")
    Wg, Wu, Wd = dequant64(inp.gate)[0], dequant64(inp.up)[0], dequant64(inp.down)[0]
    want = (silu64(x @ Wg.T) * (x @ Wu.T)) @ Wd.T
    assert rel_l2(res["y_f32"], want) < 2e-6
    assert np.all(res["w"] == 1.0)


def test_all_experts_selected_is_the_dense_softmax_mixture():
    inp = mi.make_inputs("tiny", k=8)
    gu = oracle.fuse_gate_up(inp.gate, inp.up)
    res = oracle.layer_forward(inp.x, inp.wr, "f16", 8, gu, inp.down)
    x = half64(inp.x, "f16")
    logits = x @ half64(inp.wr, "f16").T
    p = np.exp(logits - logits.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    Wg, Wu, Wd = dequant64(inp.gate), dequant64(inp.up), dequant64(inp.down)
    want = sum(p[:, e:e + 1] * ((silu64(x @ Wg[e].T) * (x @ Wu[e].T)) @ Wd[e].T) for e in range(inp.E))
    assert rel_l2(res["y_f32"], want) < 2e-6


# ---------------------------------------------------------------- layer --

@pytest.mark.parametrize("kw", [
    dict(name="tiny"),
    dict(name="tiny", bits=8, dtype="bf16"),
    dict(name="tiny", bits=16, T=9),
    dict(name="tiny", k=3, E=16, T=7, H=192, I=320),
    dict(name="batched_decode", T=16, H=256, E=8, I=192),
    dict(name="prefill", T=24, H=128, E=16, I=128),
    dict(name="entropy", T=8, H=256, E=8, I=128, bits=4),
    dict(name="decode_b1", T=3, H=256, E=8, I=192, bits=6),
    dict(name="decode_b1", T=2, H=192, E=8, I=256, bits=5),
    dict(name="tiny", fmt="nvfp4"),
    dict(name="prefill", T=24, H=128, E=16, I=192, fmt="nvfp4"),
], ids=lambda kw: "-".join("%s%s" % (k, v) for k, v in kw.items()))
def test_layer_matches_dense_fp64_brute_force(kw):
    kw = dict(kw)
    inp = mi.make_inputs(kw.pop("name"), **kw)
    gu = oracle.fuse_gate_up(inp.gate, inp.up)
    res = oracle.layer_forward(inp.x, inp.wr, inp.dtype, inp.k, gu, inp.down)
    y64, idx64, w64 = dense_layer64(inp.x, inp.wr, inp.dtype, inp.k, inp.gate, inp.up, inp.down)
    ku = res["k_used"]
    assert np.array_equal(res["idx"][:, :ku], idx64)
    assert np.max(np.abs(res["w"][:, :ku] - w64)) < 1e-6
    assert rel_l2(res["y_f32"], y64) < 1e-5
    # the rounded output is the fp32 result rounded once
    assert np.array_equal(res["y"], oracle.round_output(res["y_f32"], inp.dtype))


def test_token_permutation_equivariance_is_bitwise():
    inp = mi.make_inputs("tiny", T=12, k=2)
    gu = oracle.fuse_gate_up(inp.gate, inp.up)
    res = oracle.layer_forward(inp.x, inp.wr, "f16", 2, gu, inp.down)
    perm = np.random.default_rng(3).permutation(12)
    res2 = oracle.layer_forward(np.ascontiguousarray(inp.x[perm]), inp.wr, "f16", 2, gu, inp.down)
    assert np.array_equal(res2["y"], res["y"][perm])
    assert np.array_equal(res2["idx"], res["idx"][perm])


def test_tokens_forward_matches_layer_forward_rows():
    inp = mi.make_inputs("tiny", T=10)
    gu = oracle.fuse_gate_up(inp.gate, inp.up)
    res = oracle.layer_forward(inp.x, inp.wr, "f16", 2, gu, inp.down)
    sub = oracle.tokens_forward(inp.x, "f16", [7, 2, 9], res["idx"], res["w"], 2, gu, inp.down)
    assert np.array_equal(sub, res["y_f32"][[7, 2, 9]])


# ------------------------------------- load-aware correction, groups, stats --
# Page "Qwen3.5-MoE与Qwen3-MoE架构差异深度解析", section 3.3: the final logits
# are the main logits minus alpha times the per-expert load index H.  Page
# "Qwen3.5 Block在llama.cpp中的映射与优化原理", section 1.1: 64 experts in 4
# groups of 16, the best expert of each group.  Closing advice of the first
# page: watch the least-used expert and the standard deviation of the counts.

def test_correction_worked_example():
    # one token, logits (2, 1.5, 1, 0), H = (1, 0, 0, 0).  alpha = 1 gives
    # (1, 1.5, 1, 0): top-2 is expert 1, then the tie at 1.0 goes to expert 0;
    # weights 1/(1+e^-0.5) and e^-0.5/(1+e^-0.5).  A plus sign would keep
    # (0, 1); alpha = 2 gives (0, 1.5, 1, 0) and the slots (1, 2).
    l = np.float32([[2.0, 1.5, 1.0, 0.0]])
    hv = np.float32([1.0, 0.0, 0.0, 0.0])
    c1 = oracle.correct_logits(l, hv, 1.0)
    assert np.array_equal(c1, np.float32([[1.0, 1.5, 1.0, 0.0]]))
    idx, w = oracle.select_topk(c1, 2)
    assert idx.tolist() == [[1, 0]]
    e = math.exp(-0.5)
    assert np.allclose(w[0], [1 / (1 + e), e / (1 + e)], rtol=4 * U, atol=0)
    idx2, _ = oracle.select_topk(oracle.correct_logits(l, hv, 2.0), 2)
    assert idx2.tolist() == [[1, 2]]
    # the raw logits are left alone
    assert np.array_equal(l, np.float32([[2.0, 1.5, 1.0, 0.0]]))


def test_correction_zero_alpha_and_constant_health_change_nothing():
    rng = np.random.default_rng(11)
    T, E, k = 16, 32, 4
    # logits on a 2^-10 grid in [-4, 4) with no repeats in a row: subtracting
    # 0.5 is exact, so the shifted softmax sees the same differences
    l = np.stack([rng.permutation(8192)[:E] for _ in range(T)]).astype(np.float32) / 1024.0 - 4.0
    i0, w0 = oracle.select_topk(l, k)
    for hv, a in [(rng.standard_normal(E).astype(np.float32), 0.0), (np.full(E, 0.25, np.float32), 2.0)]:
        c = oracle.correct_logits(l, hv, a)
        i1, w1 = oracle.select_topk(c, k)
        assert np.array_equal(i0, i1)
        assert np.array_equal(w0, w1)


def test_correction_steers_away_from_an_overloaded_expert():
    rng = np.random.default_rng(12)
    T, E, k = 64, 32, 2
    l = rng.standard_normal((T, E)).astype(np.float32)
    hot = int(np.argmax(np.bincount(oracle.select_topk(l, k)[0].ravel(), minlength=E)))
    hv = np.zeros(E, np.float32)
    hv[hot] = 100.0  # far above any logit gap of N(0,1) logits
    idx, _ = oracle.select_topk(oracle.correct_logits(l, hv, 1.0), k)
    assert (idx != hot).all()
    # every other expert keeps its rank order: the selection equals the top-k
    # of the logits with the hot expert removed
    l2 = l.copy()
    l2[:, hot] = -np.inf
    assert np.array_equal(idx, np.argsort(-l2, axis=1, kind="stable")[:, :k])


def _grouped_brute(l, G, k):
    """All k-sets with at most one expert per group; the chosen set has the
    lexicographically best key sequence (larger logit, then lower index)."""
    import itertools
    E = l.size
    gs = E // G
    best = None
    for S in itertools.combinations(range(E), k):
        if len({e // gs for e in S}) < k:
            continue
        key = sorted((-float(l[e]), e) for e in S)
        if best is None or key < best:
            best = key
    return [e for _, e in best]


@pytest.mark.parametrize("E,G", [(8, 4), (12, 3), (16, 4)])
def test_grouped_selection_brute_force(E, G):
    rng = np.random.default_rng(E * 10 + G)
    for trial in range(60):
        # coarse values so that ties inside and across groups occur
        l = (rng.integers(-3, 4, size=E) / 2.0).astype(np.float32)
        for k in range(1, G + 1):
            idx, w = oracle.select_topk(l[None], k, groups=G)
            assert idx[0].tolist() == _grouped_brute(l, G, k), (l, k)
            p = np.exp(l.astype(np.float64) - l.max())
            want = p[idx[0]] / p[idx[0]].sum()
            assert np.allclose(w[0], want, rtol=64 * U, atol=0)


def test_grouped_with_singleton_groups_is_plain_topk():
    rng = np.random.default_rng(13)
    l = rng.standard_normal((32, 16)).astype(np.float32)
    for k in (1, 3, 8):
        a = oracle.select_topk(l, k)
        b = oracle.select_topk(l, k, groups=16)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_grouped_page_shape_one_best_per_group():
    # 64 experts in 4 groups of 16, one from each group: 4 slots, and each
    # slot is the first maximum of its group
    rng = np.random.default_rng(14)
    l = rng.standard_normal((200, 64)).astype(np.float32)
    idx, w = oracle.select_topk(l, 4, groups=4)
    for t in range(l.shape[0]):
        assert sorted(e // 16 for e in idx[t]) == [0, 1, 2, 3]
        assert set(idx[t]) == {g * 16 + int(np.argmax(l[t, g * 16:(g + 1) * 16])) for g in range(4)}
        assert list(l[t, idx[t]]) == sorted(l[t, idx[t]], reverse=True)
    assert np.allclose(w.sum(axis=1), 1.0, atol=8 * U)


def test_load_stats_closed_forms():
    import statistics
    E = 32
    assert oracle.load_stats(np.full(E, 7, np.int32)) == (0, 0.0)
    for j, c in [(0, 9), (5, 12), (31, 1)]:
        v = np.zeros(E, np.int32)
        v[j] = c
        lu, sd = oracle.load_stats(v)
        assert lu == (1 if j == 0 else 0)
        # one count c among E: the deviation is c * sqrt(E - 1) / E
        assert sd == np.float32(c * math.sqrt(E - 1) / E)
    assert oracle.load_stats(np.int32([3, 10])) == (0, 3.5)
    # an activation vector like the trace example on the same page (counts of
    # 12 and 8 for two experts, the rest silent), against the library routine
    v = np.zeros(E, np.int32)
    v[2], v[5] = 12, 8
    lu, sd = oracle.load_stats(v)
    assert lu == 0 and sd == np.float32(statistics.pstdev(v.tolist()))
    rng = np.random.default_rng(15)
    for _ in range(20):
        v = rng.integers(0, 5000, size=E).astype(np.int32)
        lu, sd = oracle.load_stats(v)
        assert lu == int(np.argmin(v))
        assert sd == np.float32(statistics.pstdev(v.tolist()))


def test_route_with_options_is_correction_then_grouped_selection():
    inp = mi.make_inputs("tiny")
    rng = np.random.default_rng(16)
    hv = rng.random(inp.E).astype(np.float32)
    idx, w, ku, hm, logits = oracle.route(inp.x, inp.wr, inp.dtype, 2, want_logits=True, health=hv, alpha=0.75,
                                          groups=4)
    raw = oracle.router_logits(inp.x, inp.wr, inp.dtype)
    assert np.array_equal(logits, oracle.correct_logits(raw, hv, 0.75))
    i2, w2 = oracle.select_topk(logits, 2, groups=4)
    assert np.array_equal(idx, i2) and np.array_equal(w, w2)


@pytest.mark.parametrize("m,shift,n_moved,k_raw,k_corr", [(12, 40.0, 9, 2, 1), (3, -40.0, 10, 1, 3)])
def test_entropy_is_taken_on_corrected_logits(m, shift, n_moved, k_raw, k_corr):
    # Page "Qwen3.5-MoE与Qwen3-MoE架构差异深度解析": section 3.3 corrects the
    # logits by the load index before routing, and section 2.2 picks k from
    # the entropy of the routing distribution, so the entropy is that of the
    # corrected logits.  m equal dominant logits 40 above the other E - m give
    # H = ln m (closed form; the others add about E e^-40).  The correction
    # alpha * health with alpha = 40 and health 1 (or -1) on n_moved experts
    # takes them down to (or up to) the others' level, moving H across a band
    # edge: ln 12 = 2.485 -> ln 3 = 1.099 (k 2 -> 1), ln 3 -> ln 13 = 2.565
    # (k 1 -> 3).
    E, H, T = 32, 64, 4
    x = mi.round_half(np.eye(T, H) * 4.0, "f16")
    wr64 = np.zeros((E, H))
    wr64[:m, :T] = 10.0  # logit 40 for the m dominant experts of every token
    wr = mi.round_half(wr64, "f16")
    health = np.zeros(E, np.float32)
    if shift > 0:
        moved = np.arange(m - n_moved, m)  # the last n_moved dominant experts drop to 0
        health[moved] = 1.0
    else:
        moved = np.arange(m, m + n_moved)  # n_moved others rise to 40
        health[moved] = -1.0
    alpha = abs(shift)
    m_corr = m - n_moved if shift > 0 else m + n_moved
    _, _, ku_raw, h_raw = oracle.route(x, wr, "f16", -1)
    assert ku_raw == k_raw and abs(h_raw - math.log(m)) < 1e-5
    idx, w, ku, hm, logits = oracle.route(x, wr, "f16", -1, want_logits=True, health=health, alpha=alpha)
    assert abs(hm - math.log(m_corr)) < 1e-5, hm
    assert ku == k_corr
    dominant = np.flatnonzero(logits[0] == 40.0)
    assert dominant.size == m_corr
    # top-k_corr of equal logits: the lowest indices, equal weights 1/k
    assert np.array_equal(idx[:, :ku], np.tile(dominant[:ku], (T, 1)))
    assert np.all(idx[:, ku:] == -1) and np.all(w[:, ku:] == 0)
    assert np.allclose(w[:, :ku], 1.0 / ku, atol=1e-7, rtol=0)


# ------------------------------------------------------------- capacity --
# Page "Qwen3.5-MoE与Qwen3-MoE架构差异深度解析", section 5.2: a per-expert token
# capacity (expert_capacity).  Reading: the first C pairs of an expert in pair
# order are kept, the rest contribute nothing.

def _keep_brute(idx, ku, C):
    T, kcap = idx.shape
    flat = idx.ravel()
    valid = (np.arange(T * kcap) % kcap) < ku
    return np.array([bool(valid[p]) and (C <= 0 or sum(1 for q in range(p) if valid[q] and flat[q] == flat[p]) < C)
                     for p in range(T * kcap)]).reshape(T, kcap)


@pytest.mark.parametrize("T,kcap,ku,E,C", [(9, 2, 2, 4, 1), (13, 3, 2, 5, 2), (20, 4, 4, 6, 3), (7, 3, 3, 3, 0),
                                           (16, 2, 2, 2, 16)])
def test_capacity_keep_brute_force_and_sort(T, kcap, ku, E, C):
    rng = np.random.default_rng(T * 100 + C)
    for _ in range(10):
        idx = rng.integers(0, E, size=(T, kcap)).astype(np.int32)
        keep = oracle.capacity_keep(idx, ku, E, C)
        assert np.array_equal(keep, _keep_brute(idx, ku, C))
        c0, o0, p0, _ = oracle.sort_pairs(idx, ku, E)
        c1, o1, p1, pos1 = oracle.sort_pairs(idx, ku, E, capacity=C)
        want = np.minimum(c0, C) if C > 0 else c0
        assert np.array_equal(c1, want)
        assert np.array_equal(o1, np.concatenate([[0], np.cumsum(want)]))
        for e in range(E):  # an expert's kept list is the prefix of its full list
            assert np.array_equal(p1[o1[e]:o1[e + 1]], p0[o0[e]:o0[e] + want[e]])
        assert (p1[o1[-1]:] == -1).all()
        flat_keep = keep.ravel()
        assert ((pos1 >= 0) == flat_keep).all()
        assert (p1[pos1[flat_keep]] == np.flatnonzero(flat_keep)).all()


def test_capacity_layer_drops_whole_pairs():
    inp = mi.make_inputs("tiny", T=12)
    gu = oracle.fuse_gate_up(inp.gate, inp.up)
    full = oracle.layer_forward(inp.x, inp.wr, inp.dtype, inp.k, gu, inp.down)
    counts = np.bincount(full["idx"].ravel(), minlength=inp.E)
    # a capacity at or above every count changes nothing, bit for bit
    same = oracle.layer_forward(inp.x, inp.wr, inp.dtype, inp.k, gu, inp.down, capacity=int(counts.max()))
    assert np.array_equal(same["y"], full["y"]) and np.array_equal(same["y_f32"], full["y_f32"])
    for C in (1, 2):
        cap = oracle.layer_forward(inp.x, inp.wr, inp.dtype, inp.k, gu, inp.down, capacity=C)
        assert np.array_equal(cap["idx"], full["idx"])  # routing itself is unchanged
        keep = oracle.capacity_keep(full["idx"], inp.k, inp.E, C)
        assert keep.sum() == np.minimum(counts, C).sum()
        for t in range(inp.T):
            # each token's output is the slot-order sum over its kept slots
            # only: the full layer rebuilt one slot at a time
            acc = np.zeros(inp.H, np.float32)
            for s in range(inp.k):
                if keep[t, s]:
                    one = np.full((1, inp.k), -1, np.int32)
                    one[0, s] = full["idx"][t, s]
                    acc = acc + oracle.tokens_forward(inp.x[t:t + 1], inp.dtype, [0], one, full["w"][t:t + 1],
                                                      inp.k, gu, inp.down)[0]
            assert np.array_equal(cap["y_f32"][t], acc)
            if not keep[t].any():
                assert not cap["y_f32"][t].any()
