"""The seeded input generator: determinism, distributions, and that each
workload recipe has the structure it is meant to have (expert-load skew,
entropy bands), measured with the oracle."""
import math

import numpy as np
import pytest

import moe_inputs as mi
import oracle
from ref64 import half64


def test_streams_are_deterministic_and_index_addressable():
    a = mi.normal_f64(42, 3, 1000)
    b = mi.normal_f64(42, 3, 600, start=400)
    assert np.array_equal(a[400:], b)
    assert not np.array_equal(a, mi.normal_f64(43, 3, 1000))
    assert not np.array_equal(a, mi.normal_f64(42, 4, 1000))


def test_normal_moments():
    v = mi.normal_f64(7, 0, 400000)
    assert abs(v.mean()) < 0.01 and abs(v.std() - 1) < 0.01
    assert abs(np.mean(v ** 4) - 3) < 0.05  # Gaussian kurtosis


def test_half_rounding_is_rne():
    v = mi.normal_f64(8, 0, 10000) * 3
    assert np.array_equal(mi.round_half(v, "f16"), v.astype(np.float32).astype(np.float16).view(np.uint16))
    assert np.array_equal(mi.decode_half(mi.round_half(v, "bf16"), "bf16"), half64(mi.round_half(v, "bf16"), "bf16"))


@pytest.mark.parametrize("bits", [4, 8])
def test_quantizer_error_is_within_half_a_step(bits):
    w = mi.quant_weights(3, 2, 2, 16, 256, bits)
    raw = mi.normal_f64(3, 2, 2 * 16 * 256, 0.02).reshape(2, 16, 256)
    deq = oracle.dequant(w).astype(np.float64)
    s = np.repeat(half64(w.scales, "f16"), 64, -1)
    # min-max grid: |w - deq| <= s/2 plus the fp16 rounding of scale and bias
    assert np.all(np.abs(raw - deq) <= 0.5 * s + 16 * s * 2 ** -11 + 1e-7)


def test_packing_low_nibble_is_even_column():
    raw = np.tile(np.arange(64, dtype=np.float64) % 16, (1, 1))
    q, s, b = mi.quantize_rows(raw, 4)
    assert q[0, 0] == (0 | (1 << 4)) and q[0, 1] == (2 | (3 << 4))


def test_zipf_prefill_is_skewed_at_least_tenfold():
    sets = mi.zipf_sets(1004, 4096, 64, 4, 1.2)
    assert np.all(np.sort(sets, 1)[:, 1:] != np.sort(sets, 1)[:, :-1])  # distinct per token
    counts = np.bincount(sets.ravel(), minlength=64)
    assert counts.max() >= 10 * counts.mean()


def test_planted_routing_selects_the_planted_experts():
    x, wr, sets = mi.make_router_inputs("batched_decode")
    idx, w, ku, _ = oracle.route(x, wr, "bf16", 2)
    agree = np.mean([set(idx[t]) == set(sets[t]) for t in range(64)])
    assert agree >= 0.98


@pytest.mark.parametrize("segment,k", [(0, 1), (1, 2), (2, 3), (3, 3)])
def test_entropy_segments_land_in_their_bands(segment, k):
    x, wr, _ = mi.make_router_inputs("entropy", segment=segment)
    logits = oracle.router_logits(x, wr, "f16")
    h = oracle.batch_entropy(logits)
    assert oracle.entropy_k(h) == k
    # at least 0.15 nats from either threshold, so fp32 rounding cannot flip k
    assert min(abs(h - 1.2), abs(h - 2.5)) >= 0.15, h
