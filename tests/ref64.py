"""Independent fp64 numpy statements of the layer, used only to pin the oracle.

Nothing here calls the oracle or the HIP path.  Dequantisation unpacks the
codes with numpy and evaluates scale*q + bias in fp64; the layer is the dense
softmax-gated mixture with every gate outside the token's top-k set to zero,
which is what sparse routing computes exactly.
"""
from __future__ import annotations

import numpy as np

import moe_inputs as mi


def half64(bits: np.ndarray, dtype: str) -> np.ndarray:
    bits = np.ascontiguousarray(bits, np.uint16)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def codes(w: mi.Weights) -> np.ndarray:
    if w.bits == 4:
        lo = (w.q & 0x0F).astype(np.int64)
        hi = (w.q >> 4).astype(np.int64)
        return np.stack([lo, hi], axis=-1).reshape(w.E, w.N, w.K)
    if w.bits in (5, 6):
        # each row's bytes as a little-endian bit stream, `bits` bits per code
        stream = np.unpackbits(w.q.reshape(-1, w.q.shape[-1]), axis=-1, bitorder="little")
        per_code = stream.reshape(-1, w.K, w.bits).astype(np.int64)
        return (per_code << np.arange(w.bits)).sum(axis=-1).reshape(w.E, w.N, w.K)
    return w.q.astype(np.int64)


# E2M1 magnitudes of codes 0..7 (NVIDIA's published NVFP4 element format);
# codes 8..15 are the same values negated (sign bit 3)
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_64(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes, np.int64)
    return np.where(c & 8, -1.0, 1.0) * E2M1_MAGNITUDES[c & 7]


def e4m3_64(b: np.ndarray) -> np.ndarray:
    """FP8 E4M3 bytes decoded by torch's float8_e4m3fn."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(b, np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def dequant64(w: mi.Weights) -> np.ndarray:
    if w.bits == 16:
        return half64(w.q, "f16")
    if w.fmt == "nvfp4":
        s = np.repeat(e4m3_64(w.scales), 16, axis=-1)
        return float(w.tensor_scale) * s * e2m1_64(codes(w))
    q = codes(w).astype(np.float64)
    s = np.repeat(half64(w.scales, "f16"), w.group_size, axis=-1)
    b = np.repeat(half64(w.biases, "f16"), w.group_size, axis=-1)
    return s * q + b


def silu64(g: np.ndarray) -> np.ndarray:
    return g / (1.0 + np.exp(-g))


def select64(logits: np.ndarray, k: int):
    """(idx, w) by larger logit first, lower index among equals; renormalised softmax."""
    T, E = logits.shape
    idx = np.empty((T, k), np.int64)
    w = np.empty((T, k))
    for t in range(T):
        order = np.lexsort((np.arange(E), -logits[t]))
        idx[t] = order[:k]
        p = np.exp(logits[t] - logits[t].max())
        p /= p.sum()
        w[t] = p[order[:k]] / p[order[:k]].sum()
    return idx, w


def entropy64(logits: np.ndarray) -> np.ndarray:
    p = np.exp(logits - logits.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(p > 0, p * np.log(p), 0.0)
    return -t.sum(axis=1)


def dense_layer64(x_bits, wr_bits, dtype, k, gate, up, down, idx=None, w=None):
    """Dense brute force: every expert on every token, gates zero off the top-k.

    idx/w may be given (e.g. an fp32 routing) to compare only the expert math.
    Returns (y [T, H] fp64, idx, w).
    """
    x = half64(x_bits, dtype)
    wr = half64(wr_bits, dtype)
    logits = x @ wr.T
    T, E = logits.shape
    if idx is None:
        kk = k
        if k < 0:
            hm = entropy64(logits).mean()
            kk = 1 if hm < 1.2 else (2 if hm < 2.5 else 3)
        idx, w = select64(logits, kk)
    G = np.zeros((T, E))
    for t in range(T):
        for s in range(idx.shape[1]):
            if idx[t, s] >= 0:
                G[t, idx[t, s]] += w[t, s]
    Wg, Wu, Wd = dequant64(gate), dequant64(up), dequant64(down)
    y = np.zeros((T, Wd.shape[1]))
    for e in range(E):
        g = x @ Wg[e].T
        u = x @ Wu[e].T
        h = silu64(g) * u
        o = h @ Wd[e].T
        y += G[:, e:e + 1] * o
    return y, idx, w


def rel_l2(a: np.ndarray, b: np.ndarray) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))
