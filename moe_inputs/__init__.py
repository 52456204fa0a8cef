"""Seeded synthetic inputs for one sparse MoE FFN layer.

Both the HIP path and the CPU oracle take their inputs from here, and from
nowhere else.  This module holds none of the layer's arithmetic: it draws
normals from a counter-based generator (``gen.c``), rounds them to fp16/bf16,
quantises expert weights with a min-max affine rule and plants Zipf-skewed
routing preferences.  Everything is a pure function of the seed.

Workload recipes (the shapes of the layer the pages describe):

* ``tiny``            T=4, H=256, E=8, top-2, I=128; 4-bit group 64; fp16.
* ``decode_b1``       one token, H=4096, E=64, top-4, I=11008; 4-bit; fp16.
  These are the MoE hyper-parameters the first page prints from a Qwen3.5
  ``config.json`` (P1 "Qwen3.5的Block本质", the config excerpt).
* ``batched_decode``  64 tokens, H=4096, E=32, static top-2 (the Qwen3-MoE
  routing of the second page), I=2816; 8-bit; bf16; Zipf s=1.1 expert load.
* ``prefill``         4096 tokens, H=4096, E=64, top-4, I=1408; 4-bit; bf16;
  Zipf s=1.2 expert load.
* ``entropy``         4 segments of 512 tokens, H=4096, E=32, I=2816,
  entropy-adaptive k; router temperature per segment; weights unquantised
  fp16 (bits=16) or 4-bit.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
_LIB = os.path.join(_HERE, "libmoe_inputs.so")
_lib = None

# tensor ids of the counter-based streams
TID_X, TID_WR, TID_GATE, TID_UP, TID_DOWN = 0, 1, 2, 3, 4

DTYPE_CODE = {"f16": 1, "bf16": 2}


def build(force: bool = True) -> str:
    """Compile gen.c into libmoe_inputs.so (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    u64, u32, i64, i32, dbl = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64, ctypes.c_int, ctypes.c_double
    vp = ctypes.c_void_p
    lib.gen_set_threads.argtypes = [i32]
    lib.gen_normal_f64.argtypes = [u64, u32, i64, i64, dbl, vp]
    lib.gen_normal_half.argtypes = [u64, u32, i64, i64, dbl, i32, vp]
    lib.gen_uniform.argtypes = [u64, u32, i64, i64, vp]
    lib.gen_round_half.argtypes = [vp, i64, i32, vp]
    lib.gen_decode_half.argtypes = [vp, i64, i32, vp]
    lib.gen_quantize_rows.argtypes = [vp, i64, i32, i32, i32, vp, vp, vp]
    lib.gen_quant_weights.argtypes = [u64, u32, i32, i32, i32, i32, i32, dbl, vp, vp, vp]
    lib.gen_quantize_rows_nvfp4.argtypes = [vp, i64, i32, dbl, vp, vp]
    lib.gen_quant_nvfp4.argtypes = [u64, u32, i32, i32, i32, dbl, dbl, vp, vp]
    lib.gen_zipf_sets.argtypes = [u64, i64, i32, i32, i32, dbl, vp]
    lib.gen_planted_x.argtypes = [u64, i64, i32, i32, i32, i32, vp, i32, vp, dbl, vp]
    _lib = lib
    return lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def set_threads(n: int) -> None:
    _load().gen_set_threads(int(n))


# ------------------------------------------------------------ primitives --

def normal_f64(seed: int, tid: int, n: int, sigma: float = 1.0, start: int = 0) -> np.ndarray:
    out = np.empty(n, np.float64)
    _load().gen_normal_f64(seed, tid, start, n, sigma, _p(out))
    return out


def normal_half(seed: int, tid: int, n: int, sigma: float, dtype: str, start: int = 0) -> np.ndarray:
    out = np.empty(n, np.uint16)
    _load().gen_normal_half(seed, tid, start, n, sigma, DTYPE_CODE[dtype], _p(out))
    return out


def uniform(seed: int, tid: int, n: int, start: int = 0) -> np.ndarray:
    out = np.empty(n, np.float64)
    _load().gen_uniform(seed, tid, start, n, _p(out))
    return out


def round_half(v: np.ndarray, dtype: str) -> np.ndarray:
    v = np.ascontiguousarray(v, np.float64)
    out = np.empty(v.shape, np.uint16)
    _load().gen_round_half(_p(v), v.size, DTYPE_CODE[dtype], _p(out))
    return out


def decode_half(b: np.ndarray, dtype: str) -> np.ndarray:
    b = np.ascontiguousarray(b, np.uint16)
    out = np.empty(b.shape, np.float64)
    _load().gen_decode_half(_p(b), b.size, DTYPE_CODE[dtype], _p(out))
    return out


@dataclasses.dataclass
class Weights:
    """One expert weight tensor [E, N, K].

    bits 4/5/6/8: ``q`` uint8 [E, N, K/2] (4-bit, low nibble = even column),
    [E, N, 5K/8] or [E, N, 3K/4] (5- or 6-bit, code k at bits b*k..b*k+b-1 of
    the row's little-endian bit stream, b = bits) or [E, N, K] (8-bit);
    ``scales``/``biases`` fp16 bits [E, N, K/group].
    bits 16:  ``q`` fp16 bits [E, N, K]; scales/biases None.
    fmt "nvfp4" (bits 4, group 16): ``q`` [E, N, K/2] E2M1 codes (sign in
    bit 3), two per byte, low nibble = even column; ``scales`` E4M3 bytes
    [E, N, K/16]; no biases; ``tensor_scale`` the fp32 per-tensor scale.
    """

    q: np.ndarray
    scales: Optional[np.ndarray]
    biases: Optional[np.ndarray]
    E: int
    N: int
    K: int
    bits: int
    group_size: int = 64
    fmt: str = "affine"  # "affine" | "nvfp4"
    tensor_scale: float = 1.0

    @property
    def nbytes(self) -> int:
        n = self.q.nbytes
        if self.scales is not None:
            n += self.scales.nbytes
        if self.biases is not None:
            n += self.biases.nbytes
        return n


def quant_weights(seed: int, tid: int, E: int, N: int, K: int, bits: int, sigma: float = 0.02,
                  gs: int = 64) -> Weights:
    if bits == 16:
        q = normal_half(seed, tid, E * N * K, sigma, "f16").reshape(E, N, K)
        return Weights(q, None, None, E, N, K, 16, gs)
    assert bits in (4, 5, 6, 8) and K % gs == 0
    q = np.empty((E, N, K * bits // 8), np.uint8)
    s = np.empty((E, N, K // gs), np.uint16)
    b = np.empty((E, N, K // gs), np.uint16)
    _load().gen_quant_weights(seed, tid, E, N, K, bits, gs, sigma, _p(q), _p(s), _p(b))
    return Weights(q, s, b, E, N, K, bits, gs)


def nvfp4_weights(seed: int, tid: int, E: int, N: int, K: int, sigma: float = 0.02,
                  ts: Optional[float] = None) -> Weights:
    """N(0, sigma) weights [E, N, K] quantised to NVFP4.  The tensor scale
    defaults to 8 sigma / (6 * 448): an amax of 8 sigma (which such a tensor
    practically never exceeds) spread over E2M1's largest value and E4M3's."""
    assert K % 16 == 0
    ts = float(np.float32(8.0 * sigma / (6.0 * 448.0))) if ts is None else float(np.float32(ts))
    q = np.empty((E, N, K // 2), np.uint8)
    s = np.empty((E, N, K // 16), np.uint8)
    _load().gen_quant_nvfp4(seed, tid, E, N, K, sigma, ts, _p(q), _p(s))
    return Weights(q, s, None, E, N, K, 4, 16, "nvfp4", ts)


def quantize_rows_nvfp4(w: np.ndarray, ts: Optional[float] = None):
    """NVFP4 codes and block scales of an explicit fp64 matrix [rows, K];
    ts defaults to amax / (6 * 448) of the matrix.  Returns (q, scales, ts)."""
    w = np.ascontiguousarray(w, np.float64)
    rows, K = w.shape
    if ts is None:
        ts = float(np.abs(w).max()) / (6.0 * 448.0)
    ts = float(np.float32(ts))
    q = np.empty((rows, K // 2), np.uint8)
    s = np.empty((rows, K // 16), np.uint8)
    _load().gen_quantize_rows_nvfp4(_p(w), rows, K, ts, _p(q), _p(s))
    return q, s, ts


def quantize_rows(w: np.ndarray, bits: int, gs: int = 64):
    """Quantise an explicit fp64 matrix [rows, K] with the same min-max rule."""
    w = np.ascontiguousarray(w, np.float64)
    rows, K = w.shape
    q = np.empty((rows, K * bits // 8), np.uint8)
    s = np.empty((rows, K // gs), np.uint16)
    b = np.empty((rows, K // gs), np.uint16)
    _load().gen_quantize_rows(_p(w), rows, K, bits, gs, _p(q), _p(s), _p(b))
    return q, s, b


def zipf_sets(seed: int, T: int, E: int, k: int, s: float, t0: int = 0) -> np.ndarray:
    """k distinct Zipf(s)-ranked experts for each of tokens [t0, t0+T)."""
    out = np.empty((T, k), np.int32)
    _load().gen_zipf_sets(seed, t0, T, E, k, s, _p(out))
    return out


def load_index(seed: int, E: int, s: float = 1.1, window: int = 100, tokens: int = 64, k: int = 2) -> np.ndarray:
    """A per-expert load index H [E] fp32 with mean 1: the activation counts of
    `window` steps of `tokens` tokens routed top-k with Zipf(s) expert
    popularity, divided by their mean (the activation frequency over a recent
    window that a load-aware router subtracts, scaled, from its logits)."""
    sets = zipf_sets(seed, window * tokens, E, min(k, E), s)
    c = np.bincount(sets.ravel(), minlength=E).astype(np.float64)
    return (c / c.mean()).astype(np.float32)


def planted_x(seed: int, T: int, H: int, wr: np.ndarray, dtype: str, sets: np.ndarray, gamma: float = 8.0,
              t0: int = 0):
    """Activations of tokens [t0, t0+T) with each token's set planted."""
    E = wr.shape[0]
    k = sets.shape[1]
    assert sets.shape[0] == T
    out = np.empty((T, H), np.uint16)
    _load().gen_planted_x(seed, t0, T, H, E, k, _p(np.ascontiguousarray(wr)), DTYPE_CODE[dtype],
                          _p(np.ascontiguousarray(sets, np.int32)), gamma, _p(out))
    return out


# ---------------------------------------------------------------- recipes --

RECIPES = {
    "tiny": dict(index=1, T=4, H=256, E=8, k=2, I=128, bits=4, dtype="f16", zipf=None),
    "decode_b1": dict(index=2, T=1, H=4096, E=64, k=4, I=11008, bits=4, dtype="f16", zipf=None),
    "batched_decode": dict(index=3, T=64, H=4096, E=32, k=2, I=2816, bits=8, dtype="bf16", zipf=1.1),
    "prefill": dict(index=4, T=4096, H=4096, E=64, k=4, I=1408, bits=4, dtype="bf16", zipf=1.2),
    "entropy": dict(index=5, T=512, H=4096, E=32, k=-1, I=2816, bits=16, dtype="f16", zipf=None),
}

# router temperature multipliers of the four entropy segments: predicted
# batch entropies about 0.7 / 1.8 / 3.0 / 2.8 nats, i.e. k = 1 / 2 / 3 / 3
ENTROPY_TEMPS = (4.69, 1.95, 0.78, 1.00)
PLANT_GAMMA = 8.0
ROUTER_SIGMA = 0.02
WEIGHT_SIGMA = 0.02


@dataclasses.dataclass
class LayerInputs:
    name: str
    T: int
    H: int
    E: int
    I: int
    k: int  # -1 = entropy-adaptive
    bits: int
    dtype: str  # "f16" | "bf16"
    seed: int
    x: np.ndarray  # uint16 bits [T, H]
    wr: np.ndarray  # uint16 bits [E, H]
    gate: Weights
    up: Weights
    down: Weights
    sets: Optional[np.ndarray] = None  # planted expert sets (Zipf recipes)
    segment: int = 0
    fmt: str = "affine"  # weight format: "affine" (bits 4/5/6/8, or 16 unquantised) | "nvfp4"

    @property
    def kcap(self) -> int:
        return 3 if self.k == -1 else self.k


def _resolve(name, T, H, E, I, k, bits, dtype, seed, zipf):
    r = dict(RECIPES[name])
    T = r["T"] if T is None else T
    H = r["H"] if H is None else H
    E = r["E"] if E is None else E
    I = r["I"] if I is None else I
    k = r["k"] if k is None else k
    bits = r["bits"] if bits is None else bits
    dtype = r["dtype"] if dtype is None else dtype
    seed = 1000 + r["index"] if seed is None else seed
    zipf_s = r["zipf"] if zipf == "recipe" else zipf
    return T, H, E, I, k, bits, dtype, seed, zipf_s


def make_router_inputs(name: str, *, T: Optional[int] = None, H: Optional[int] = None, E: Optional[int] = None,
                       k: Optional[int] = None, dtype: Optional[str] = None, seed: Optional[int] = None,
                       segment: int = 0, zipf="recipe", token_offset: int = 0):
    """Activations and router weights only: returns (x, wr, sets)."""
    T, H, E, _, k, _, dtype, seed, zipf_s = _resolve(name, T, H, E, 64, k, 4, dtype, seed, zipf)
    sigma_r = ROUTER_SIGMA
    if name == "entropy":
        sigma_r = ROUTER_SIGMA * ENTROPY_TEMPS[segment]
        token_offset += segment * T
    wr = normal_half(seed, TID_WR, E * H, sigma_r, dtype).reshape(E, H)
    sets = None
    if zipf_s is not None:
        assert k > 0
        sets = zipf_sets(seed, T, E, k, zipf_s, t0=token_offset)
        x = planted_x(seed, T, H, wr, dtype, sets, PLANT_GAMMA, t0=token_offset)
    else:
        x = normal_half(seed, TID_X, T * H, 1.0, dtype, start=token_offset * H).reshape(T, H)
    return x, wr, sets


def make_inputs(name: str, *, T: Optional[int] = None, H: Optional[int] = None, E: Optional[int] = None,
                I: Optional[int] = None, k: Optional[int] = None, bits: Optional[int] = None,
                dtype: Optional[str] = None, seed: Optional[int] = None, segment: int = 0,
                zipf="recipe", token_offset: int = 0, fmt: str = "affine") -> LayerInputs:
    """Build one call's inputs for a recipe, optionally with smaller shapes.

    ``segment`` selects the router temperature and token range of the
    ``entropy`` recipe.  ``token_offset`` starts the activation rows further
    along the stream (a pool of decode tokens).  ``fmt="nvfp4"`` quantises
    the expert weights to NVFP4 instead (bits is then 4).
    """
    T, H, E, I, k, bits, dtype, seed, _ = _resolve(name, T, H, E, I, k, bits, dtype, seed, zipf)
    x, wr, sets = make_router_inputs(name, T=T, H=H, E=E, k=k, dtype=dtype, seed=seed, segment=segment, zipf=zipf,
                                     token_offset=token_offset)
    if fmt == "nvfp4":
        bits = 4
        gate = nvfp4_weights(seed, TID_GATE, E, I, H, WEIGHT_SIGMA)
        up = nvfp4_weights(seed, TID_UP, E, I, H, WEIGHT_SIGMA)
        down = nvfp4_weights(seed, TID_DOWN, E, H, I, WEIGHT_SIGMA)
    else:
        assert fmt == "affine", fmt
        gate = quant_weights(seed, TID_GATE, E, I, H, bits, WEIGHT_SIGMA)
        up = quant_weights(seed, TID_UP, E, I, H, bits, WEIGHT_SIGMA)
        down = quant_weights(seed, TID_DOWN, E, H, I, bits, WEIGHT_SIGMA)
    return LayerInputs(name, T, H, E, I, k, bits, dtype, seed, x, wr, gate, up, down, sets, segment, fmt)


def exact_router_inputs(seed: int, T: int, H: int, E: int, dtype: str = "f16"):
    """Activations and router rows on a coarse grid so every partial sum of a
    router dot product is exactly representable in fp32 (x in {j/16: |j|<=16},
    Wr in {j/1024: |j|<=32}); logits then agree bit for bit in any order."""
    ux = uniform(seed, 11, T * H)
    uw = uniform(seed, 12, E * H)
    x = np.floor(ux * 33).astype(np.int64) - 16
    w = np.floor(uw * 65).astype(np.int64) - 32
    xb = round_half(x / 16.0, dtype).reshape(T, H)
    wb = round_half(w / 1024.0, dtype).reshape(E, H)
    return xb, wb
