"""CPU oracle for one sparse MoE FFN layer — TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The library path never does: it shares
no code, header, table or helper with ``oracle.c``.

This module only marshals numpy arrays into ``liboracle.so`` (plain C, fp32,
sequential sums, -ffp-contract=off).  The arithmetic and the passages of the
pages it follows are documented at the top of ``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

DTYPE_CODE = {"f16": 1, "bf16": 2}
NVFP4 = 0x104  # `bits` code of NVFP4 weights (E2M1 codes, E4M3 block scales, fp32 tensor scale)


def build(force: bool = True) -> str:
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-ffp-contract=off",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
    lib.oracle_half_to_float.argtypes = [ctypes.c_uint16, i32]
    lib.oracle_half_to_float.restype = f32
    lib.oracle_float_to_half.argtypes = [f32, i32]
    lib.oracle_float_to_half.restype = ctypes.c_uint16
    lib.oracle_dequant_row.argtypes = [vp, vp, vp, i32, i32, i32, f32, vp]
    lib.oracle_e2m1_to_float.argtypes = [i32]
    lib.oracle_e2m1_to_float.restype = f32
    lib.oracle_e4m3_to_float.argtypes = [i32]
    lib.oracle_e4m3_to_float.restype = f32
    lib.oracle_router_logits.argtypes = [vp, i32, i32, i32, vp, i32, vp]
    lib.oracle_select_topk.argtypes = [vp, i32, i32, i32, i32, vp, vp]
    lib.oracle_select_topk_grouped.argtypes = [vp, i32, i32, i32, i32, i32, vp, vp]
    lib.oracle_correct_logits.argtypes = [vp, i32, i32, vp, f32]
    lib.oracle_load_stats.argtypes = [vp, i32, vp, vp]
    lib.oracle_route_ex.argtypes = [vp, i32, i32, i32, vp, i32, i32, vp, f32, i32, vp, vp, vp, vp, vp]
    lib.oracle_layer_forward_ex.argtypes = [vp, i32, i32, i32, vp, i32, i32, vp, f32, i32, i32, vp, vp, vp, vp, vp,
                                            vp, i32, i32, i32, f32, f32, vp, vp, vp, vp, vp, vp]
    lib.oracle_capacity_keep.argtypes = [vp, i32, i32, i32, i32, i32, vp]
    lib.oracle_sort_pairs_capped.argtypes = [vp, i32, i32, i32, i32, i32, vp, vp, vp, vp]
    lib.oracle_token_entropy.argtypes = [vp, i32]
    lib.oracle_token_entropy.restype = f32
    lib.oracle_entropy_k.argtypes = [f32]
    lib.oracle_entropy_k.restype = i32
    lib.oracle_batch_entropy.argtypes = [vp, i32, i32]
    lib.oracle_batch_entropy.restype = f32
    lib.oracle_route.argtypes = [vp, i32, i32, i32, vp, i32, i32, vp, vp, vp, vp, vp]
    lib.oracle_sort_pairs.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, vp]
    lib.oracle_fuse_gate_up.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, vp, vp]
    lib.oracle_expert_ffn.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, f32, vp, vp]
    lib.oracle_expert_ffn_unfused.argtypes = [vp] + [vp] * 9 + [i32, i32, i32, i32, f32, f32, f32, vp, vp]
    lib.oracle_tokens_forward.argtypes = [vp, i32, i32, vp, i32, vp, vp, i32, i32, vp, vp, vp, vp, vp, vp, i32,
                                          i32, i32, f32, f32, vp, vp]
    lib.oracle_round_output.argtypes = [vp, i64, i32, vp]
    lib.oracle_layer_forward.argtypes = [vp, i32, i32, i32, vp, i32, i32, vp, vp, vp, vp, vp, vp, i32, i32, i32,
                                         f32, f32, vp, vp, vp, vp, vp, vp]
    lib.oracle_num_threads.restype = i32
    lib.oracle_set_threads.argtypes = [i32]
    _lib = lib
    return lib


def _p(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dt):
    return None if a is None else np.ascontiguousarray(a, dt)


def num_threads() -> int:
    return _load().oracle_num_threads()


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


# ------------------------------------------------------------- scalars --

def half_to_float(bits: int, dtype: str) -> float:
    return float(_load().oracle_half_to_float(int(bits), DTYPE_CODE[dtype]))


def float_to_half(v: float, dtype: str) -> int:
    return int(_load().oracle_float_to_half(float(v), DTYPE_CODE[dtype]))


def round_output(y_f32: np.ndarray, dtype: str) -> np.ndarray:
    y_f32 = _c(y_f32, np.float32)
    out = np.empty(y_f32.shape, np.uint16)
    _load().oracle_round_output(_p(y_f32), y_f32.size, DTYPE_CODE[dtype], _p(out))
    return out


def e2m1_to_float(code: int) -> float:
    return float(_load().oracle_e2m1_to_float(int(code)))


def e4m3_to_float(byte: int) -> float:
    return float(_load().oracle_e4m3_to_float(int(byte)))


def code_of(w) -> int:
    """The oracle's `bits` code of a moe_inputs.Weights (NVFP4 or its width)."""
    return NVFP4 if getattr(w, "fmt", "affine") == "nvfp4" else w.bits


def tensor_scale(w) -> float:
    return float(getattr(w, "tensor_scale", 1.0)) if w is not None else 1.0


# -------------------------------------------------------------- steps ---

def dequant_row(q_row, s_row, b_row, K: int, bits: int, gs: int = 64, ts: float = 1.0) -> np.ndarray:
    """bits 4/5/6/8/16, or NVFP4 (s_row: E4M3 bytes, gs 16, ts the tensor scale)."""
    out = np.empty(K, np.float32)
    qd = np.uint16 if bits == 16 else np.uint8
    sd = np.uint8 if bits == NVFP4 else np.uint16
    _load().oracle_dequant_row(_p(_c(q_row, qd)), _p(_c(s_row, sd)), _p(_c(b_row, np.uint16)), K, bits, gs,
                               float(ts), _p(out))
    return out


def dequant(w) -> np.ndarray:
    """Whole [E, N, K] tensor of a moe_inputs.Weights, row by row (small shapes only)."""
    out = np.empty((w.E, w.N, w.K), np.float32)
    for e in range(w.E):
        for n in range(w.N):
            out[e, n] = dequant_row(w.q[e, n], None if w.scales is None else w.scales[e, n],
                                    None if w.biases is None else w.biases[e, n], w.K, code_of(w), w.group_size,
                                    tensor_scale(w))
    return out


def router_logits(x: np.ndarray, wr: np.ndarray, dtype: str) -> np.ndarray:
    x = _c(x, np.uint16)
    wr = _c(wr, np.uint16)
    T, H = x.shape
    E = wr.shape[0]
    out = np.empty((T, E), np.float32)
    _load().oracle_router_logits(_p(x), DTYPE_CODE[dtype], T, H, _p(wr), E, _p(out))
    return out


def select_topk(logits: np.ndarray, k: int, kcap: Optional[int] = None, groups: int = 0):
    """groups > 1: at most one expert per group of E/groups consecutive experts."""
    logits = _c(logits, np.float32)
    T, E = logits.shape
    kcap = k if kcap is None else kcap
    idx = np.empty((T, kcap), np.int32)
    w = np.empty((T, kcap), np.float32)
    if groups > 1:
        assert E % groups == 0 and k <= groups
        _load().oracle_select_topk_grouped(_p(logits), T, E, groups, k, kcap, _p(idx), _p(w))
    else:
        _load().oracle_select_topk(_p(logits), T, E, k, kcap, _p(idx), _p(w))
    return idx, w


def correct_logits(logits: np.ndarray, health: np.ndarray, alpha: float) -> np.ndarray:
    """logits - alpha * health[e] in fp32 (a new array)."""
    out = np.array(logits, np.float32, order="C", copy=True)
    h = _c(health, np.float32)
    T, E = out.shape
    assert h.shape == (E,)
    _load().oracle_correct_logits(_p(out), T, E, _p(h), float(alpha))
    return out


def load_stats(counts: np.ndarray):
    """(least-used expert, population standard deviation) of per-expert counts."""
    c = _c(counts, np.int32)
    lu = np.zeros(1, np.int32)
    sd = np.zeros(1, np.float32)
    _load().oracle_load_stats(_p(c), c.size, _p(lu), _p(sd))
    return int(lu[0]), float(sd[0])


def token_entropy(logit_row: np.ndarray) -> float:
    r = _c(logit_row, np.float32)
    return float(_load().oracle_token_entropy(_p(r), r.size))


def batch_entropy(logits: np.ndarray) -> float:
    logits = _c(logits, np.float32)
    return float(_load().oracle_batch_entropy(_p(logits), logits.shape[0], logits.shape[1]))


def entropy_k(h: float) -> int:
    return int(_load().oracle_entropy_k(float(h)))


def route(x: np.ndarray, wr: np.ndarray, dtype: str, k: int, want_logits: bool = False,
          health: Optional[np.ndarray] = None, alpha: float = 0.0, groups: int = 0):
    """Returns (idx [T,kcap], w [T,kcap], k_used, h_mean[, logits]); logits are the corrected ones."""
    x = _c(x, np.uint16)
    wr = _c(wr, np.uint16)
    T, H = x.shape
    E = wr.shape[0]
    kcap = k if k > 0 else 3
    idx = np.empty((T, kcap), np.int32)
    w = np.empty((T, kcap), np.float32)
    ku = np.zeros(1, np.int32)
    hm = np.zeros(1, np.float32)
    logits = np.empty((T, E), np.float32) if want_logits else None
    h = _c(health, np.float32)
    _load().oracle_route_ex(_p(x), DTYPE_CODE[dtype], T, H, _p(wr), E, k, _p(h), float(alpha), int(groups), _p(idx),
                            _p(w), _p(ku), _p(hm), _p(logits))
    res = (idx, w, int(ku[0]), float(hm[0]))
    return res + (logits,) if want_logits else res


def sort_pairs(idx: np.ndarray, k_used: int, E: int, capacity: int = 0):
    """Returns (counts [E], offsets [E+1], perm [P], pos [P]); capacity > 0
    keeps the first `capacity` pairs of every expert (dropped: pos -1)."""
    idx = _c(idx, np.int32)
    T, kcap = idx.shape
    P = T * kcap
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    perm = np.empty(P, np.int32)
    pos = np.empty(P, np.int32)
    if capacity > 0:
        _load().oracle_sort_pairs_capped(_p(idx), T, kcap, k_used, E, int(capacity), _p(counts), _p(offsets),
                                         _p(perm), _p(pos))
    else:
        _load().oracle_sort_pairs(_p(idx), T, kcap, k_used, E, _p(counts), _p(offsets), _p(perm), _p(pos))
    return counts, offsets, perm, pos


def capacity_keep(idx: np.ndarray, k_used: int, E: int, capacity: int) -> np.ndarray:
    """bool [T, kcap]: the pairs kept under a per-expert capacity."""
    idx = _c(idx, np.int32)
    T, kcap = idx.shape
    keep = np.empty((T, kcap), np.uint8)
    _load().oracle_capacity_keep(_p(idx), T, kcap, k_used, E, int(capacity), _p(keep))
    return keep.astype(bool)


def fuse_gate_up(gate, up):
    """[gate, up] concatenation of two moe_inputs.Weights along the output axis."""
    import dataclasses
    assert code_of(gate) == code_of(up) and gate.q.shape == up.q.shape
    assert tensor_scale(gate) == tensor_scale(up), "fused NVFP4 gate and up share one tensor scale"
    E, I, K, bits, gs = gate.E, gate.N, gate.K, code_of(gate), gate.group_size
    oq = np.empty((E, 2 * I) + gate.q.shape[2:], gate.q.dtype)
    os_ = None if gate.scales is None else np.empty((E, 2 * I, K // gs), gate.scales.dtype)
    ob = None if gate.biases is None else np.empty((E, 2 * I, K // gs), np.uint16)
    _load().oracle_fuse_gate_up(_p(gate.q), _p(gate.scales), _p(gate.biases), _p(up.q), _p(up.scales), _p(up.biases),
                                E, I, K, bits, gs, _p(oq), _p(os_), _p(ob))
    return dataclasses.replace(gate, q=oq, scales=os_, biases=ob, N=2 * I)


def _expert_slice(w, e):
    q = np.ascontiguousarray(w.q[e])
    s = None if w.scales is None else np.ascontiguousarray(w.scales[e])
    b = None if w.biases is None else np.ascontiguousarray(w.biases[e])
    return q, s, b


def expert_ffn(x_f32: np.ndarray, gate_up, down, e: int):
    """One (token, expert) through the fused gate_up tensor.  Returns (h [I], o [H])."""
    x_f32 = _c(x_f32, np.float32)
    H, I = down.N, down.K
    gq, gs_, gb = _expert_slice(gate_up, e)
    dq, ds, db = _expert_slice(down, e)
    h = np.empty(I, np.float32)
    o = np.empty(H, np.float32)
    _load().oracle_expert_ffn(_p(x_f32), _p(gq), _p(gs_), _p(gb), _p(dq), _p(ds), _p(db), H, I, code_of(down),
                              down.group_size, tensor_scale(gate_up), tensor_scale(down), _p(h), _p(o))
    return h, o


def expert_ffn_unfused(x_f32: np.ndarray, gate, up, down, e: int):
    x_f32 = _c(x_f32, np.float32)
    H, I = down.N, down.K
    a = _expert_slice(gate, e)
    b = _expert_slice(up, e)
    d = _expert_slice(down, e)
    h = np.empty(I, np.float32)
    o = np.empty(H, np.float32)
    _load().oracle_expert_ffn_unfused(_p(x_f32), *[_p(v) for v in a + b + d], H, I, code_of(down), down.group_size,
                                      tensor_scale(gate), tensor_scale(up), tensor_scale(down), _p(h), _p(o))
    return h, o


def tokens_forward(x: np.ndarray, dtype: str, tokens: Sequence[int], idx: np.ndarray, w: np.ndarray, k_used: int,
                   gate_up, down, want_h: bool = False):
    """fp32 layer outputs [n, H] of the listed tokens under the given routing."""
    x = _c(x, np.uint16)
    idx = _c(idx, np.int32)
    w = _c(w, np.float32)
    toks = np.ascontiguousarray(np.asarray(tokens, np.int32))
    H = x.shape[1]
    kcap = idx.shape[1]
    I = down.K
    y = np.empty((toks.size, H), np.float32)
    h = np.zeros((toks.size, kcap, I), np.float32) if want_h else None
    _load().oracle_tokens_forward(_p(x), DTYPE_CODE[dtype], H, _p(toks), toks.size, _p(idx), _p(w), kcap, k_used,
                                  _p(gate_up.q), _p(gate_up.scales), _p(gate_up.biases), _p(down.q),
                                  _p(down.scales), _p(down.biases), I, code_of(down), down.group_size,
                                  tensor_scale(gate_up), tensor_scale(down), _p(y), _p(h))
    return (y, h) if want_h else y


def layer_forward(x: np.ndarray, wr: np.ndarray, dtype: str, k: int, gate_up, down,
                  health: Optional[np.ndarray] = None, alpha: float = 0.0, groups: int = 0, capacity: int = 0):
    """The whole layer.  Returns dict(y bits, y_f32, idx, w, k_used, h_mean)."""
    x = _c(x, np.uint16)
    wr = _c(wr, np.uint16)
    T, H = x.shape
    E = wr.shape[0]
    kcap = k if k > 0 else 3
    y = np.empty((T, H), np.uint16)
    yf = np.empty((T, H), np.float32)
    idx = np.empty((T, kcap), np.int32)
    w = np.empty((T, kcap), np.float32)
    ku = np.zeros(1, np.int32)
    hm = np.zeros(1, np.float32)
    h = _c(health, np.float32)
    _load().oracle_layer_forward_ex(_p(x), DTYPE_CODE[dtype], T, H, _p(wr), E, k, _p(h), float(alpha), int(groups),
                                    int(capacity),
                                    _p(gate_up.q), _p(gate_up.scales), _p(gate_up.biases), _p(down.q),
                                    _p(down.scales), _p(down.biases), down.K, code_of(down), down.group_size,
                                    tensor_scale(gate_up), tensor_scale(down), _p(y), _p(yf), _p(idx), _p(w),
                                    _p(ku), _p(hm))
    return dict(y=y, y_f32=yf, idx=idx, w=w, k_used=int(ku[0]), h_mean=float(hm[0]))
