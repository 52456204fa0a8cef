"""Python binding of the MI355X MoE-layer library (libmoe_amd.so).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  PyTorch provides device memory and the current stream.  The names
mirror the C ABI in include/moe.h:

    route, topk_from_logits, layer_forward, fuse_gate_up,
    layer_workspace_size, route_workspace_size

If the library is not built this module raises on first use; there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_amd.so")

MOE_F16, MOE_BF16 = 1, 2
MOE_K_ENTROPY = -1
MOE_K_ENTROPY_CAP = 3
FLAG_UNFUSED, FLAG_FORCE_GEMV, FLAG_FORCE_MFMA = 0x1, 0x2, 0x4

STATUS = {0: "MOE_OK", -1: "MOE_ERR_NULL", -2: "MOE_ERR_SHAPE", -3: "MOE_ERR_DTYPE", -4: "MOE_ERR_ALIGN",
          -5: "MOE_ERR_K", -6: "MOE_ERR_QUANT", -7: "MOE_ERR_INCOMPATIBLE", -8: "MOE_ERR_WORKSPACE",
          -9: "MOE_ERR_DEVICE", -10: "MOE_ERR_HIP", -11: "MOE_ERR_INTERNAL", -12: "MOE_ERR_OPTION",
          -13: "MOE_ERR_SCRATCH"}
NOALLOC_SCRATCH_BYTES = 64 << 20

EXPORTS = ("moe_route_workspace_size", "moe_route", "moe_route_ex", "moe_topk_from_logits",
           "moe_topk_from_logits_ex", "moe_layer_workspace_size", "moe_layer_forward", "moe_layer_forward_ex",
           "moe_layer_forward_noalloc",
           "moe_expert_load_stats", "moe_fuse_gate_up", "moe_packed_sb_bytes", "moe_pack_sb", "moe_packed_q_bytes", "moe_pack_q", "moe_status_string",
           "moe_debug_set_events",
           "moe_debug_last_plan", "moe_debug_set_tuning", "moe_debug_stream_read")


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        self.name = STATUS.get(status, str(status))
        super().__init__("%s failed: %s (%s)" % (what, self.name, _status_text(status)))


class CWeights(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("biases", ctypes.c_void_p),
                ("E", ctypes.c_int32), ("N", ctypes.c_int32), ("K", ctypes.c_int32), ("bits", ctypes.c_int32),
                ("group_size", ctypes.c_int32), ("expert_stride_rows", ctypes.c_int64), ("packed_sb", ctypes.c_void_p),
                ("format", ctypes.c_int32), ("tensor_scale", ctypes.c_float), ("packed_q", ctypes.c_void_p)]


FMT_AFFINE, FMT_NVFP4 = 0, 1


class CRouteOpts(ctypes.Structure):
    _fields_ = [("health", ctypes.c_void_p), ("alpha", ctypes.c_float), ("groups", ctypes.c_int32),
                ("capacity", ctypes.c_int32)]


class CTaps(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("logits", "topk_idx", "topk_w", "k_used", "entropy", "counts", "offsets", "perm", "h",
                 "gate_up_preact")]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmoe_amd.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libmoe_amd.so is not built; run `python -m mixture_experts_router_amd.build` "
                           "(or __graft_entry__.build()) first")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    u32 = ctypes.c_uint32
    L.moe_route_workspace_size.argtypes = [i32, i32, i32]
    L.moe_route_workspace_size.restype = sz
    L.moe_route.argtypes = [vp, i32, i32, i32, vp, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_route.restype = i32
    L.moe_topk_from_logits.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]
    L.moe_topk_from_logits.restype = i32
    ropt = ctypes.POINTER(CRouteOpts)
    L.moe_route_ex.argtypes = [vp, i32, i32, i32, vp, i32, i32, ropt, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_route_ex.restype = i32
    L.moe_topk_from_logits_ex.argtypes = [vp, i32, i32, i32, ropt, vp, vp, vp, vp, vp, sz, vp]
    L.moe_topk_from_logits_ex.restype = i32
    L.moe_layer_forward_ex.argtypes = [vp, i32, i32, i32, vp, i32, i32, ropt, ctypes.POINTER(CWeights),
                                       ctypes.POINTER(CWeights), ctypes.POINTER(CWeights), ctypes.POINTER(CWeights),
                                       vp, u32, ctypes.POINTER(CTaps), vp, sz, vp]
    L.moe_layer_forward_ex.restype = i32
    L.moe_layer_forward_noalloc.argtypes = [vp, i32, i32, i32, vp, i32, i32, ropt, ctypes.POINTER(CWeights),
                                            ctypes.POINTER(CWeights), ctypes.POINTER(CWeights),
                                            ctypes.POINTER(CWeights), vp, u32, ctypes.POINTER(CTaps), vp]
    L.moe_layer_forward_noalloc.restype = i32
    L.moe_expert_load_stats.argtypes = [vp, i32, vp, vp, vp]
    L.moe_expert_load_stats.restype = i32
    L.moe_layer_workspace_size.argtypes = [i32, i32, i32, i32, i32, u32]
    L.moe_layer_workspace_size.restype = sz
    L.moe_layer_forward.argtypes = [vp, i32, i32, i32, vp, i32, i32, ctypes.POINTER(CWeights),
                                    ctypes.POINTER(CWeights), ctypes.POINTER(CWeights), ctypes.POINTER(CWeights),
                                    vp, u32, ctypes.POINTER(CTaps), vp, sz, vp]
    L.moe_layer_forward.restype = i32
    L.moe_fuse_gate_up.argtypes = [ctypes.POINTER(CWeights), ctypes.POINTER(CWeights), vp, vp, vp, vp]
    L.moe_fuse_gate_up.restype = i32
    L.moe_packed_sb_bytes.argtypes = [i32, ctypes.c_int64, i32]
    L.moe_packed_sb_bytes.restype = sz
    L.moe_pack_sb.argtypes = [ctypes.POINTER(CWeights), vp, vp]
    L.moe_packed_q_bytes.argtypes = [i32, ctypes.c_int64, i32, i32]
    L.moe_packed_q_bytes.restype = sz
    L.moe_pack_q.argtypes = [ctypes.POINTER(CWeights), vp, vp]
    L.moe_pack_sb.restype = i32
    L.moe_status_string.argtypes = [i32]
    L.moe_status_string.restype = ctypes.c_char_p
    L.moe_debug_set_events.argtypes = [vp, i32]
    L.moe_debug_set_events.restype = None
    L.moe_debug_last_plan.argtypes = [ctypes.c_char_p, sz]
    L.moe_debug_last_plan.restype = i32
    L.moe_debug_set_tuning.argtypes = [i32, i32]
    L.moe_debug_set_tuning.restype = None
    L.moe_debug_stream_read.argtypes = [vp, sz, vp, vp]
    L.moe_debug_stream_read.restype = i32
    _lib = L
    return L


def _status_text(s: int) -> str:
    try:
        return lib().moe_status_string(s).decode()
    except Exception:  # pragma: no cover
        return "?"


def _check(status: int, what: str) -> None:
    if status != 0:
        raise MoeError(status, what)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float16:
        return MOE_F16
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    raise TypeError("activations must be float16 or bfloat16, got %s" % t.dtype)


@dataclasses.dataclass
class Weights:
    """Device weight tensor [E, N, K] in the library's layout (see include/moe.h).

    bits 4: q uint8 [E, N, K/2]; bits 5 / 6: q uint8 [E, N, 5K/8] / [E, N, 3K/4]
    (code k at bits b*k..b*k+b-1 of the row's little-endian bit stream, b =
    bits; the batched path takes 5-bit rows when hidden and inter are multiples
    of 128); bits 8: q uint8 [E, N, K];
    bits 16: q float16 [E, N, K].  scales/biases float16 [E, N, K/64] (None for bits 16).
    ``fmt="nvfp4"`` (bits 4, group_size 16): q uint8 [E, N, K/2] E2M1 codes
    (even column in the low nibble), scales uint8 [E, N, K/16] E4M3 block
    scales, biases None, ``tensor_scale`` the fp32 per-tensor scale.
    ``row_offset``/``stride`` describe a view (the gate or up half of a fused
    tensor): rows start ``row_offset`` rows in, experts are ``stride`` rows apart.
    ``packed_sb`` (optional, uint8): the scales and biases repacked by pack_sb
    for the batched path (the whole tensor's; views share it).  ``packed_q``
    (optional, uint8): the codes repacked by pack_q for the batched path (the
    whole tensor's; views share it).
    """

    q: torch.Tensor
    scales: Optional[torch.Tensor]
    biases: Optional[torch.Tensor]
    E: int
    N: int
    K: int
    bits: int
    group_size: int = 64
    stride: Optional[int] = None
    row_offset: int = 0
    packed_sb: Optional[torch.Tensor] = None
    fmt: str = "affine"  # "affine" | "nvfp4"
    tensor_scale: float = 1.0
    packed_q: Optional[torch.Tensor] = None

    _cstruct: Optional[CWeights] = dataclasses.field(default=None, repr=False, compare=False)

    def c(self) -> CWeights:
        if self._cstruct is not None:
            return self._cstruct
        stride = self.N if self.stride is None else self.stride
        rb = self.K * self.bits // 8
        ng = self.K // self.group_size
        f4 = self.fmt == "nvfp4"
        srb = ng if f4 else ng * 2  # scale bytes per row
        q = self.q.data_ptr() + self.row_offset * rb
        s = None if self.scales is None else self.scales.data_ptr() + self.row_offset * srb
        b = None if self.biases is None else self.biases.data_ptr() + self.row_offset * srb
        sb = None if self.packed_sb is None else self.packed_sb.data_ptr() + self.row_offset * 8
        pq = None
        if self.packed_q is not None:
            ug = 1 if self.bits in (6, 16) else 2  # groups per unit
            nu = (self.K + 64 * ug - 1) // (64 * ug)
            pq = self.packed_q.data_ptr() + self.row_offset // 32 * nu * 32 * 8 * self.bits * ug
        self._cstruct = CWeights(q, s, b, self.E, self.N, self.K, self.bits, self.group_size, stride, sb,
                                 FMT_NVFP4 if f4 else FMT_AFFINE, float(self.tensor_scale), pq)
        return self._cstruct

    def split_gate_up(self):
        """(gate, up) views of a fused [E, 2I, K] tensor, gate rows first."""
        I = self.N // 2
        g = dataclasses.replace(self, N=I, stride=self.N, row_offset=0, _cstruct=None)
        u = dataclasses.replace(self, N=I, stride=self.N, row_offset=I, _cstruct=None)
        return g, u


def route_workspace_size(T: int, E: int, k: int) -> int:
    return int(lib().moe_route_workspace_size(T, E, k))


def layer_workspace_size(T: int, H: int, E: int, k: int, inter: int, flags: int = 0) -> int:
    return int(lib().moe_layer_workspace_size(T, H, E, k, inter, flags))


def _kcap(k: int) -> int:
    return k if k > 0 else MOE_K_ENTROPY_CAP


def _opts(health: Optional[torch.Tensor], alpha: float, groups: int, capacity: int = 0):
    """moe_route_opts for the *_ex entry points, or None when no option is set."""
    if health is None and not groups and not capacity:
        return None
    if health is not None:
        assert health.dtype == torch.float32 and health.is_contiguous()
    return CRouteOpts(_ptr(health), float(alpha), int(groups), int(capacity))


def route(x: torch.Tensor, router_w: torch.Tensor, k: int, want_logits: bool = False, stream=None,
          health: Optional[torch.Tensor] = None, alpha: float = 0.0, groups: int = 0):
    """Router + selection.  Returns dict(idx [T,kcap] int32, w [T,kcap] fp32,
    k_used [1] int32, entropy [1] fp32[, logits [T,E] fp32]).  health/alpha:
    load-aware correction of the logits; groups: at most one expert per group
    of E/groups consecutive experts (moe_route_opts)."""
    T, H = x.shape
    E = router_w.shape[0]
    dev = x.device
    kc = _kcap(k)
    idx = torch.empty((T, kc), dtype=torch.int32, device=dev)
    w = torch.empty((T, kc), dtype=torch.float32, device=dev)
    ku = torch.zeros(1, dtype=torch.int32, device=dev)
    ent = torch.zeros(1, dtype=torch.float32, device=dev)
    logits = torch.empty((T, E), dtype=torch.float32, device=dev) if want_logits else None
    ws = torch.empty(max(route_workspace_size(T, E, k), 256), dtype=torch.uint8, device=dev)
    o = _opts(health, alpha, groups)
    if o is None:
        st = lib().moe_route(_ptr(x), _dtype_code(x), T, H, _ptr(router_w), E, k, _ptr(idx), _ptr(w), _ptr(ku),
                             _ptr(ent), _ptr(logits), _ptr(ws), ws.numel(), _stream(stream))
    else:
        st = lib().moe_route_ex(_ptr(x), _dtype_code(x), T, H, _ptr(router_w), E, k, ctypes.byref(o), _ptr(idx),
                                _ptr(w), _ptr(ku), _ptr(ent), _ptr(logits), _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "moe_route")
    out = dict(idx=idx, w=w, k_used=ku, entropy=ent)
    if logits is not None:
        out["logits"] = logits
    return out


def topk_from_logits(logits: torch.Tensor, k: int, stream=None, groups: int = 0):
    T, E = logits.shape
    dev = logits.device
    kc = _kcap(k)
    idx = torch.empty((T, kc), dtype=torch.int32, device=dev)
    w = torch.empty((T, kc), dtype=torch.float32, device=dev)
    ku = torch.zeros(1, dtype=torch.int32, device=dev)
    ent = torch.zeros(1, dtype=torch.float32, device=dev)
    lg = logits.contiguous()
    if not groups:
        st = lib().moe_topk_from_logits(_ptr(lg), T, E, k, _ptr(idx), _ptr(w), _ptr(ku), _ptr(ent), None, 0,
                                        _stream(stream))
    else:
        o = CRouteOpts(None, 0.0, int(groups), 0)
        st = lib().moe_topk_from_logits_ex(_ptr(lg), T, E, k, ctypes.byref(o), _ptr(idx), _ptr(w), _ptr(ku),
                                           _ptr(ent), None, 0, _stream(stream))
    _check(st, "moe_topk_from_logits")
    return dict(idx=idx, w=w, k_used=ku, entropy=ent)


TAP_NAMES = ("logits", "topk_idx", "topk_w", "k_used", "entropy", "counts", "offsets", "perm", "h",
             "gate_up_preact")


def make_taps(T: int, E: int, k: int, inter: int, device, names: Sequence[str] = TAP_NAMES):
    """Allocate tap buffers (logits, routing, sort results, SwiGLU rows, fp32
    gate+up pre-activations)."""
    kc = _kcap(k)
    P = T * kc
    spec = dict(logits=((T, E), torch.float32), topk_idx=((T, kc), torch.int32), topk_w=((T, kc), torch.float32),
                k_used=((1,), torch.int32), entropy=((1,), torch.float32), counts=((E,), torch.int32),
                offsets=((E + 1,), torch.int32), perm=((P,), torch.int32), h=((P, inter), torch.float16),
                gate_up_preact=((P, 2 * inter), torch.float32))
    return {n: torch.zeros(spec[n][0], dtype=spec[n][1], device=device) for n in names}


def layer_forward(x: torch.Tensor, router_w: torch.Tensor, k: int, down: Weights, gate_up: Optional[Weights] = None,
                  gate: Optional[Weights] = None, up: Optional[Weights] = None, flags: int = 0,
                  taps: Optional[dict] = None, out: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None, stream=None, health: Optional[torch.Tensor] = None,
                  alpha: float = 0.0, groups: int = 0, capacity: int = 0) -> torch.Tensor:
    """The whole layer: y [T, H] in the activation dtype (routing options as in
    route(); capacity > 0: at most that many pairs per expert, moe_route_opts)."""
    T, H = x.shape
    E = router_w.shape[0]
    inter = down.K
    y = torch.empty_like(x) if out is None else out
    need = layer_workspace_size(T, H, E, k, inter, flags)
    ws = workspace
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
    ctaps = None
    if taps:
        ctaps = CTaps(*[(taps[n].data_ptr() if n in taps and taps[n] is not None else None) for n in TAP_NAMES])
    cgu = gate_up.c() if gate_up is not None else None
    cg = gate.c() if gate is not None else None
    cu = up.c() if up is not None else None
    cd = down.c()
    wargs = (ctypes.byref(cgu) if cgu is not None else None, ctypes.byref(cg) if cg is not None else None,
             ctypes.byref(cu) if cu is not None else None, ctypes.byref(cd), _ptr(y), flags,
             ctypes.byref(ctaps) if ctaps is not None else None, _ptr(ws), ws.numel(), _stream(stream))
    o = _opts(health, alpha, groups, capacity)
    if o is None:
        st = lib().moe_layer_forward(_ptr(x), _dtype_code(x), T, H, _ptr(router_w), E, k, *wargs)
    else:
        st = lib().moe_layer_forward_ex(_ptr(x), _dtype_code(x), T, H, _ptr(router_w), E, k, ctypes.byref(o),
                                        *wargs)
    _check(st, "moe_layer_forward")
    return y


def layer_forward_noalloc(x: torch.Tensor, router_w: torch.Tensor, k: int, down: Weights,
                          gate_up: Optional[Weights] = None, gate: Optional[Weights] = None,
                          up: Optional[Weights] = None, flags: int = 0, taps: Optional[dict] = None,
                          out: Optional[torch.Tensor] = None, stream=None, health: Optional[torch.Tensor] = None,
                          alpha: float = 0.0, groups: int = 0, capacity: int = 0) -> torch.Tensor:
    """layer_forward through moe_layer_forward_noalloc: no workspace argument,
    the library's per-device scratch array instead (calls on one GPU must not
    overlap).  With `out` given, nothing is allocated."""
    T, H = x.shape
    E = router_w.shape[0]
    y = torch.empty_like(x) if out is None else out
    ctaps = None
    if taps:
        ctaps = CTaps(*[(taps[n].data_ptr() if n in taps and taps[n] is not None else None) for n in TAP_NAMES])
    ref = lambda w: ctypes.byref(w.c()) if w is not None else None
    o = _opts(health, alpha, groups, capacity)
    st = lib().moe_layer_forward_noalloc(_ptr(x), _dtype_code(x), T, H, _ptr(router_w), E, k,
                                         ctypes.byref(o) if o is not None else None, ref(gate_up), ref(gate),
                                         ref(up), ref(down), _ptr(y), flags,
                                         ctypes.byref(ctaps) if ctaps is not None else None, _stream(stream))
    _check(st, "moe_layer_forward_noalloc")
    return y


def expert_load_stats(counts: torch.Tensor, stream=None):
    """(least-used expert [1] int32, standard deviation [1] fp32) of int32 counts [E] on the device."""
    assert counts.dtype == torch.int32 and counts.dim() == 1 and counts.is_contiguous()
    lu = torch.empty(1, dtype=torch.int32, device=counts.device)
    sd = torch.empty(1, dtype=torch.float32, device=counts.device)
    _check(lib().moe_expert_load_stats(_ptr(counts), counts.numel(), _ptr(lu), _ptr(sd), _stream(stream)),
           "moe_expert_load_stats")
    return lu, sd


def fuse_gate_up(gate: Weights, up: Weights, stream=None) -> Weights:
    """Pack gate [E, I, K] and up [E, I, K] into a new fused [E, 2I, K] tensor."""
    E, I, K, bits = gate.E, gate.N, gate.K, gate.bits
    dev = gate.q.device
    qshape = (E, 2 * I) + tuple(gate.q.shape[2:])
    q = torch.empty(qshape, dtype=gate.q.dtype, device=dev)
    s = b = None
    if gate.scales is not None:
        sdt = torch.uint8 if gate.fmt == "nvfp4" else torch.float16
        s = torch.empty((E, 2 * I, K // gate.group_size), dtype=sdt, device=dev)
    if gate.biases is not None:
        b = torch.empty((E, 2 * I, K // gate.group_size), dtype=torch.float16, device=dev)
    cg, cu = gate.c(), up.c()
    st = lib().moe_fuse_gate_up(ctypes.byref(cg), ctypes.byref(cu), _ptr(q), _ptr(s), _ptr(b), _stream(stream))
    _check(st, "moe_fuse_gate_up")
    return Weights(q, s, b, E, 2 * I, K, bits, gate.group_size, fmt=gate.fmt, tensor_scale=gate.tensor_scale)


def pack_sb(w: Weights, stream=None) -> Weights:
    """The same weights with packed_sb filled (scales and biases in the batched
    path's layout; a one-time repack, like fusing gate and up)."""
    if w.bits == 16 or w.row_offset != 0:
        raise ValueError("pack_sb: needs a whole quantised tensor")
    stride = w.N if w.stride is None else w.stride
    nbytes = int(lib().moe_packed_sb_bytes(w.E, stride, w.K))
    out = torch.empty(nbytes, dtype=torch.uint8, device=w.q.device)
    _check(lib().moe_pack_sb(ctypes.byref(w.c()), _ptr(out), _stream(stream)), "moe_pack_sb")
    return dataclasses.replace(w, packed_sb=out, _cstruct=None)


def pack_q(w: Weights, stream=None) -> Weights:
    """The same weights with packed_q filled (the codes in the batched path's
    block layout; a one-time repack, a second copy of the codes)."""
    if w.row_offset != 0:
        raise ValueError("pack_q: needs a whole tensor")
    stride = w.N if w.stride is None else w.stride
    nbytes = int(lib().moe_packed_q_bytes(w.E, stride, w.K, w.bits))
    if nbytes == 0:
        raise ValueError("pack_q: rows per expert and N must be multiples of 32")
    out = torch.empty(nbytes, dtype=torch.uint8, device=w.q.device)
    _check(lib().moe_pack_q(ctypes.byref(w.c()), _ptr(out), _stream(stream)), "moe_pack_q")
    return dataclasses.replace(w, packed_q=out, _cstruct=None)


def debug_set_events(events: Optional[Sequence]) -> None:
    """Record the given torch.cuda.Events around each kernel of later calls on this thread."""
    if not events:
        lib().moe_debug_set_events(None, 0)
        debug_set_events._keep = None
        return
    arr = (ctypes.c_void_p * len(events))(*[e.cuda_event for e in events])
    debug_set_events._keep = arr  # keep the array alive while the library holds it
    lib().moe_debug_set_events(ctypes.cast(arr, ctypes.c_void_p), len(events))


def debug_set_tuning(key: int, value: int) -> None:
    """Launch-shape knob (0: decode gate+up waves/CU, 1: decode down waves/CU, 2: GEMM row tiles per group,
    3: GEMM row tile 32/64/128 (else automatic), 4: GEMM K groups per stage (1 or 2), 5: GEMM N subtiles
    per wave (2 or 4), 6: GEMM waves per column block (1 or 2), 7: GEMM workgroups per CU at 32/64-row
    tiles (1 or 2; 3 for 4-bit and NVFP4 weights at 64-row tiles), 8: decode gate+up waves per pair (2: from the wave target alone, else equal iterations
    per wave), 9: tokens per small-batch router workgroup at eight experts each (1, 2 or 4; default 2))."""
    lib().moe_debug_set_tuning(int(key), int(value))


STREAM_READ_WAVES = 8192


def debug_stream_read(src: torch.Tensor, sink: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """The streaming-read reference over all of `src` (see moe_debug_stream_read);
    returns the int32 sink [STREAM_READ_WAVES] of per-wave XORs."""
    if sink is None:
        sink = torch.empty(STREAM_READ_WAVES, dtype=torch.int32, device=src.device)
    nbytes = src.numel() * src.element_size()
    _check(lib().moe_debug_stream_read(_ptr(src), nbytes, _ptr(sink), _stream(stream)), "moe_debug_stream_read")
    return sink


def source_hash() -> str:
    """sha256 over the library's sources (identifies which kernels a profile measured)."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(_HERE, "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def last_plan() -> list:
    buf = ctypes.create_string_buffer(1024)
    lib().moe_debug_last_plan(buf, 1024)
    s = buf.value.decode()
    return s.split(",") if s else []
