"""The C ABI on the CPU: the library loads, exports what include/moe.h
declares, and validates arguments on the host before touching a device.

Pointers here are fake aligned addresses: validation never dereferences them,
and every call below returns before the first HIP call (or, for the valid
call without a GPU, at the device check).
"""
import ctypes
import os
import re
import subprocess

import pytest

import mixture_experts_router_amd as moe
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "moe.h")
P = 0x100000  # a 16-byte aligned fake address


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    names = header_functions()
    assert "moe_route" in names and "moe_layer_forward" in names
    out = subprocess.run(["nm", "-D", "--defined-only", moe.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r" T (\w+)$", out, flags=re.M))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    assert set(moe.EXPORTS) == set(names)


def test_status_strings():
    L = moe.lib()
    for code, name in moe.STATUS.items():
        s = L.moe_status_string(code).decode()
        assert s and s != "unknown status", name
    assert L.moe_status_string(12345).decode() == "unknown status"


def W(E, N, K, bits=4, q=P, s=P, b=P, gs=64, stride=None, sb=None):
    return moe.CWeights(q, None if bits == 16 else s, None if bits == 16 else b, E, N, K, bits, gs,
                        N if stride is None else stride, sb)


def fwd(T=4, H=256, E=8, k=2, I=128, dt=moe.MOE_F16, x=P, wr=P, y=P, gu="fused", gate=None, up=None, down=None,
        flags=0, ws=P, ws_bytes=None, bits=4):
    L = moe.lib()
    if gu == "fused":
        gu = W(E, 2 * I, H, bits)
    down = W(E, H, I, bits) if down is None else down
    if ws_bytes is None:
        ws_bytes = L.moe_layer_workspace_size(T, H, E, k, I, flags)
    ref = lambda w: ctypes.byref(w) if w is not None else None
    return L.moe_layer_forward(x, dt, T, H, wr, E, k, ref(gu), ref(gate), ref(up), ref(down), y, flags, None, ws,
                               ws_bytes, None)


def test_zero_tokens_is_a_noop():
    assert fwd(T=0) == 0
    assert fwd(T=0, x=None, y=None, ws=None) == 0  # empty tensors have NULL data pointers


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), "MOE_ERR_NULL"),
    (dict(wr=None), "MOE_ERR_NULL"),
    (dict(y=None), "MOE_ERR_NULL"),
    (dict(gu=None), "MOE_ERR_NULL"),
    (dict(dt=3), "MOE_ERR_DTYPE"),
    (dict(H=200), "MOE_ERR_SHAPE"),
    (dict(E=0), "MOE_ERR_SHAPE"),
    (dict(E=257, k=2), "MOE_ERR_SHAPE"),
    (dict(k=0), "MOE_ERR_K"),
    (dict(k=9, E=16), "MOE_ERR_K"),
    (dict(k=5, E=4), "MOE_ERR_K"),
    (dict(k=-1, E=2), "MOE_ERR_K"),
    (dict(k=-2), "MOE_ERR_K"),
    (dict(I=100, down=W(8, 256, 100)), "MOE_ERR_SHAPE"),
    (dict(x=P + 8), "MOE_ERR_ALIGN"),
    (dict(y=P + 2), "MOE_ERR_ALIGN"),
    (dict(ws=None), "MOE_ERR_WORKSPACE"),
    (dict(ws_bytes=1024), "MOE_ERR_WORKSPACE"),
    (dict(ws=P + 16), "MOE_ERR_ALIGN"),
    (dict(gu=W(8, 2 * 128, 256, bits=7)), "MOE_ERR_QUANT"),
    (dict(gu=W(8, 2 * 128, 256, bits=3)), "MOE_ERR_QUANT"),
    (dict(gu=W(8, 2 * 128, 256, gs=32)), "MOE_ERR_QUANT"),
    (dict(gu=W(8, 2 * 128, 256, s=None)), "MOE_ERR_NULL"),
    (dict(gu=W(8, 2 * 128, 256, q=P + 4)), "MOE_ERR_ALIGN"),
    (dict(gu=W(8, 2 * 100, 256)), "MOE_ERR_SHAPE"),
    (dict(gu=W(7, 2 * 128, 256)), "MOE_ERR_SHAPE"),
    (dict(gu=W(8, 2 * 128, 256, stride=100)), "MOE_ERR_SHAPE"),
    (dict(gu=W(8, 2 * 128, 256, bits=8)), "MOE_ERR_QUANT"),
    (dict(down=W(8, 256, 128, bits=16)), "MOE_ERR_QUANT"),
    (dict(gu=W(8, 2 * 128, 256, sb=P + 8)), "MOE_ERR_ALIGN"),
    (dict(down=W(8, 256, 128, sb=P + 4)), "MOE_ERR_ALIGN"),
    # packed_sb holds scales and biases: quantised weights only
    (dict(gu=W(8, 2 * 128, 256, bits=16, sb=P), down=W(8, 256, 128, bits=16), bits=16), "MOE_ERR_QUANT"),
    # 5-bit codes on the batched path: hidden and inter multiples of 128
    (dict(I=192, gu=W(8, 2 * 192, 256, bits=5), down=W(8, 256, 192, bits=5), bits=5,
          flags=moe.FLAG_FORCE_MFMA), "MOE_ERR_QUANT"),
    (dict(H=320, gu=W(8, 2 * 128, 320, bits=5), down=W(8, 320, 128, bits=5), bits=5,
          flags=moe.FLAG_FORCE_MFMA), "MOE_ERR_QUANT"),
])
def test_validation_errors(kw, status):
    assert moe.STATUS[fwd(**kw)] == status


def test_bits16_rejects_scales():
    bad = moe.CWeights(P, P, P, 8, 256, 256, 16, 64, 256)
    assert moe.STATUS[fwd(gu=bad, down=W(8, 256, 128, bits=16), bits=16)] == "MOE_ERR_QUANT"


def test_separate_gate_up_must_be_compatible():
    # the _can_fuse rule of the oMLX page: same bits, group size, shape, scale presence
    ok = W(8, 128, 256)
    assert moe.STATUS[fwd(gu=None, gate=ok, up=W(8, 128, 256, bits=8))] == "MOE_ERR_INCOMPATIBLE"
    assert moe.STATUS[fwd(gu=None, gate=ok, up=W(8, 128, 256, gs=32))] == "MOE_ERR_INCOMPATIBLE"
    assert moe.STATUS[fwd(gu=None, gate=ok, up=W(8, 64, 256))] == "MOE_ERR_INCOMPATIBLE"
    assert moe.STATUS[fwd(gu=None, gate=ok, up=None)] == "MOE_ERR_NULL"


def test_packed_sb_size_and_validation():
    L = moe.lib()
    # E * ceil(K/128) * rows * 8: odd group counts round up to a pair
    assert L.moe_packed_sb_bytes(8, 256, 256) == 8 * 2 * 256 * 8
    assert L.moe_packed_sb_bytes(4, 100, 192) == 4 * 2 * 100 * 8
    assert L.moe_packed_sb_bytes(64, 2816, 4096) == 64 * 32 * 2816 * 8
    assert L.moe_packed_sb_bytes(0, 256, 256) == 0 and L.moe_packed_sb_bytes(8, 256, 100) == 0
    w = W(8, 256, 256)
    assert moe.STATUS[L.moe_pack_sb(ctypes.byref(w), None, None)] == "MOE_ERR_NULL"
    assert moe.STATUS[L.moe_pack_sb(None, P, None)] == "MOE_ERR_NULL"
    assert moe.STATUS[L.moe_pack_sb(ctypes.byref(w), P + 8, None)] == "MOE_ERR_ALIGN"
    w16 = W(8, 256, 256, bits=16)
    assert moe.STATUS[L.moe_pack_sb(ctypes.byref(w16), P, None)] == "MOE_ERR_QUANT"
    bad = W(8, 256, 200)
    assert moe.STATUS[L.moe_pack_sb(ctypes.byref(bad), P, None)] == "MOE_ERR_SHAPE"


def test_fuse_gate_up_validation():
    L = moe.lib()
    g, u = W(8, 128, 256), W(8, 128, 256, bits=8)
    assert moe.STATUS[L.moe_fuse_gate_up(ctypes.byref(g), ctypes.byref(u), P, P, P, None)] == "MOE_ERR_INCOMPATIBLE"
    u = W(8, 128, 512)
    assert moe.STATUS[L.moe_fuse_gate_up(ctypes.byref(g), ctypes.byref(u), P, P, P, None)] == "MOE_ERR_INCOMPATIBLE"
    u = W(8, 128, 256)
    assert moe.STATUS[L.moe_fuse_gate_up(ctypes.byref(g), ctypes.byref(u), None, P, P, None)] == "MOE_ERR_NULL"
    assert moe.STATUS[L.moe_fuse_gate_up(ctypes.byref(g), ctypes.byref(u), P, None, P, None)] == "MOE_ERR_NULL"
    assert moe.STATUS[L.moe_fuse_gate_up(ctypes.byref(g), ctypes.byref(u), P + 8, P, P, None)] == "MOE_ERR_ALIGN"


def F4(E, N, K, q=P, s=P, b=None, gs=16, ts=0.01, bits=4, fmt=moe.FMT_NVFP4, stride=None):
    return moe.CWeights(q, s, b, E, N, K, bits, gs, N if stride is None else stride, None, fmt, ts)


def test_nvfp4_weights_validation():
    ok_gu, ok_d = F4(8, 256, 256), F4(8, 256, 128)
    assert fwd(T=0, gu=ok_gu, down=ok_d) == 0
    for bad, status in [
        (F4(8, 256, 256, bits=8), "MOE_ERR_QUANT"),     # E2M1 codes are 4 bits
        (F4(8, 256, 256, gs=64), "MOE_ERR_QUANT"),      # one block scale per 16 columns
        (F4(8, 256, 256, b=P), "MOE_ERR_QUANT"),        # no biases
        (F4(8, 256, 256, ts=0.0), "MOE_ERR_QUANT"),
        (F4(8, 256, 256, ts=-1.0), "MOE_ERR_QUANT"),
        (F4(8, 256, 256, ts=float("nan")), "MOE_ERR_QUANT"),
        (F4(8, 256, 256, ts=float("inf")), "MOE_ERR_QUANT"),
        (F4(8, 256, 256, s=None), "MOE_ERR_NULL"),
        (F4(8, 256, 256, s=P + 4), "MOE_ERR_ALIGN"),
        (F4(8, 256, 256, fmt=2), "MOE_ERR_QUANT"),
        (F4(8, 256, 200), "MOE_ERR_SHAPE"),
    ]:
        assert moe.STATUS[fwd(T=4, gu=bad, down=ok_d)] == status, (bad.bits, bad.group_size, bad.tensor_scale)
    # gate_up and down in one format
    assert moe.STATUS[fwd(gu=ok_gu, down=W(8, 256, 128))] == "MOE_ERR_QUANT"
    assert moe.STATUS[fwd(gu=W(8, 256, 256), down=ok_d)] == "MOE_ERR_QUANT"
    # separate gate and up: one format; their tensor scales may differ
    assert moe.STATUS[fwd(gu=None, gate=F4(8, 128, 256), up=W(8, 128, 256), down=ok_d)] == "MOE_ERR_INCOMPATIBLE"
    assert fwd(T=0, gu=None, gate=F4(8, 128, 256, ts=0.5), up=F4(8, 128, 256, ts=0.25), down=ok_d) == 0


def test_nvfp4_fuse_and_pack_validation():
    L = moe.lib()
    g = F4(8, 128, 256)
    # a fused tensor holds one tensor scale
    u = F4(8, 128, 256, ts=0.02)
    assert moe.STATUS[L.moe_fuse_gate_up(ctypes.byref(g), ctypes.byref(u), P, P, None, None)] == \
        "MOE_ERR_INCOMPATIBLE"
    u = F4(8, 128, 256)
    assert moe.STATUS[L.moe_fuse_gate_up(ctypes.byref(g), ctypes.byref(u), P, P, P, None)] == "MOE_ERR_QUANT"
    assert moe.STATUS[L.moe_fuse_gate_up(ctypes.byref(g), ctypes.byref(u), P, None, None, None)] == "MOE_ERR_NULL"
    assert moe.STATUS[L.moe_pack_sb(ctypes.byref(F4(8, 256, 256, gs=64)), P, None)] == "MOE_ERR_QUANT"


def test_packed_q_size_and_validation():
    L = moe.lib()
    # E * (rows/32) * units * 32 * unit bytes; two-group units for 4/5/8 bits, one group for 6 and 16
    assert L.moe_packed_q_bytes(8, 256, 256, 4) == 8 * 8 * 2 * 32 * 64
    assert L.moe_packed_q_bytes(8, 256, 192, 5) == 8 * 8 * 2 * 32 * 80
    assert L.moe_packed_q_bytes(8, 256, 192, 8) == 8 * 8 * 2 * 32 * 128
    assert L.moe_packed_q_bytes(2, 64, 64, 6) == 2 * 2 * 1 * 32 * 48
    assert L.moe_packed_q_bytes(2, 64, 192, 6) == 2 * 2 * 3 * 32 * 48
    assert L.moe_packed_q_bytes(64, 2816, 4096, 4) == 64 * 88 * 32 * 32 * 64
    assert L.moe_packed_q_bytes(4, 96, 4096, 16) == 4 * 3 * 64 * 32 * 128
    for bad in [(0, 256, 256, 4), (8, 100, 256, 4), (8, 256, 200, 4), (8, 256, 256, 7)]:
        assert L.moe_packed_q_bytes(*bad) == 0, bad
    w = W(8, 256, 256)
    assert moe.STATUS[L.moe_pack_q(ctypes.byref(w), None, None)] == "MOE_ERR_NULL"
    assert moe.STATUS[L.moe_pack_q(ctypes.byref(w), P + 8, None)] == "MOE_ERR_ALIGN"
    assert moe.STATUS[L.moe_pack_q(ctypes.byref(W(8, 256, 256, stride=272)), P, None)] == "MOE_ERR_SHAPE"
    # the layer: packed codes 16-byte aligned, whole 32-row blocks, gate and up alike
    def wq(E, N, K, pq, stride=None):
        c = W(E, N, K, stride=stride)
        c.packed_q = pq
        return c
    assert moe.STATUS[fwd(gu=wq(8, 256, 256, P + 8))] == "MOE_ERR_ALIGN"
    assert moe.STATUS[fwd(gu=wq(8, 256, 256, P, stride=272))] == "MOE_ERR_SHAPE"
    assert moe.STATUS[fwd(gu=None, gate=wq(8, 128, 256, P), up=W(8, 128, 256))] == "MOE_ERR_INCOMPATIBLE"
    assert fwd(T=0, gu=None, gate=wq(8, 128, 256, P), up=wq(8, 128, 256, P)) == 0


def test_stream_read_validation():
    L = moe.lib()
    sink = P + 1024
    assert moe.STATUS[L.moe_debug_stream_read(None, 1024, sink, None)] == "MOE_ERR_NULL"
    assert moe.STATUS[L.moe_debug_stream_read(P, 1024, None, None)] == "MOE_ERR_NULL"
    assert moe.STATUS[L.moe_debug_stream_read(P + 8, 1024, sink, None)] == "MOE_ERR_ALIGN"
    assert moe.STATUS[L.moe_debug_stream_read(P, 1024, sink + 2, None)] == "MOE_ERR_ALIGN"
    for bad in (0, 15, 1000, 1 << 32):
        assert moe.STATUS[L.moe_debug_stream_read(P, bad, sink, None)] == "MOE_ERR_SHAPE", bad


def test_route_validation():
    L = moe.lib()
    ws = 1 << 20
    call = lambda **kw: L.moe_route(kw.get("x", P), kw.get("dt", 1), kw.get("T", 4), kw.get("H", 256),
                                    kw.get("wr", P), kw.get("E", 8), kw.get("k", 2), kw.get("idx", P),
                                    kw.get("w", P), None, None, kw.get("logits", None), kw.get("ws", P),
                                    kw.get("ws_bytes", ws), None)
    assert call(T=0) == 0
    assert call(T=0, x=None, idx=None, w=None, ws=None) == 0
    assert moe.STATUS[call(x=None)] == "MOE_ERR_NULL"
    assert moe.STATUS[call(idx=None)] == "MOE_ERR_NULL"
    assert moe.STATUS[call(k=3, E=2)] == "MOE_ERR_K"
    assert moe.STATUS[call(H=100)] == "MOE_ERR_SHAPE"
    assert moe.STATUS[call(ws=None)] == "MOE_ERR_WORKSPACE"
    assert moe.STATUS[call(ws_bytes=16)] == "MOE_ERR_WORKSPACE"
    assert moe.STATUS[L.moe_topk_from_logits(None, 4, 8, 2, P, P, None, None, None, 0, None)] == "MOE_ERR_NULL"
    assert moe.STATUS[L.moe_topk_from_logits(P, 4, 8, 9, P, P, None, None, None, 0, None)] == "MOE_ERR_K"


def test_workspace_size_is_host_arithmetic():
    L = moe.lib()
    a = L.moe_layer_workspace_size(4096, 4096, 64, 4, 1408, 0)
    b = L.moe_layer_workspace_size(4096, 4096, 64, 4, 1408, moe.FLAG_UNFUSED)
    P_ = 4096 * 4
    # h (fp16 [P, I]) and o (fp16 [P, H]) dominate; unfused adds g and u in fp32
    assert a >= P_ * 1408 * 2 + P_ * 4096 * 2
    assert b - a >= 2 * P_ * 1408 * 4
    assert L.moe_layer_workspace_size(1, 4096, 64, -1, 11008, 0) > L.moe_layer_workspace_size(1, 4096, 64, 1, 11008, 0)
    assert L.moe_layer_workspace_size(0, 4096, 64, 4, 11008, 0) > 0
    assert L.moe_route_workspace_size(512, 32, -1) >= 512 * 32 * 4


def test_valid_call_without_gpu_reports_no_device():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    assert moe.STATUS[fwd()] == "MOE_ERR_DEVICE"


def test_debug_plan_hooks_are_callable_without_gpu():
    L = moe.lib()
    L.moe_debug_set_events(None, 0)
    buf = ctypes.create_string_buffer(64)
    assert L.moe_debug_last_plan(buf, 64) >= 0


def test_route_options_validation():
    """moe_route_opts: group count, k against the groups, health alignment,
    and health refused where the logits are taken as final."""
    L = moe.lib()
    ws = 1 << 20
    O = lambda health=None, alpha=0.0, groups=0, capacity=0: ctypes.byref(moe.CRouteOpts(health, alpha, groups, capacity))
    call = lambda opts, E=8, k=2: L.moe_route_ex(P, 1, 4, 256, P, E, k, opts, P, P, None, None, None, P, ws, None)
    st = lambda v: moe.STATUS[v]
    assert st(call(O(groups=-1))) == "MOE_ERR_OPTION"
    assert st(call(O(groups=3))) == "MOE_ERR_OPTION"          # 8 % 3 != 0
    assert st(call(O(groups=2), k=4)) == "MOE_ERR_OPTION"     # one per group: k <= groups
    assert st(call(O(groups=2), k=-1)) == "MOE_ERR_OPTION"    # entropy mode needs 3 groups
    assert st(call(O(health=P + 2, alpha=1.0))) == "MOE_ERR_ALIGN"
    # valid options get past validation to the device check (no GPU here)
    import torch
    if not torch.cuda.is_available():
        for o in (None, O(groups=4), O(groups=1), O(health=P, alpha=0.5, groups=2), O(groups=8, health=P)):
            assert st(call(o)) == "MOE_ERR_DEVICE"
        assert st(call(O(groups=4), k=-1, E=12)) == "MOE_ERR_DEVICE"
    tk = lambda opts, k=2: L.moe_topk_from_logits_ex(P, 4, 8, k, opts, P, P, None, None, None, 0, None)
    assert st(tk(O(health=P))) == "MOE_ERR_OPTION"
    assert st(tk(O(groups=2), k=3)) == "MOE_ERR_OPTION"
    # the layer entry point applies the same checks
    ref = lambda w: ctypes.byref(w)
    gu, dn = W(8, 256, 256), W(8, 256, 128)
    lay = lambda opts: L.moe_layer_forward_ex(P, 1, 4, 256, P, 8, 2, opts, ref(gu), None, None, ref(dn), P, 0, None,
                                              P, L.moe_layer_workspace_size(4, 256, 8, 2, 128, 0), None)
    assert st(lay(O(groups=5))) == "MOE_ERR_OPTION"
    assert st(lay(O(capacity=-1))) == "MOE_ERR_OPTION"
    assert st(call(O(capacity=4))) == "MOE_ERR_OPTION"  # a dispatch option: layer only
    assert st(tk(O(capacity=4))) == "MOE_ERR_OPTION"
    if not torch.cuda.is_available():
        assert st(lay(O(capacity=3))) == "MOE_ERR_DEVICE"
    assert st(lay(O(health=P + 1))) == "MOE_ERR_ALIGN"


def test_load_stats_validation():
    L = moe.lib()
    st = lambda v: moe.STATUS[v]
    assert st(L.moe_expert_load_stats(P, 0, P, P, None)) == "MOE_ERR_SHAPE"
    assert st(L.moe_expert_load_stats(P, 257, P, P, None)) == "MOE_ERR_SHAPE"
    assert st(L.moe_expert_load_stats(None, 8, P, P, None)) == "MOE_ERR_NULL"
    assert st(L.moe_expert_load_stats(P, 8, P + 2, P, None)) == "MOE_ERR_ALIGN"


def noalloc(T=4, H=256, E=8, k=2, I=128, x=P, wr=P, y=P, gu=None, down=None, bits=4, flags=0):
    L = moe.lib()
    gu = W(E, 2 * I, H, bits) if gu is None else gu
    down = W(E, H, I, bits) if down is None else down
    return L.moe_layer_forward_noalloc(x, moe.MOE_F16, T, H, wr, E, k, None, ctypes.byref(gu), None, None,
                                       ctypes.byref(down), y, flags, None, None)


def test_noalloc_validates_on_the_host():
    # no workspace argument; the same checks as moe_layer_forward, all before any HIP call
    assert noalloc(T=0) == 0
    assert moe.STATUS[noalloc(x=None)] == "MOE_ERR_NULL"
    assert moe.STATUS[noalloc(k=9, E=16)] == "MOE_ERR_K"
    assert moe.STATUS[noalloc(H=200)] == "MOE_ERR_SHAPE"


def test_noalloc_refuses_calls_beyond_its_scratch():
    # a 4096-token prefill (h, o and the fp16 operand alone are ~214 MB) does
    # not fit the 64 MiB array: refused before the device is touched
    st = noalloc(T=4096, H=4096, E=64, k=4, I=1408)
    assert moe.STATUS[st] == "MOE_ERR_SCRATCH"
    assert "MOE_NOALLOC_SCRATCH_BYTES" in moe.lib().moe_status_string(st).decode()
    # a decode-sized call fits: it passes validation and stops at the device
    # check here (no GPU in this process), never at the size check
    st = noalloc(T=1, H=4096, E=64, k=4, I=11008)
    assert moe.STATUS[st] != "MOE_ERR_SCRATCH"
