"""Helpers shared by the GPU tests: moving generated inputs to the device and
comparing the HIP path with the oracle under the acceptance rules.

Acceptance (layer output against the oracle's fp32 result): max-abs error
<= 2e-2 and relative L2 error <= 5e-3.  Routing is compared on identical
logits (the GPU logits fed to the oracle's selection must give the GPU's
experts exactly); where the oracle's own fp32 logits put the k-th and
(k+1)-th experts within 1e-4 of each other the two sides may legitimately
select differently, and that token is compared under the GPU's routing.
"""
import numpy as np
import torch

import mixture_experts_router_amd as moe
import moe_inputs as mi
import oracle
from ref64 import half64

MAX_ABS = 2e-2
REL_L2 = 5e-3
NEAR_TIE = 1e-4


def dev_half(u16: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(u16).view(np.int16))
    return t.view(torch.float16 if dtype == "f16" else torch.bfloat16).cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def dev_weights(w: mi.Weights) -> moe.Weights:
    if w.bits == 16:
        q = torch.from_numpy(np.ascontiguousarray(w.q).view(np.int16)).view(torch.float16).cuda()
        return moe.Weights(q, None, None, w.E, w.N, w.K, 16)
    q = torch.from_numpy(np.ascontiguousarray(w.q)).cuda()
    if w.fmt == "nvfp4":
        s = torch.from_numpy(np.ascontiguousarray(w.scales)).cuda()
        return moe.Weights(q, s, None, w.E, w.N, w.K, 4, 16, fmt="nvfp4", tensor_scale=w.tensor_scale)
    s = torch.from_numpy(np.ascontiguousarray(w.scales).view(np.int16)).view(torch.float16).cuda()
    b = torch.from_numpy(np.ascontiguousarray(w.biases).view(np.int16)).view(torch.float16).cuda()
    return moe.Weights(q, s, b, w.E, w.N, w.K, w.bits)


class Dev:
    """Device copies of one LayerInputs (gate and up kept separate; fused on the GPU)."""

    def __init__(self, inp: mi.LayerInputs, fuse: bool = True):
        self.inp = inp
        self.x = dev_half(inp.x, inp.dtype)
        self.wr = dev_half(inp.wr, inp.dtype)
        self.gate = dev_weights(inp.gate)
        self.up = dev_weights(inp.up)
        self.down = dev_weights(inp.down)
        self.gate_up = moe.fuse_gate_up(self.gate, self.up) if fuse else None

    def forward(self, flags=0, fused_tensor=True, taps=None, x=None):
        kw = dict(gate_up=self.gate_up) if fused_tensor else dict(gate=self.gate, up=self.up)
        y = moe.layer_forward(self.x if x is None else x, self.wr, self.inp.k, self.down, flags=flags, taps=taps, **kw)
        torch.cuda.synchronize()
        return y


def batched_path_takes(inp: mi.LayerInputs) -> bool:
    """Whether the batched (MFMA) path takes these weights: every width, with
    hidden and inter multiples of 128 for 5-bit codes (two-group stages)."""
    return inp.bits != 5 or (inp.H % 128 == 0 and inp.I % 128 == 0)


def boundary_gap(logits_row: np.ndarray, k: int) -> float:
    s = np.sort(logits_row.astype(np.float64))[::-1]
    return float(s[k - 1] - s[k]) if k < s.size else np.inf


def check_routing_identical_logits(gpu_logits, gpu_idx, gpu_w, k_used):
    """GPU selection == oracle selection on the GPU's own logits (bit-exact indices)."""
    kcap = gpu_idx.shape[1]
    oi, ow = oracle.select_topk(gpu_logits, k_used, kcap)
    assert np.array_equal(oi, gpu_idx), "selection differs on identical logits"
    assert np.max(np.abs(ow - gpu_w)) <= 1e-6


def reference_outputs(inp: mi.LayerInputs, gate_up_np, tokens, gpu_idx, gpu_w, gpu_k_used):
    """Oracle fp32 outputs of the listed tokens, plus routing agreement stats.

    Tokens whose oracle routing differs from the GPU's are accepted only at a
    near-tie of the oracle logits; their reference is computed under the GPU
    routing.
    """
    idx_o, w_o, ku_o, hm_o, logits_o = oracle.route(inp.x, inp.wr, inp.dtype, inp.k, want_logits=True)
    assert ku_o == gpu_k_used, "k_used differs: oracle %d (H=%.5f) gpu %d" % (ku_o, hm_o, gpu_k_used)
    toks = np.asarray(tokens)
    same = np.all(idx_o[toks] == gpu_idx[toks], axis=1)
    flips = toks[~same]
    for t in flips:
        gap = boundary_gap(logits_o[t], ku_o)
        assert gap < NEAR_TIE, "token %d routed differently with gap %.3g" % (t, gap)
    y = oracle.tokens_forward(inp.x, inp.dtype, toks[same], idx_o, w_o, ku_o, gate_up_np, inp.down) if same.any() \
        else np.zeros((0, inp.H), np.float32)
    out = np.zeros((toks.size, inp.H), np.float32)
    out[same] = y
    if flips.size:
        out[~same] = oracle.tokens_forward(inp.x, inp.dtype, flips, gpu_idx, gpu_w, gpu_k_used, gate_up_np, inp.down)
    return out, int(flips.size)


def errors(y_bits: np.ndarray, y_ref: np.ndarray, dtype: str):
    y = half64(y_bits, dtype)
    d = y - y_ref.astype(np.float64)
    max_abs = float(np.max(np.abs(d))) if d.size else 0.0
    rel = float(np.linalg.norm(d) / max(np.linalg.norm(y_ref.astype(np.float64)), 1e-30))
    floor = half64(oracle.round_output(y_ref, dtype), dtype) - y_ref.astype(np.float64)
    return max_abs, rel, float(np.max(np.abs(floor))) if floor.size else 0.0


def assert_within_tolerance(y_bits, y_ref, dtype, label=""):
    max_abs, rel, floor = errors(y_bits, y_ref, dtype)
    print("%s max_abs=%.3g rel_l2=%.3g (rounding floor %.3g)" % (label, max_abs, rel, floor), flush=True)
    assert np.all(np.isfinite(half64(y_bits, dtype))), "non-finite output"
    assert max_abs <= MAX_ABS, (label, max_abs)
    assert rel <= REL_L2, (label, rel)
    return max_abs, rel
