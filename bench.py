"""Benchmark of one sparse MoE FFN layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one moe_layer_forward call (router, top-k, expert FFN over the
selected experts, combine) on one batch of synthetic inputs already resident
in HBM.  The default workload is single-token decode: hidden 4096, 64 experts,
top-4, intermediate 11008, 4-bit group-64 weights, fp16 activations; each
step takes the next token of a 256-token pool, so consecutive steps select
different experts.  Prints one JSON line.

Per-kernel durations come from HIP event pairs that the library attaches to
each kernel launch (hipExtLaunchKernelGGL: the events take the kernel's own
start and end timestamps), in a separate loop whose launches are queued
behind a spin kernel so the GPU runs them back to back.  The dominant kernel's
algorithmic bytes (or flops) per launch over its mean duration give the
roofline fraction.  The CPU baseline times the oracle (plain C, all host
cores) on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s; decode HBM TB/s % peak; prefill MFMA util %"
HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0

WORKLOADS = {
    "decode_b1": dict(recipe="decode_b1", pool=256, T=1,
                      label="decode b1: 1 token/step, H=4096, E=64, top-4, I=11008, 4-bit g64 weights, fp16"),
    "decode_q5": dict(recipe="decode_b1", pool=256, T=1, bits=5, I=2816,
                      label="decode b1: 1 token/step, H=4096, E=64, top-4, I=2816, 5-bit g64 weights, fp16"),
    "decode_q6": dict(recipe="decode_b1", pool=256, T=1, bits=6, I=2816,
                      label="decode b1: 1 token/step, H=4096, E=64, top-4, I=2816, 6-bit g64 weights, fp16"),
    "batched_decode": dict(recipe="batched_decode", pool=None, T=64,
                           label="batched decode: 64 tokens, H=4096, E=32, top-2, I=2816, 8-bit g64, bf16, Zipf 1.1"),
    "prefill": dict(recipe="prefill", pool=None, T=4096,
                    label="prefill: 4096 tokens, H=4096, E=64, top-4, I=1408, 4-bit g64, bf16, Zipf 1.2"),
    "decode_f4": dict(recipe="decode_b1", pool=256, T=1, fmt="nvfp4",
                      label="decode b1: 1 token/step, H=4096, E=64, top-4, I=11008, NVFP4 weights, fp16"),
    "prefill_f4": dict(recipe="prefill", pool=None, T=4096, fmt="nvfp4",
                       label="prefill: 4096 tokens, H=4096, E=64, top-4, I=1408, NVFP4 weights, bf16, Zipf 1.2"),
    "entropy_q4": dict(recipe="entropy", pool=None, T=512, bits=4,
                       label="entropy-adaptive: 512 tokens (segment k=3), H=4096, E=32, I=2816, 4-bit g64, fp16"),
    "entropy_all_q4": dict(recipe="entropy", pool=None, T=512, bits=4, segments=4,
                           label="entropy-adaptive: 4 segments x 512 tokens (k 1/2/3/3), H=4096, E=32, I=2816, "
                                 "4-bit g64, fp16"),
    "entropy_all_fp16": dict(recipe="entropy", pool=None, T=512, bits=16, segments=4,
                             label="entropy-adaptive: 4 segments x 512 tokens (k 1/2/3/3), H=4096, E=32, I=2816, "
                                   "fp16 weights"),
    "entropy_fp16": dict(recipe="entropy", pool=None, T=512, bits=16,
                         label="entropy-adaptive: 512 tokens (segment k=3), H=4096, E=32, I=2816, fp16 weights"),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def weight_bytes_per_row(K: int, bits) -> int:
    """Bytes of one weight row: codes plus scales (and biases); bits "nvfp4":
    K/2 code bytes and K/16 E4M3 block scales."""
    if bits == "nvfp4":
        return K // 2 + K // 16
    return K * bits // 8 + (0 if bits == 16 else 2 * 2 * (K // 64))


def capacity_keep(idx: np.ndarray, k_used: int, capacity: int) -> np.ndarray:
    """bool [T, kcap]: pairs within the first `capacity` of their expert in pair order."""
    T, kcap = idx.shape
    keep = np.zeros((T, kcap), bool)
    keep[:, :k_used] = True
    if capacity > 0:
        flat = idx.ravel()
        valid = keep.ravel()
        seen = {}
        for p in np.flatnonzero(valid):
            e = int(flat[p])
            seen[e] = seen.get(e, 0) + 1
            if seen[e] > capacity:
                valid[p] = False
        keep = valid.reshape(T, kcap)
    return keep


def algorithmic(name: str, kernel: str, *, T, H, E, I, bits, idx, k_used, kcap, keep=None):
    """Algorithmic HBM bytes and flops of one launch of `kernel`.

    Bytes: every touched expert's weight rows (codes plus fp16 scale/bias)
    read once, plus the activations read and the outputs written once.
    """
    if keep is not None and kernel != "gemv_gate_up_swiglu":  # the decode gate+up computes dropped pairs too
        sel = idx[keep]
    else:
        sel = idx[:, :k_used]
    touched = np.unique(sel)
    pairs = sel.size
    if kernel in ("gemv_gate_up_swiglu", "gemm_gate_up_swiglu"):
        # decode GEMV reads each selected (token, expert) row block; MFMA reads each touched expert once
        n_exp = pairs if kernel.startswith("gemv") else touched.size
        b = n_exp * 2 * I * weight_bytes_per_row(H, bits) + T * H * 2 + pairs * I * 2
        f = 2.0 * pairs * 2 * I * H
    elif kernel in ("gemv_down_combine",):
        b = pairs * H * weight_bytes_per_row(I, bits) + pairs * I * 2 + T * H * 2
        f = 2.0 * pairs * H * I
    elif kernel == "gemm_down":
        b = touched.size * H * weight_bytes_per_row(I, bits) + pairs * I * 2 + pairs * H * 2
        f = 2.0 * pairs * H * I
    elif kernel == "router_logits":
        b = E * H * 2 + T * H * 2 + T * E * 4
        f = 2.0 * T * E * H
    else:
        b, f = 0, 0.0
    return float(b), f


def layer_algorithmic(*, T, H, E, I, bits, idx, k_used, keep=None):
    """Algorithmic HBM bytes and flops of one whole layer call: every touched
    expert's gate_up and down weights (codes plus fp16 scale/bias) read once,
    the router weights, x and y; flops 2 P (3 I H) + 2 T E H over the P
    computed (token, slot) pairs."""
    sel = idx[keep] if keep is not None else idx[:, :k_used]
    touched = np.unique(sel).size
    pairs = sel.size
    b = touched * (2 * I * weight_bytes_per_row(H, bits) + H * weight_bytes_per_row(I, bits)) + E * H * 2 \
        + 2 * T * H * 2
    f = 2.0 * pairs * 3 * I * H + 2.0 * T * E * H
    return float(b), f


def traffic_from_profiles(kernel: str, workload: str):
    """HBM bytes per launch measured with rocprofv3 counters, if the summary in
    profiles/ was taken on the current kernel source (matching hash)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        data = json.load(open(path))
        ent = data.get(workload, {}).get(kernel)
        if not ent:
            return None
        from mixture_experts_router_amd import source_hash
        if ent.get("source_hash") != source_hash():
            return None
        return float(ent["bytes_per_launch"])
    except Exception:
        return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="decode_b1", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target wall time of the oracle sample")
    ap.add_argument("--no-graph", action="store_true", help="skip the hipGraph timed region (counter runs)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run a plain elementwise copy (torch.neg) of this many MiB, 5 launches: the known-size "
                         "kernel that calibrates rocprofv3's FETCH_SIZE / WRITE_SIZE")
    ap.add_argument("--load-aware", type=float, default=None, metavar="ALPHA",
                    help="route with the load-aware correction: logits - ALPHA * H, H a seeded load index "
                         "(activation counts of a Zipf-1.1 window, mean 1)")
    ap.add_argument("--groups", type=int, default=0, help="group-limited routing: at most one expert per group")
    ap.add_argument("--capacity", type=int, default=0, help="expert capacity: at most this many pairs per expert")
    ap.add_argument("--tune", action="append", default=[], metavar="KEY=VALUE",
                    help="launch-shape knob for measurement sweeps (moe_debug_set_tuning); results do not depend on it")
    ap.add_argument("--no-packed-q", action="store_true",
                    help="batched workloads: keep the row-major codes only (no packed_q repack)")
    ap.add_argument("--flush-mib", type=int, default=0,
                    help="also time the layer's kernels with a read of this many MiB of another buffer between "
                         "steps, which evicts the 256 MB Infinity Cache, so their weight bytes must come from HBM")
    ap.add_argument("--flush-write", action="store_true",
                    help="with --flush-mib: write the buffer instead of reading it (its dirty lines are then "
                         "written back while the next step's kernels read)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the layer is benchmarked on one device's share "
              "(multi-GPU sharding is a design note, not built); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import mixture_experts_router_amd as moe
    import moe_inputs as mi

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    moe.lib()  # fails loudly if the HIP library is missing
    for kv in args.tune:
        key, val = kv.split("=")
        moe.debug_set_tuning(int(key), int(val))
    wl = WORKLOADS[args.workload]
    recipe = wl["recipe"]
    mi.set_threads(min(os.cpu_count() or 1, 16))

    t0 = time.time()
    kw = {}
    for key in ("bits", "I", "fmt"):
        if key in wl:
            kw[key] = wl[key]
    if recipe == "entropy":
        kw["segment"] = 2
    T_pool = wl["pool"] or wl["T"]
    inp = mi.make_inputs(recipe, T=T_pool, **kw)
    log("generated %s inputs in %.1fs" % (args.workload, time.time() - t0))
    H, E, I, k = inp.H, inp.E, inp.I, inp.k
    bits = "nvfp4" if inp.fmt == "nvfp4" else inp.bits  # the byte counts' weight format
    dt = torch.float16 if inp.dtype == "f16" else torch.bfloat16

    def dev_bits(a, dtype):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(dtype).cuda()

    def dev_w(w):
        if w.bits == 16:
            return moe.Weights(dev_bits(w.q, torch.float16), None, None, w.E, w.N, w.K, 16)
        if w.fmt == "nvfp4":
            return moe.Weights(torch.from_numpy(w.q).cuda(), torch.from_numpy(w.scales).cuda(), None, w.E, w.N,
                               w.K, 4, 16, fmt="nvfp4", tensor_scale=w.tensor_scale)
        return moe.Weights(torch.from_numpy(w.q).cuda(), dev_bits(w.scales, torch.float16),
                           dev_bits(w.biases, torch.float16), w.E, w.N, w.K, w.bits)

    x_pool = dev_bits(inp.x, dt)
    wr = dev_bits(inp.wr, dt)
    # entropy segments: one layer call per segment (its own tokens and router
    # temperature, the same experts), a step being all of them
    nseg = wl.get("segments", 1)
    if nseg > 1:
        seg_np = [mi.make_router_inputs(recipe, segment=sg)[:2] for sg in range(nseg)]
        seg_dev = [(dev_bits(a, dt), dev_bits(b, dt)) for a, b in seg_np]
    else:
        seg_np = [(inp.x, inp.wr)]
        seg_dev = [(x_pool, wr)]
    gate, up = dev_w(inp.gate), dev_w(inp.up)
    gate_up = moe.fuse_gate_up(gate, up)  # the caller then frees the separate tensors
    del gate, up
    down = dev_w(inp.down)
    if wl["T"] > 1:
        # one-time repacks for the batched path (like the gate/up fusion, done
        # when the weights are loaded): scales and biases, and the codes in
        # 32-row blocks (a second copy of the codes)
        if bits != 16:
            gate_up, down = moe.pack_sb(gate_up), moe.pack_sb(down)
        if not args.no_packed_q:
            gate_up, down = moe.pack_q(gate_up), moe.pack_q(down)
    torch.cuda.synchronize()

    T = wl["T"]
    kcap = inp.kcap
    ws = torch.empty(moe.layer_workspace_size(T, H, E, k, I, 0), dtype=torch.uint8, device="cuda")
    y = torch.empty((T, H), dtype=dt, device="cuda")
    stream = torch.cuda.current_stream()

    def x_of(step):
        if wl["pool"]:
            i = step % wl["pool"]
            return x_pool[i:i + 1]
        return x_pool

    ropt = {}
    if args.load_aware is not None:
        ropt["health"] = torch.from_numpy(mi.load_index(5, E)).cuda()
        ropt["alpha"] = args.load_aware
    if args.groups:
        ropt["groups"] = args.groups
    lopt = dict(ropt, capacity=args.capacity) if args.capacity else ropt

    def step(i, evs=None):
        """One step; evs: the step's event pairs, handed to each call in turn
        (every library call starts again at the first pair it is given)."""
        if nseg > 1:
            for c_, (xs_, wrs_) in enumerate(seg_dev):
                if evs is not None:
                    moe.debug_set_events(evs[2 * nk * c_:2 * nk * (c_ + 1)])
                moe.layer_forward(xs_, wrs_, k, down, gate_up=gate_up, out=y, workspace=ws, **lopt)
        else:
            if evs is not None:
                moe.debug_set_events(evs)
            moe.layer_forward(x_of(i), wr, k, down, gate_up=gate_up, out=y, workspace=ws, **lopt)

    # discover the kernel plan (every segment's call launches the same kernels)
    plans = []
    for xs_, wrs_ in seg_dev[:nseg]:
        moe.layer_forward(xs_ if nseg > 1 else x_of(0), wrs_, k, down, gate_up=gate_up, out=y, workspace=ws, **lopt)
        torch.cuda.synchronize()
        plans.append(moe.last_plan())
    assert all(p_ == plans[0] for p_ in plans), plans
    plan = plans[0]
    nk = len(plan)
    nl = nk * nseg  # launches per step

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    K = args.steps

    # ---- timed region 1: stream launches, no instrumentation
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(args.warmup + i)
    torch.cuda.synchronize()
    eager_s = time.perf_counter() - t0

    # ---- timed region 2: hipGraph replays of consecutive layer calls,
    # exactly K steps in chunks: first a 2-step graph, then 64-step graphs and
    # a remainder.  A replay's kernels start only once its whole graph is
    # submitted (about 70 us for 20 steps), so the short first chunk lets the
    # GPU start while the longer ones are submitted behind it.
    graph_s = None
    sizes = [min(2, K)]
    while sum(sizes) < K:
        sizes.append(min(64, K - sum(sizes)))
    try:
        if args.no_graph:
            raise RuntimeError("skipped (--no-graph)")
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            for i in range(min(K, 66)):
                step(i)
        torch.cuda.current_stream().wait_stream(cap)
        torch.cuda.synchronize()
        # chunk j covers steps s_j .. s_j + n_j - 1 of the token pool; chunks
        # of the same size and pool offset share one graph
        graphs, plan_g, s0 = {}, [], 0
        for n in sizes:
            key = (n, s0 % 256)
            if key not in graphs:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    for i in range(n):
                        step(s0 + i)
                graphs[key] = g
            plan_g.append(graphs[key])
            s0 += n
        for g in graphs.values():
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for g in plan_g:
            g.replay()
        torch.cuda.synchronize()
        graph_s = time.perf_counter() - t0
    except Exception as ex:  # graph capture unavailable: report stream launches only
        log("graph capture failed:", ex)

    # ---- timed region 3: per-kernel durations.  The library launches each
    # kernel with hipExtLaunchKernelGGL and a start/stop HIP event pair, which
    # take the kernel's own start and end timestamps on the launch stream.
    # Each chunk of steps is queued behind a spin kernel, so the GPU runs the
    # chunk back to back as in the untimed loop.
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * nl)] for _ in range(K)]
    for evs in events:  # create the underlying HIP events
        for e in evs:
            e.record(stream)
    torch.cuda.synchronize()
    CH = 32
    t0 = time.perf_counter()
    for c0 in range(0, K, CH):
        torch.cuda._sleep(20_000_000)
        for i in range(c0, min(K, c0 + CH)):
            step(args.warmup + i, events[i])
    torch.cuda.synchronize()
    moe.debug_set_events(None)

    flush = None
    if args.flush_mib:
        # ---- timed region 4: the layer's kernels, each step preceded by a
        # read (a sum) or a write (a fill) of flush_mib MiB outside the events,
        # so no weight byte of the previous steps is left in the Infinity Cache
        buf = torch.ones(args.flush_mib << 18, dtype=torch.float32, device="cuda")
        nf = min(K, 64)
        fevents = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * nl)] for _ in range(nf)]
        for evs in fevents:
            for e in evs:
                e.record(stream)
        torch.cuda.synchronize()
        for i in range(nf):
            if args.flush_write:
                buf.fill_(float(i))
            else:
                buf.sum()
            step(args.warmup + i, fevents[i])
        torch.cuda.synchronize()
        moe.debug_set_events(None)
        fk = np.zeros(nk)
        for evs in fevents:
            for j in range(nl):
                fk[j % nk] += evs[2 * j].elapsed_time(evs[2 * j + 1])
        fk = fk / nf * 1e3
        flush = {"mib": args.flush_mib, "mode": "write" if args.flush_write else "read", "steps": nf,
                 "per_kernel_us": [round(float(v), 3) for v in fk],
                 "kernel_sum_us": round(float(fk.sum()), 3)}
        del buf

    if args.copy_probe_mib:
        n = args.copy_probe_mib << 19  # fp16 elements
        src = torch.empty(n, dtype=torch.float16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    best_s = min(v for v in (eager_s, graph_s) if v is not None)
    mode = "graph" if graph_s is not None and graph_s <= eager_s else "eager"
    elapsed = best_s
    ms_per_step = elapsed * 1e3 / K
    value = K * T * nseg / elapsed
    per_kernel = np.zeros(nk)  # summed over the step's calls
    per_call = np.zeros(nseg)
    for evs in events:
        for j in range(nl):
            d_ = evs[2 * j].elapsed_time(evs[2 * j + 1])
            per_kernel[j % nk] += d_
            per_call[j // nk] += d_
    per_kernel_us = per_kernel / K * 1e3
    per_call_us = per_call / K * 1e3
    gpu_step_us = float(sum(per_kernel_us))
    log("plan:", ", ".join("%s %.2fus" % (n, t) for n, t in zip(plan, per_kernel_us)))
    log("per step: eager %.2f us, graph %s us, sum of kernel durations %.2f us" % (
        eager_s * 1e6 / K, "%.2f" % (graph_s * 1e6 / K) if graph_s else "n/a", gpu_step_us))

    # ---- roofline of the dominant kernel
    j = int(np.argmax(per_kernel_us))
    kern = plan[j]
    # routing of a representative step (decode: over the pool; averaged bytes)
    routes = []
    for xs_, wrs_ in seg_dev:
        r = moe.route(xs_, wrs_, k, **ropt)
        torch.cuda.synchronize()
        routes.append((r["idx"].cpu().numpy(), int(r["k_used"].item())))
    idx_all, ku = routes[0]
    if wl["pool"]:
        bs, fs = [], []
        for s in range(min(wl["pool"], K)):
            b_, f_ = algorithmic(args.workload, kern, T=1, H=H, E=E, I=I, bits=bits, idx=idx_all[s:s + 1],
                                 k_used=ku, kcap=kcap,
                                 keep=capacity_keep(idx_all[s:s + 1], ku, args.capacity) if args.capacity else None)
            bs.append(b_)
            fs.append(f_)
        alg_b, alg_f = float(np.mean(bs)), float(np.mean(fs))
    else:
        alg_b, alg_f = 0.0, 0.0
        for idx_s, ku_s in routes:  # summed over the step's calls
            b_, f_ = algorithmic(args.workload, kern, T=T, H=H, E=E, I=I, bits=bits, idx=idx_s, k_used=ku_s,
                                 kcap=kcap, keep=capacity_keep(idx_s, ku_s, args.capacity) if args.capacity else None)
            alg_b += b_
            alg_f += f_
    dur_s = per_kernel_us[j] * 1e-6
    gbs = alg_b / dur_s / 1e9
    tflops = alg_f / dur_s / 1e12
    if gbs / HBM_PEAK_GBS >= tflops / MFMA_F16_PEAK_TFLOPS:
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tflops / MFMA_F16_PEAK_TFLOPS, 4)}
    roof["kernel"] = kern
    roof["mean_launch_us"] = round(float(per_kernel_us[j]), 3)
    roof["algorithmic_bytes"] = int(alg_b)
    roof["algorithmic_flops"] = int(alg_f)
    # counters are taken without routing options: with options the traffic is unmeasured
    # (per dispatch; a step of several calls launches the kernel once per call)
    tr_ = None if lopt else traffic_from_profiles(kern, args.workload)
    roof["traffic"] = tr_ * nseg if tr_ is not None else None

    # ---- the whole layer against its roofline: all algorithmic bytes (or
    # flops) of a step over the measured time per step
    if wl["pool"]:
        lb, lf = [], []
        for s_ in range(min(wl["pool"], K)):
            b_, f_ = layer_algorithmic(T=1, H=H, E=E, I=I, bits=bits, idx=idx_all[s_:s_ + 1], k_used=ku,
                                       keep=capacity_keep(idx_all[s_:s_ + 1], ku, args.capacity)
                                       if args.capacity else None)
            lb.append(b_)
            lf.append(f_)
        lay_b, lay_f = float(np.mean(lb)), float(np.mean(lf))
    else:
        lay_b, lay_f = 0.0, 0.0
        for idx_s, ku_s in routes:
            b_, f_ = layer_algorithmic(T=T, H=H, E=E, I=I, bits=bits, idx=idx_s, k_used=ku_s,
                                       keep=capacity_keep(idx_s, ku_s, args.capacity) if args.capacity else None)
            lay_b += b_
            lay_f += f_
    step_s = ms_per_step * 1e-3
    t_hbm = lay_b / (HBM_PEAK_GBS * 1e9)
    t_mfma = lay_f / (MFMA_F16_PEAK_TFLOPS * 1e12)
    if t_hbm >= t_mfma:
        roof["layer"] = {"bound": "hbm", "achieved": round(lay_b / step_s / 1e9, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(t_hbm / step_s, 4), "algorithmic_bytes": int(lay_b),
                         "algorithmic_flops": int(lay_f), "roofline_us": round(t_hbm * 1e6, 2)}
    else:
        roof["layer"] = {"bound": "mfma", "achieved": round(lay_f / step_s / 1e12, 2), "peak": MFMA_F16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(t_mfma / step_s, 4), "algorithmic_bytes": int(lay_b),
                         "algorithmic_flops": int(lay_f), "roofline_us": round(t_mfma * 1e6, 2)}

    # ---- the practical read ceiling: the library's streaming-read reference
    # (16-byte non-temporal loads, a contiguous segment per workgroup) over
    # as many bytes as a step's algorithmic bytes, timed with events over 10
    # launches
    nbytes = int(min(max(lay_b, 1 << 24), (1 << 32) - (1 << 20))) // 16 * 16
    sbuf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.empty(moe.STREAM_READ_WAVES, dtype=torch.int32, device="cuda")
    for _ in range(2):
        moe.debug_stream_read(sbuf, sink)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(10):
        moe.debug_stream_read(sbuf, sink)
    e1.record(stream)
    torch.cuda.synchronize()
    s_us = e0.elapsed_time(e1) * 1e3 / 10
    s_gbs = nbytes / (s_us * 1e-6) / 1e9
    roof["stream_read"] = {"bytes": nbytes, "us": round(s_us, 2), "achieved": round(s_gbs, 1), "unit": "GB/s",
                           "frac": round(s_gbs / HBM_PEAK_GBS, 4)}
    roof["layer"]["bytes_rate_vs_stream_read"] = round(lay_b / step_s / 1e9 / s_gbs, 4)
    del sbuf, sink

    # ---- CPU baseline: the oracle on a bounded sample of the same workload
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        gu_np = oracle.fuse_gate_up(inp.gate, inp.up)
        cores = oracle.num_threads()
        oopt = {}
        if "health" in ropt:
            oopt = dict(health=ropt["health"].cpu().numpy(), alpha=ropt["alpha"])
        if args.groups:
            oopt["groups"] = args.groups
        lo = dict(oopt, capacity=args.capacity) if args.capacity else oopt
        if wl["pool"]:
            def run(n):
                t = time.perf_counter()
                oracle.layer_forward(np.ascontiguousarray(inp.x[:n]), inp.wr, inp.dtype, k, gu_np, inp.down, **lo)
                return time.perf_counter() - t
            n0 = 4
            t_probe = run(n0)
            n = int(max(n0, min(wl["pool"], args.cpu_seconds / max(t_probe / n0, 1e-6))))
            t_run = run(n)
            cpu = {"value": round(n / t_run, 3), "unit": "tokens/s", "cores": cores, "kind": "oracle",
                   "sample": "%d single tokens of the decode pool (each: route + 4 experts), %.1fs" % (n, t_run)}
            oracle.set_threads(1)
            n1 = max(2, n // max(cores, 1))
            t1 = run(n1)
            oracle.set_threads(cores)
            cpu["value_1core"] = round(n1 / t1, 3)
            cpu["sample_1core"] = "%d single tokens of the decode pool on 1 thread, %.1fs" % (n1, t1)
        else:
            # per call (segment): routing of all T tokens plus T token FFNs at
            # the cost of a random sample of them; the step is the sum
            rng = np.random.default_rng(0)

            def sample(n_tok):
                t_route_, t_tok_, total_ = 0.0, 0.0, 0.0
                for xn, wrn in seg_np:
                    t = time.perf_counter()
                    idx_o, w_o, ku_o, _ = oracle.route(xn, wrn, inp.dtype, k, **oopt)
                    tr = time.perf_counter() - t
                    toks = np.sort(rng.choice(T, n_tok, replace=False))
                    t = time.perf_counter()
                    oracle.tokens_forward(xn, inp.dtype, toks, idx_o, w_o, ku_o, gu_np, inp.down)
                    tt = time.perf_counter() - t
                    t_route_ += tr
                    t_tok_ += tt
                    total_ += tr + tt / n_tok * T
                return t_route_, t_tok_, total_

            x0, wr0 = seg_np[-1]  # the last call: the largest k of the entropy segments
            idx_o, w_o, ku_o, _ = oracle.route(x0, wr0, inp.dtype, k, **oopt)
            t = time.perf_counter()
            oracle.tokens_forward(x0, inp.dtype, [0], idx_o, w_o, ku_o, gu_np, inp.down)
            per_tok = time.perf_counter() - t
            n = int(max(2, min(T, args.cpu_seconds / nseg / max(per_tok, 1e-6))))
            t_route, t_tok, total = sample(n)
            what = "routing of all %d tokens (%.1fs) + expert FFN of %d sampled tokens (%.1fs)" % (T, t_route, n,
                                                                                                  t_tok)
            if nseg > 1:
                what = "per segment (%d segments): %d tokens routed, %d sampled; totals: routing %.1fs, FFN %.1fs" % (
                    nseg, T, n, t_route, t_tok)
            cpu = {"value": round(T * nseg / total, 3), "unit": "tokens/s", "cores": cores, "kind": "oracle",
                   "sample": what + ", scaled to the batch"}
            oracle.set_threads(1)
            n1 = max(2, n // max(cores, 1))
            t_route1, t_tok1, total1 = sample(n1)
            oracle.set_threads(cores)
            cpu["value_1core"] = round(T * nseg / total1, 3)
            cpu["sample_1core"] = "1 thread: routing %.1fs + expert FFN of %d sampled tokens per call (%.1fs), " \
                                  "scaled to the batch" % (t_route1, n1, t_tok1)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": wl["label"], "tokens_per_step": T * nseg, "hidden": H, "experts": E, "top_k": k,
                   "intermediate": I, "weight_bits": bits, "activations": inp.dtype,
                   "arithmetic": "fp16 operands (dequantised weights, activations, SwiGLU rows), fp32 accumulation",
                   "launch": mode, "eager_tokens_per_s": round(K * T * nseg / eager_s, 2),
                   "graph_tokens_per_s": round(K * T * nseg / graph_s, 2) if graph_s else None,
                   "kernels_per_step": nk, "plan": plan,
                   "routing_options": {"load_aware_alpha": args.load_aware, "groups": args.groups,
                                       "capacity": args.capacity} if lopt else None,
                   "per_kernel_us": [round(float(v), 3) for v in per_kernel_us],
                   "segments": [{"segment": sg, "tokens": T, "k_used": routes[sg][1],
                                 "kernel_sum_us": round(float(per_call_us[sg]), 3)} for sg in range(nseg)]
                   if nseg > 1 else None,
                   "tuning": args.tune or None,
                   "cache_flush": flush,
                   "packed_q": bool(wl["T"] > 1 and not args.no_packed_q)},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
