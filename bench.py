"""MoE-layer forward throughput on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload dsv2_lite] [--tokens 64]
                    [--mode lore] [--quick]

One step = one moe_layer_forward over one batch of synthetic tokens (router,
softmax/top-k, residency split, permutation, expert + shared FFNs, LoRE
surrogate fused into the combine), eager launches on torch's current stream,
inputs and weights resident in HBM.  The headline workload is the largest
layer: the Qwen2-57B-A14B-shaped decode layer (H=3584, 64 experts top-8,
I=2560, one shared expert of 20480 channels with a sigmoid gate,
renormalised weights) at 256 tokens, every routed expert computed exactly.
Steps cycle through enough copies of the layer's weights that the 256 MB
Infinity Cache cannot serve one step's weights to the next.

Prints ONE JSON line.  `roofline` is for the dominant kernel (the expert
gate/up projection): algorithmic bytes (or flops) per launch divided by its
average duration, timed live with HIP events recorded around that kernel on
the launch stream.  `cpu_baseline` times the CPU oracle on a bounded sample of
the same workload.  `also` lists the other token counts and workloads.
"""
from __future__ import annotations

import argparse
import ctypes
import dataclasses
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFS = 2500.0    # MI355X dense bf16 MFMA, TFLOP/s
METRIC = "MoE-layer tokens/s at 1 GPU; % HBM BW peak (decode) / % MFMA peak (prefill)"
PROF_EVERY = 8                 # timed steps between kernel-event samples


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="qwen2_57b")
    ap.add_argument("--tokens", type=int, default=256)
    ap.add_argument("--mode", default="standard")
    ap.add_argument("--quick", action="store_true", help="headline only (no other workloads)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain device-to-device copy of COPY_BYTES (counter calibration)")
    return ap.parse_args()


COPY_BYTES = 256 << 20         # copy-probe size: 256 MiB read + 256 MiB written per launch

# HBM bytes per launch of the dominant kernel, from rocprofv3 FETCH_SIZE and
# WRITE_SIZE passes scaled by the copy probe's counters.  Each record names the
# sources the counted kernel was built from; a digest mismatch means the kernel
# changed since the counters were taken and the figure no longer applies.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_expert_gate_up_dsv2_lite_T64_lore.md")
TRAFFIC_FILES = {
    ("dsv2_lite", 64, "lore"): TRAFFIC_FILE,
    ("qwen2_57b", 256, "standard"): os.path.join(
        ROOT, "profiles", "traffic_expert_gate_up_qwen2_57b_T256.md"),
    ("granite_prefill", 4096, "standard"): os.path.join(
        ROOT, "profiles", "traffic_expert_gate_up_granite_prefill_T4096.md"),
}


def kernel_digest(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(path=TRAFFIC_FILE):
    """(bytes per launch, sources, digest) from a traffic record, or None."""
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for ln in fh:
            if ln.startswith("- ") and ": " in ln:
                key, val = ln[2:].split(": ", 1)
                fields[key.strip()] = val.strip().strip("`")
    try:
        return (float(fields["hbm_bytes_per_launch"]), fields["sources"].split(), fields["source_digest"])
    except KeyError:
        return None


def copy_probe():
    import torch
    n = COPY_BYTES // 2
    a = torch.randn(n, device="cuda").to(torch.bfloat16)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(4):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": COPY_BYTES, "copy_probe_bytes_written": COPY_BYTES,
                      "launches": 4}))


class HipEvents:
    """hipEvent_t pairs from the HIP runtime torch already loaded."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so.7")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        ev = ctypes.c_void_p()
        assert self.lib.hipEventCreate(ctypes.byref(ev)) == 0
        return ev.value

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        assert self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value

    def destroy(self, ev):
        self.lib.hipEventDestroy(ev)


# ------------------------------------------------------ algorithmic bytes --
def step_traffic(cfg, T, mode, ids, exact, keep_count=None, shared_apart=False):
    """Algorithmic bytes and flops of one layer forward, from the routing the
    GPU actually took: each touched weight byte once, activations once.
    `up` is the gate/up launch: routed experts, plus the shared experts
    unless they run in launches of their own (shared_apart)."""
    H, I, E, k = cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k
    eb = 4 if cfg.dtype == "f32" else 2
    exact_experts = {int(e) for e, x in zip(ids.reshape(-1), exact.reshape(-1)) if x}
    miss_experts = {int(e) for e, x in zip(ids.reshape(-1), exact.reshape(-1)) if not x}
    P = int(exact.sum())
    b = H * E * eb + 2 * T * H * eb                    # router, x in, out
    f = 2 * T * H * E
    up = {}
    if mode == "floe":
        nk = cfg.floe_keep
        per_pair_rows = nk
        for e in exact_experts:
            b += I * H // 4 + 2 * I * (H // 64) * 2     # INT2 codes + fp16 scale/zero
        b += P * 2 * per_pair_rows * H * eb            # kept gate and down rows
        f += P * (2 * I * H + 2 * 2 * nk * H)
        up = dict(bytes=len(exact_experts) * (I * H // 4 + 2 * I * (H // 64) * 2) + P * H * eb,
                  flops=P * 2 * I * H)
    else:
        b += len(exact_experts) * 3 * I * H * eb
        f += P * 2 * 3 * I * H
        sh = cfg.n_shared * cfg.shared_inter
        b += 3 * sh * H * eb + (H * eb if cfg.shared_gate else 0)
        f += T * 2 * 3 * sh * H
        b += len(miss_experts) * 2 * cfg.lore_rank * H * eb
        f += int((1 - exact).sum()) * 2 * 2 * cfg.lore_rank * H
        act_b = eb                                     # activations in the layer's dtype
        n_miss = int((1 - exact).sum())
        r = cfg.lore_rank
        sh_up = 0 if shared_apart else sh
        up = dict(bytes=(len(exact_experts) * 2 * I * H + 2 * sh_up * H + len(miss_experts) * r * H) * eb
                  + T * H * eb + (P * I + T * sh_up + n_miss * r) * act_b,
                  flops=P * 2 * 2 * I * H + T * 2 * 2 * sh_up * H + n_miss * 2 * r * H)
    return dict(bytes=b, flops=f, up=up, distinct_experts=len(exact_experts),
                lore_experts=len(miss_experts), pairs=P)


# ------------------------------------------------------------- measurement --
def measure(name, T, mode, steps, warmup, ev=None, want_roofline=False, layer=None):
    import numpy as np
    import torch

    import workloads as W
    from workloads.device import dims_dict, mask_tensor, tensor, upload
    import sparse_moe_layer_route_amd as M

    layer = layer if layer is not None else W.make_layer(name)
    cfg = layer.cfg
    w0 = upload(layer, "cuda")
    dd = M.Dims(**dims_dict(cfg))
    if cfg.dtype == "bf16" and cfg.up_format == "dense":
        # expert matrices packed fragment-major once, as a deployment would
        dd = dataclasses.replace(dd, weight_layout="mfma16")
        w0 = M.pack_weights(dd, w0)
    dims = dd.c()
    x = tensor(layer.x(T), cfg.dtype, "cuda")
    stride = 0
    res = None
    if mode == "lore":
        res = mask_tensor([layer.resident()], "cuda")
    elif mode == "stall_free":
        d = torch.from_numpy(layer.delta(T).astype(np.int32)).cuda()
        res = torch.empty(T, dtype=torch.int64, device="cuda")
        fl = torch.empty(T, dtype=torch.int32, device="cuda")
        M.moe_prefetch_mask(dims, T, x, w0["w_prefetch"], d, res, fl)
        stride = 1
    ws = torch.empty(M.moe_workspace_size(dims, T, mode), dtype=torch.uint8, device="cuda")
    odt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    out = torch.empty(T, cfg.hidden, dtype=odt, device="cuda")
    k = cfg.top_k
    ids = torch.empty(T * k, dtype=torch.int32, device="cuda")
    exact = torch.empty(T * k, dtype=torch.uint8, device="cuda")
    M.moe_layer_forward(dims, T, x, w0, res, stride, mode, out, ws,
                        debug={"topk_ids": ids, "exact": exact})
    torch.cuda.synchronize()
    # do the shared experts run in launches of their own (a non-empty bracket)?
    shared_apart = False
    if ev is not None and cfg.n_shared > 0:
        a, b = ev.create(), ev.create()
        dbg = M.MoeDebug()
        dbg.prof_start, dbg.prof_stop, dbg.prof_kernel = a, b, M.binding.KERNELS["shared_ffn"]
        M.moe_layer_forward(dims, T, x, w0, res, stride, mode, out, ws, debug=dbg)
        torch.cuda.synchronize()
        shared_apart = ev.elapsed_ms(a, b) > 0.02   # an empty bracket reads ~0
        ev.destroy(a)
        ev.destroy(b)
    tr = step_traffic(cfg, T, mode, ids.cpu().numpy(), exact.cpu().numpy(),
                      shared_apart=shared_apart)
    # weight copies so consecutive steps stream different bytes
    n_copies = max(1, min(16, math.ceil(1.0e9 / max(tr["bytes"], 1))))
    copies = [w0] + [{n: t.clone() for n, t in w0.items()} for _ in range(n_copies - 1)]
    wstructs = [M.weights_struct(c) for c in copies]
    dom = "floe_up" if mode == "floe" else "expert_gate_up"
    # events around the dominant kernel on every PROF_EVERY-th timed step:
    # each record is a timestamp packet that would otherwise add a few
    # microseconds to every step
    evs = []
    dbgs = {}
    if ev is not None:
        for i in range(0, steps, PROF_EVERY):
            a, b = ev.create(), ev.create()
            evs.append((a, b))
            dbg = M.MoeDebug()
            dbg.prof_start, dbg.prof_stop, dbg.prof_kernel = a, b, M.binding.KERNELS[dom]
            dbgs[i] = dbg

    def step(i, dbg=None):
        M.moe_layer_forward(dims, T, x, wstructs[i % n_copies], res, stride, mode, out, ws,
                            debug=dbg)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_stop = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t_start.record()
    for i in range(steps):
        step(i, dbgs.get(i))
    t_stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = t_start.elapsed_time(t_stop) / steps
    # eager step-time distribution: a second pass with events around every step
    se = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for i in range(steps):
        se[i][0].record()
        step(i)
        se[i][1].record()
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) * 1e3 for a, b in se)
    pick = lambda q: per[min(len(per) - 1, int(q * (len(per) - 1) + 0.5))]
    # HIP graph replay: one graph holding one step per weight copy, replayed
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for i in range(n_copies):
            step(i)
    reps = max(1, steps // n_copies)
    g.replay()
    torch.cuda.synchronize()
    t_start.record()
    for _ in range(reps):
        g.replay()
    t_stop.record()
    torch.cuda.synchronize()
    g_ms = t_start.elapsed_time(t_stop) / (reps * n_copies)
    del g
    r = dict(workload=name, tokens=T, mode=mode, ms_per_step=ms, tokens_per_s=T / (ms * 1e-3),
             step_us=dict(p10=pick(0.1), p50=pick(0.5), p90=pick(0.9)),
             graph=dict(ms_per_step=g_ms, tokens_per_s=T / (g_ms * 1e-3)),
             wall_ms_per_step=wall * 1e3 / steps, weight_copies=n_copies,
             step_bytes=tr["bytes"], step_flops=tr["flops"],
             step_gbs=tr["bytes"] / (ms * 1e-3) / 1e9,
             distinct_experts=tr["distinct_experts"], lore_experts=tr["lore_experts"], pairs=tr["pairs"])
    r["step_hbm_frac"] = r["step_gbs"] / HBM_PEAK_GBS
    r["step_mfma_frac"] = tr["flops"] / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS
    if evs:
        kms = [ev.elapsed_ms(a, b) for a, b in evs]
        avg_us = 1e3 * sum(kms) / len(kms)
        up = tr["up"]
        prefill = T >= 1024
        if prefill:
            achieved = up["flops"] / (avg_us * 1e-6) / 1e12
            roof = dict(bound="mfma", achieved=achieved, peak=MFMA_BF16_PEAK_TFS, unit="TFLOP/s",
                        frac=achieved / MFMA_BF16_PEAK_TFS)
        else:
            achieved = up["bytes"] / (avg_us * 1e-6) / 1e9
            roof = dict(bound="hbm", achieved=achieved, peak=HBM_PEAK_GBS, unit="GB/s",
                        frac=achieved / HBM_PEAK_GBS)
        traffic = None
        tf = TRAFFIC_FILES.get((name, T, mode))
        rec = recorded_traffic(tf) if tf else None
        if rec is not None and kernel_digest(rec[1]) == rec[2]:
            traffic = rec[0]
        roof.update(traffic=traffic, kernel=dom + (" (routed)" if shared_apart else ""),
                    avg_us=avg_us, bytes_per_launch=up["bytes"],
                    flops_per_launch=up["flops"], launches_timed=len(kms))
        r["roofline"] = roof
        for a, b in evs:
            ev.destroy(a)
            ev.destroy(b)
    del copies, wstructs, w0
    torch.cuda.empty_cache()
    return r


def cpu_baseline(name, T, mode, budget_s=8.0, layer=None):
    """The CPU oracle as it stands, timed on the host cores on a bounded
    sample of the same workload: the fp32 variant (the same steps on float32
    copies, BLAS matmuls) with every host thread and with one thread, and the
    fp64 parity oracle for information.  Each leg takes the first S tokens (S
    doubled from 1 until one call takes about budget_s/2 or covers all T
    tokens) and repeats that call until about budget_s has been timed."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    import oracle as O
    import workloads as W
    from workloads.device import dims_dict

    layer = layer if layer is not None else W.make_layer(name)
    cfg = layer.cfg
    d = dims_dict(cfg)
    res = layer.resident() if mode == "lore" else None
    if mode == "stall_free":
        masks, _, _ = O.prefetch_masks(O.decode(layer.x(T), cfg.dtype),
                                       O.decode(layer.w_prefetch(), cfg.dtype), layer.delta(T), cfg.top_k)
        res = masks

    def call(S, precision):
        sub_res = res[:S] if isinstance(res, list) else res
        t0 = time.perf_counter()
        O.layer_forward(layer.x(T)[:S], layer, d, mode, resident=sub_res, precision=precision)
        return time.perf_counter() - t0

    def leg(precision, threads, budget):
        with threadpool_limits(limits=threads):
            call(1, precision)       # untimed: first-call set-up (weight draws cached)
            S = 1
            while True:
                dt = call(S, precision)
                if dt >= budget / 2 or S >= T:
                    break
                S = min(T, S * 2)
            total, calls = dt, 1
            while total < budget:
                total += call(S, precision)
                calls += 1
            used = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        return dict(value=S * calls / total, unit="tokens/s", cores=int(used), tokens=S,
                    calls=calls, seconds=total)

    host = len(os.sched_getaffinity(0))
    f32_all = leg("f32", host, budget_s)
    f32_one = leg("f32", 1, budget_s)
    f64_all = leg("f64", host, budget_s / 2)
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")),
                         model)
    except OSError:
        pass
    # the baseline is the faster fp32 leg: on a shared host the all-thread BLAS
    # leg can fall far below the one-thread leg (threads waiting on each other)
    best = f32_all if f32_all["value"] >= f32_one["value"] else f32_one
    return dict(value=best["value"], unit="tokens/s", cores=best["cores"], kind="oracle",
                sample=f"first {best['tokens']} of the {T} tokens of the same {name} layer in mode "
                       f"{mode}, {best['calls']} fp32 NumPy oracle call(s) with BLAS on "
                       f"{best['cores']} thread(s), {best['seconds']:.1f} s in total (the faster "
                       f"of the all-thread and one-thread legs)",
                all_threads=f32_all, one_thread=f32_one, fp64_parity_oracle=f64_all,
                cpu_model=model, host_cpus=host)


def measure_library_gemm(ev, name="granite_prefill", T=4096, reps=30):
    """Context for the grouped GEMM: its gate/up and down launches at the
    prefill layer beside the vendor GEMM (torch.matmul / torch.bmm, bf16) on
    the same flops without the token gather: one dense product over all
    (token, slot) pairs, and a batched product with every expert given an
    equal segment.  Timed with events; inputs are random bf16 tensors."""
    import torch

    import workloads as W
    from workloads.device import dims_dict, tensor, upload
    import sparse_moe_layer_route_amd as M

    layer = W.make_layer(name)
    cfg = layer.cfg
    w0 = upload(layer, "cuda")
    dd = dataclasses.replace(M.Dims(**dims_dict(cfg)), weight_layout="mfma16")
    w0 = M.pack_weights(dd, w0)
    dims = dd.c()
    x = tensor(layer.x(T), cfg.dtype, "cuda")
    ws = torch.empty(M.moe_workspace_size(dims, T, "standard"), dtype=torch.uint8, device="cuda")
    out = torch.empty(T, cfg.hidden, dtype=torch.bfloat16, device="cuda")
    ours = {}
    for kern in ("expert_gate_up", "expert_down"):
        times = []
        for i in range(reps + 3):
            a, b = ev.create(), ev.create()
            dbg = M.MoeDebug()
            dbg.prof_start, dbg.prof_stop, dbg.prof_kernel = a, b, M.binding.KERNELS[kern]
            M.moe_layer_forward(dims, T, x, w0, None, 0, "standard", out, ws, debug=dbg)
            torch.cuda.synchronize()
            if i >= 3:
                times.append(ev.elapsed_ms(a, b) * 1e3)
            ev.destroy(a)
            ev.destroy(b)
        ours[kern] = sorted(times)[len(times) // 2]
    del w0, ws
    P, H, I, E = T * cfg.top_k, cfg.hidden, cfg.inter, cfg.n_experts
    seg = P // E

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / reps

    g = torch.Generator(device="cuda").manual_seed(0)
    rnd = lambda *shape: torch.randn(*shape, device="cuda", generator=g).to(torch.bfloat16)
    res = {}
    for part, K, N in (("gate_up", H, 2 * I), ("down", I, H)):
        flops = 2.0 * P * K * N
        a2, b2 = rnd(P, K), rnd(K, N)
        dense = timed(lambda: torch.matmul(a2, b2))
        del a2, b2
        a3, b3 = rnd(E, seg, K), rnd(E, K, N)   # both contiguous
        batched = timed(lambda: torch.bmm(a3, b3))
        del a3, b3
        mine = ours["expert_gate_up" if part == "gate_up" else "expert_down"]
        res[part] = dict(ours_us=mine, ours_tflops=flops / (mine * 1e-6) / 1e12,
                         dense_us=dense, dense_tflops=flops / (dense * 1e-6) / 1e12,
                         batched_us=batched, batched_tflops=2.0 * E * seg * K * N / (batched * 1e-6) / 1e12)
    torch.cuda.empty_cache()
    return dict(kind="library_gemm_context", workload=name, tokens=T, pairs=P,
                dense=f"[{P} x K] @ [K x N]", batched=f"{E} x [{seg} x K] @ [K x N]", **res)


def measure_prefetch_adaptive(name, T, steps, warmup, tau=0.9):
    """The APEX adaptive prefetch call (budget, list, delta* and overlap) on
    its own: time per call, its HBM rate against the bytes it must move
    (x, W_p, w_delta, theta, the router's ids in; budget, mask, flags,
    delta*, overlap out), and the budget and overlap it reaches."""
    import numpy as np
    import torch

    import workloads as W
    from workloads.device import dims_dict, tensor
    import sparse_moe_layer_route_amd as M

    layer = W.make_layer(name)
    cfg = layer.cfg
    k, E, H = cfg.top_k, cfg.n_experts, cfg.hidden
    dims = M.Dims(**dims_dict(cfg)).c()
    x = tensor(layer.x(T), cfg.dtype, "cuda")
    wp = tensor(layer.w_prefetch(), cfg.dtype, "cuda")
    w_delta, theta = layer.ordinal(tau)
    wd = tensor(w_delta, cfg.dtype, "cuda")
    th = torch.from_numpy(np.ascontiguousarray(theta, np.float32)).cuda()
    # the router's choices from the layer's own router (moe_route)
    wr = tensor(layer.w_router(), cfg.dtype, "cuda")
    ids = torch.empty(T * k, dtype=torch.int32, device="cuda")
    tw = torch.empty(T * k, dtype=torch.float32, device="cuda")
    ex = torch.empty(T * k, dtype=torch.uint8, device="cuda")
    fl = torch.empty(T, dtype=torch.int32, device="cuda")
    lg = torch.empty(T * E, dtype=torch.float32, device="cuda")
    M.moe_route(dims, T, x, wr, None, 0, "standard", ids, tw, ex, fl, lg)
    delta = torch.empty(T, dtype=torch.int32, device="cuda")
    mask = torch.empty(T, dtype=torch.int64, device="cuda")
    ds = torch.empty(T, dtype=torch.int32, device="cuda")
    ov = torch.empty(T, dtype=torch.int32, device="cuda")

    def call():
        M.moe_prefetch_adaptive(dims, T, x, wp, wd, th, tau, delta, mask, fl, topk_ids=ids,
                                delta_star=ds, overlap=ov)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        call()
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / steps
    esz = 4 if cfg.dtype == "f32" else 2
    nbytes = (T * H + E * H + H) * esz + (E - k + 1) * 4 + T * k * 4 + T * (4 + 8 + 4 + 4 + 4)
    d, o, st = delta.cpu().numpy(), ov.cpu().numpy(), ds.cpu().numpy()
    return dict(workload=name, tokens=T, mode="prefetch_adaptive", us_per_call=us,
                gbs=nbytes / (us * 1e-6) / 1e9, hbm_frac=nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                bytes=nbytes, tau=tau, mean_budget=float(d.mean()),
                overlap=float(o.mean() / k), covered=float((d >= st).mean()))


def measure_floe_predict(steps, warmup, T=1, T_recall=8):
    """FloE intra-expert predictor (previous hidden state through the INT2 up,
    channel selection) and compact gate/down packing for Mixtral-8x7B-shaped
    experts: time per call, HBM rate against the bytes each must move, and
    the recall of the predicted masks against the true ones."""
    import numpy as np
    import torch

    import workloads as W
    from workloads.device import dims_dict, tensor, upload
    import sparse_moe_layer_route_amd as M

    cfg = dataclasses.replace(W.CONFIGS["mixtral_floe"], token_counts=(1, T_recall))
    layer = W.Layer(cfg)
    dims = M.Dims(**dims_dict(cfg))
    k, nk, H, I, E = cfg.top_k, cfg.floe_keep, cfg.hidden, cfg.inter, cfg.n_experts
    w = upload(layer, "cuda")
    Tm = max(T, T_recall)
    ws = torch.empty(M.moe_workspace_size(dims, Tm, "floe"), dtype=torch.uint8, device="cuda")
    # this layer's experts: the router on x (moe_route)
    ids = torch.empty(Tm * k, dtype=torch.int32, device="cuda")
    tw = torch.empty(Tm * k, dtype=torch.float32, device="cuda")
    ex = torch.empty(Tm * k, dtype=torch.uint8, device="cuda")
    fl = torch.zeros(Tm, dtype=torch.int32, device="cuda")
    lg = torch.empty(Tm * E, dtype=torch.float32, device="cuda")
    x = tensor(layer.x(Tm), cfg.dtype, "cuda")
    xp = tensor(layer.x_prev(Tm), cfg.dtype, "cuda")
    M.moe_route(dims, Tm, x, w["w_router"], None, 0, "standard", ids, tw, ex, fl, lg)
    keep_p = torch.empty(Tm * k * nk, dtype=torch.int32, device="cuda")
    keep_t = torch.empty(Tm * k * nk, dtype=torch.int32, device="cuda")
    M.moe_floe_predict(dims, Tm, xp, w, ids, keep_p, fl, ws)
    M.moe_floe_predict(dims, Tm, x, w, ids, keep_t, fl, ws)
    torch.cuda.synchronize()
    kp = keep_p.cpu().numpy().reshape(-1, nk)
    kt = keep_t.cpu().numpy().reshape(-1, nk)
    recall = float(np.mean([len(set(a) & set(b)) / nk for a, b in zip(kp, kt)]))
    esz = 2 if cfg.dtype == "bf16" else 4
    gate = torch.empty(T * k * nk * H * esz // 2, dtype=torch.int16, device="cuda")
    down = torch.empty_like(gate)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ev[0].record()
        for _ in range(steps):
            fn()
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) * 1e3 / steps

    us_pred = timed(lambda: M.moe_floe_predict(dims, T, xp, w, ids, keep_p, fl, ws))
    us_pack = timed(lambda: M.moe_floe_pack(dims, T, ids, keep_p, w["w_gate"], w["w_down"], gate, down))
    # bytes: INT2 codes + fp16 scale and zero of each pair's expert, and h;
    # packing reads and writes the kept gate and down rows
    pred_bytes = T * k * (I * H // 4 + 2 * I * (H // 64) * 2) + T * H * esz
    pack_bytes = T * k * nk * H * esz * 2 * 2
    return dict(workload="mixtral_floe", tokens=T, mode="floe_predict_pack",
                predict_us=us_pred, predict_gbs=pred_bytes / (us_pred * 1e-6) / 1e9,
                pack_us=us_pack, pack_gbs=pack_bytes / (us_pack * 1e-6) / 1e9,
                pack_hbm_frac=pack_bytes / (us_pack * 1e-6) / 1e9 / HBM_PEAK_GBS,
                recall=recall, recall_tokens=T_recall, prev_noise=cfg.prev_noise)


def measure_lore_fit(name="dsv2_lite", expert=0, ranks=(8, 16, 32), cols=64, n_iter=20):
    """LoRE fitting for one expert of the named layer: targets y_e - y_s on an
    orthogonal calibration design of H rows, then the rank-r fit for each r;
    time per step and the relative calibration error per rank."""
    import numpy as np
    import torch

    import workloads as W
    from workloads.device import dims_dict, tensor, upload
    import sparse_moe_layer_route_amd as M

    layer = W.make_layer(name)
    cfg = layer.cfg
    H, N = cfg.hidden, cfg.hidden
    dims = M.Dims(**dims_dict(cfg))
    w = upload(layer, "cuda")
    h = tensor(layer.calibration(N), cfg.dtype, "cuda")
    d1 = dataclasses.replace(dims, top_k=1)
    ws = torch.empty(M.moe_workspace_size(d1, N, "standard"), dtype=torch.uint8, device="cuda")
    R = torch.empty(N * H, dtype=torch.float32, device="cuda")
    om = torch.from_numpy(np.ascontiguousarray(layer.omega(cols))).cuda()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    M.moe_lore_targets(dims, N, h, w, expert, R, ws)   # warm-up
    torch.cuda.synchronize()
    ev[0].record()
    M.moe_lore_targets(dims, N, h, w, expert, R, ws)
    ev[1].record()
    torch.cuda.synchronize()
    out = dict(workload=name, tokens=N, mode="lore_fit", expert=expert, cols=cols, n_iter=n_iter,
               targets_ms=ev[0].elapsed_time(ev[1]), fits=[])
    tdt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    for r in ranks:
        A = torch.empty(r * H, dtype=tdt, device="cuda")
        B = torch.empty(H * r, dtype=tdt, device="cuda")
        sig = torch.empty(r, dtype=torch.float32, device="cuda")
        err = torch.empty(4, dtype=torch.float32, device="cuda")
        fws = torch.empty(M.moe_lore_fit_size(H, N, r, cols), dtype=torch.uint8, device="cuda")
        M.moe_lore_fit(dims, N, h, R, r, cols, n_iter, om, A, B, sig, err, fws)
        torch.cuda.synchronize()
        ev[0].record()
        M.moe_lore_fit(dims, N, h, R, r, cols, n_iter, om, A, B, sig, err, fws)
        ev[1].record()
        torch.cuda.synchronize()
        out["fits"].append(dict(rank=r, ms=ev[0].elapsed_time(ev[1]), rel_error=float(err[0]),
                                sigma_max=float(sig[0]), sigma_r=float(sig[r - 1])))
    return out


def measure_offload(ev, name="dsv2_lite", tokens=(1, 8), steps=20):
    """Exact execution of missed experts (moe_layer_forward_offload) with the
    layer's resident mask: the cost table is calibrated here (host -> GPU
    copy rate of one expert, the host FFN on one expert with one and four
    pairs, the GPU forward per active expert), then each batch runs under
    four plans: fetch every missed expert, run every one on the host, the
    cost rule, and the cost rule with the link and the host as queues.  Wall time per call (through a final synchronisation),
    with the LoRE-mode forward (misses -> surrogate, no transfers) and the
    all-resident STANDARD forward of the same batch as context."""
    import numpy as np
    import torch

    import workloads as W
    from workloads.device import dims_dict, mask_tensor, tensor, upload
    import sparse_moe_layer_route_amd as M

    layer = W.make_layer(name)
    cfg = layer.cfg
    dims = M.Dims(**dims_dict(cfg))
    threads = min(16, os.cpu_count() or 1)
    wdev = upload(layer, "cuda")
    names = ("w_gate", "w_up", "w_down")

    def pinned(a):
        a = np.ascontiguousarray(a)
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if cfg.dtype == "bf16" \
            else torch.from_numpy(a)
        return t.pin_memory()

    host = {n: pinned(layer.full(n)) for n in names}
    res = layer.resident()
    elem = 2 if cfg.dtype == "bf16" else 4
    w_bytes = 3 * cfg.inter * cfg.hidden * elem

    # calibration: link rate, host FFN per expert and per pair, GPU per expert
    e_miss = next(e for e in range(cfg.n_experts) if not (res >> e) & 1)
    dst = [torch.empty_like(host[n][e_miss], device="cuda") for n in names]
    for _ in range(3):
        for d_, n in zip(dst, names):
            d_.copy_(host[n][e_miss], non_blocking=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    reps = 8
    for _ in range(reps):
        for d_, n in zip(dst, names):
            d_.copy_(host[n][e_miss], non_blocking=True)
    torch.cuda.synchronize()
    pcie = reps * w_bytes / (time.perf_counter() - t0)
    # host throughput per expert and per pair, from a batch of eight missed
    # experts with one and with four pairs each (a lone expert leaves most
    # of the host's memory bandwidth idle)
    x_np = layer.x(max(tokens))
    cal = [e for e in range(cfg.n_experts) if not (res >> e) & 1][:8]
    hws = np.zeros(M.moe_host_ffn_workspace_size(dims, 4 * len(cal)), np.uint8)
    y = np.zeros((4 * len(cal), cfg.hidden), np.float32)
    hw = {n: host[n] for n in names}

    def host_time(n):
        best = float("inf")
        ex = [e for e in cal for _ in range(n)]
        for _ in range(5):
            t = time.perf_counter()
            M.moe_host_expert_ffn(dims, max(tokens), x_np, hw, [i % max(tokens) for i in range(len(ex))],
                                  ex, threads, y, hws)
            best = min(best, time.perf_counter() - t)
        return best / len(cal)
    t1, t4 = host_time(1), host_time(4)
    cpu_pair = max(0.0, (t4 - t1) / 3)
    cpu_expert = max(0.0, t1 - cpu_pair)

    def forward_ms(T, mode):
        x = tensor(layer.x(T), cfg.dtype, "cuda")
        out = torch.empty(T, cfg.hidden, dtype=torch.bfloat16 if cfg.dtype == "bf16" else torch.float32,
                          device="cuda")
        ws = torch.empty(M.moe_workspace_size(dims, T, mode), dtype=torch.uint8, device="cuda")
        rm = mask_tensor([res], "cuda")
        for _ in range(3):
            M.moe_layer_forward(dims, T, x, wdev, rm, 0, mode, out, ws)
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(steps):
            M.moe_layer_forward(dims, T, x, wdev, rm, 0, mode, out, ws)
            torch.cuda.synchronize()
        return (time.perf_counter() - t) / steps * 1e3

    out = dict(workload=f"{name} MoE layer, exact miss execution", mode="offload",
               resident_experts=bin(res).count("1"), host_threads=threads,
               calibration=dict(pcie_gbs=pcie / 1e9, expert_bytes=w_bytes,
                                host_expert_us=cpu_expert * 1e6, host_pair_us=cpu_pair * 1e6),
               batches=[])
    dev_b, host_b = M.moe_offload_workspace_size(dims, max(tokens))
    ws = torch.empty(dev_b, dtype=torch.uint8, device="cuda")
    hws_p = torch.empty(host_b, dtype=torch.uint8).pin_memory()
    g0, g1 = ev.create(), ev.create()
    for T in tokens:
        x = tensor(layer.x(T), cfg.dtype, "cuda")
        o = torch.empty(T, cfg.hidden, dtype=torch.bfloat16 if cfg.dtype == "bf16" else torch.float32,
                        device="cuda")
        std_ms = forward_ms(T, "standard")
        lore_ms = forward_ms(T, "lore")
        # GPU time per active expert: the all-resident forward over its experts
        dbg_ids = torch.empty(T * cfg.top_k, dtype=torch.int32, device="cuda")
        wsr = torch.empty(M.moe_workspace_size(dims, T, "standard"), dtype=torch.uint8, device="cuda")
        M.moe_layer_forward(dims, T, x, wdev, None, 0, "standard", o, wsr, debug={"topk_ids": dbg_ids})
        torch.cuda.synchronize()
        ids = dbg_ids.cpu().numpy()
        active = len(set(ids.tolist()))
        gpu_expert = std_ms * 1e-3 / max(1, active)
        plans = {"fetch_all": M.offload_cost(pcie, 0.0, 1.0, threads),
                 "host_all": M.offload_cost(pcie, 1.0, 0.0, threads),
                 "cost_rule": M.offload_cost(pcie, gpu_expert, cpu_pair, threads, cpu_expert),
                 "cost_rule_queued": M.offload_cost(pcie, gpu_expert, cpu_pair, threads,
                                                    cpu_expert, queue_aware=True)}
        row = dict(tokens=T, standard_all_resident_ms=std_ms, lore_surrogate_ms=lore_ms,
                   gpu_expert_us=gpu_expert * 1e6, plans={})
        for pname, cost in plans.items():
            for _ in range(2):
                M.moe_layer_forward_offload(dims, T, x, wdev, host, res, cost, o, ws, hws_p)
            torch.cuda.synchronize()
            t = time.perf_counter()
            for _ in range(steps):
                M.moe_layer_forward_offload(dims, T, x, wdev, host, res, cost, o, ws, hws_p)
                torch.cuda.synchronize()
            ms = (time.perf_counter() - t) / steps * 1e3
            st = M.MoeOffloadStats()
            st.gpu_start, st.gpu_stop = g0, g1
            M.moe_layer_forward_offload(dims, T, x, wdev, host, res, cost, o, ws, hws_p, stats=st)
            gpu_ms = ev.elapsed_ms(g0, g1)
            row["plans"][pname] = dict(
                ms=ms, missed=st.missed_experts, fetched=st.fetched_experts,
                host_experts=st.host_experts, host_pairs=st.host_pairs, route_ms=st.route_ms,
                host_ms=st.host_ms, gpu_ms=gpu_ms, parallel_ms=st.parallel_ms,
                hidden_ms=max(0.0, st.host_ms + gpu_ms - st.parallel_ms))
        out["batches"].append(row)
    ev.destroy(g0)
    ev.destroy(g1)
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_probe:
        copy_probe()
        return
    ev = HipEvents()
    import workloads as W
    head_layer = W.make_layer(args.workload)
    head = measure(args.workload, args.tokens, args.mode, args.steps, args.warmup, ev=ev,
                   layer=head_layer)
    also = []
    if not args.quick:
        plan = [("dsv2_lite", 1, "standard"), ("dsv2_lite", 1, "lore"),
                ("dsv2_lite", 8, "standard"), ("dsv2_lite", 8, "lore"),
                ("dsv2_lite", 64, "standard"), ("dsv2_lite", 64, "lore"),
                ("qwen2_57b", 1, "standard"), ("qwen2_57b", 1, "lore"),
                ("qwen2_57b", 32, "standard"), ("qwen2_57b", 32, "lore"),
                ("qwen2_57b", 256, "standard"), ("qwen2_57b", 256, "lore"),
                ("mixtral_floe", 1, "floe"),
                ("granite_prefill", 4096, "standard"), ("granite_prefill", 4096, "stall_free"),
                ("tiny", 16, "standard"), ("tiny", 16, "lore")]
        for name, T, mode in plan:
            if (name, T, mode) == (args.workload, args.tokens, args.mode):
                continue
            steps = max(10, min(args.steps, 50)) if T >= 256 else args.steps
            r = measure(name, T, mode, steps, min(args.warmup, 5), ev=ev)
            also.append(r)
            print(f"# {name} T={T} {mode}: {r['ms_per_step']*1e3:.1f} us/step "
                  f"(wall {r['wall_ms_per_step']*1e3:.1f} us, graph {r['graph']['ms_per_step']*1e3:.1f} us, "
                  f"p50 {r['step_us']['p50']:.1f} us) "
                  f"{r['tokens_per_s']:.0f} tok/s, {r['step_gbs']:.0f} GB/s"
                  + (f", {r['roofline']['kernel']} {r['roofline']['frac']*100:.1f}% of {r['roofline']['bound']}"
                     if 'roofline' in r else ""), file=sys.stderr, flush=True)
        r = measure_library_gemm(ev)
        also.append(r)
        print("# granite_prefill T=4096 grouped GEMM vs vendor GEMM on the same flops (no gather): " +
              "; ".join(f"{k}: ours {r[k]['ours_us']:.1f} us ({r[k]['ours_tflops']:.0f} TFLOP/s), "
                        f"dense {r[k]['dense_us']:.1f} us, batched {r[k]['batched_us']:.1f} us"
                        for k in ("gate_up", "down")), file=sys.stderr, flush=True)
        r = measure_prefetch_adaptive("granite_prefill_distilled", 4096, args.steps, min(args.warmup, 5))
        also.append(r)
        print(f"# granite_prefill_distilled T=4096 adaptive prefetch: {r['us_per_call']:.1f} us/call, "
              f"{r['gbs']:.0f} GB/s, mean budget {r['mean_budget']:.2f}, overlap {r['overlap']:.3f}, "
              f"covered {r['covered']:.3f}", file=sys.stderr, flush=True)
        r = measure_floe_predict(args.steps, min(args.warmup, 5))
        also.append(r)
        print(f"# mixtral_floe T=1 FloE predictor: {r['predict_us']:.1f} us/call "
              f"({r['predict_gbs']:.0f} GB/s); compact pack {r['pack_us']:.1f} us "
              f"({r['pack_gbs']:.0f} GB/s); recall {r['recall']:.3f} over {r['recall_tokens']} tokens",
              file=sys.stderr, flush=True)
        r = measure_offload(ev)
        also.append(r)
        for b in r["batches"]:
            print(f"# dsv2_lite T={b['tokens']} exact miss execution (resident "
                  f"{r['resident_experts']}/64): " + "; ".join(
                      f"{k} {v['ms']:.2f} ms (fetch {v['fetched']}, host {v['host_experts']})"
                      for k, v in b["plans"].items())
                  + f"; LoRE {b['lore_surrogate_ms']:.3f} ms, all resident "
                  f"{b['standard_all_resident_ms']:.3f} ms", file=sys.stderr, flush=True)
        r = measure_lore_fit()
        also.append(r)
        print(f"# dsv2_lite LoRE fit (expert 0, {r['tokens']} calibration rows): targets "
              f"{r['targets_ms']:.2f} ms; " + "; ".join(
                  f"rank {f['rank']}: {f['ms']:.1f} ms, error {f['rel_error']:.3f}" for f in r["fits"]),
              file=sys.stderr, flush=True)
    cpu = None if args.no_cpu else cpu_baseline(args.workload, args.tokens, args.mode,
                                                layer=head_layer)
    line = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) hidden states)",
        "config": {"workload": f"{args.workload} MoE layer, T={args.tokens}, mode={args.mode}",
                   "tokens": args.tokens, "mode": args.mode, "weight_copies": head["weight_copies"],
                   "step_bytes": head["step_bytes"], "step_gbs": head["step_gbs"],
                   "step_hbm_frac": head["step_hbm_frac"]},
        "roofline": head.get("roofline"),
        "step_us": head["step_us"],
        "graph": head["graph"],
        "cpu_baseline": cpu,
        "also": also,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
