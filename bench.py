"""Benchmark: quantized FFN layer tokens/s and achieved HBM GB/s on one MI355X.

A step is one call of the hot path (ffnq_dense: gate/up dequant GEMV with the
fused SiLU gate-multiply, down dequant GEMV, raw residual add) on the
Llama-3-8B-shaped FFN layer (hidden 4096, inter 14336, INT4-affine g64
weights, bf16 activations) at M tokens.  Inputs are synthetic and already
resident in HBM.  Steps rotate over several distinct copies of the layer's
weights (more bytes than the 256 MB Infinity Cache) so each step streams its
weights from HBM, as consecutive layers of a model do.

The weights are packed once per copy into the tiled layout (ffnq_pack, at
set-up, untimed: model-load work); --rowmajor streams the row-major layout.
The roofline object is for the dominant kernel (the gate/up kernel): its
algorithmic bytes (gate and up codes, scales and zeros, plus x) divided by its
average duration, timed live with HIP events that the library records around
its kernels on the call's stream (ffnq_set_phase_events: the events are
attached to the kernel dispatches, so they time the kernel itself).  `traffic` is the
HBM byte count of that kernel from rocprofv3 FETCH_SIZE + WRITE_SIZE counters,
scaled by the same counters on a plain copy of known size; it is read from
profiles/ and reported only while the kernel sources are the ones it was
measured on, else null.

Each roofline entry whose kernel streams 16 MB or more also carries
`read_ceiling_GBs`: the rate a plain streaming-read kernel of the library
(ffnq_stream_read) reaches for the same number of bytes on this GPU, read at
successive offsets of a 1 GiB sweep so that nothing comes from the Infinity
Cache -- the practical ceiling beside the published 8 TB/s (`read_ceiling`
lists them).

`value` is tokens/s over the wall clock of replays of a HIP graph that holds
one call per weight copy (the host's launch cost is not the product's);
per_m gives the eager per-call times (HIP events around each call).

Prints one JSON line.  --gpus above 1 is refused: this benchmark runs on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
KERNEL_SOURCES = tuple(f"moe_expert_dequant_amd/csrc/{f}" for f in
                       ("device.h", "qgemm.h", "tiled.h", "route.h", "stream.h", "prefill.h", "tail.h", "ffnq.hip"))
TRAFFIC_FILE = "profiles/traffic_gu_burst_kernel_int4_llama3-8b_m1.txt"


def weight_bytes(fmt: int, n: int, k: int) -> int:
    if fmt == 2:   # INT4-affine g64: codes + bf16 scale + bf16 zero per 64 inputs
        return n * k // 2 + 2 * 2 * (n * k // 64)
    return n * k + 4 * n   # INT8 per row: codes + fp32 scale


def layer_bytes(hidden: int, inter: int, fmt: int, m: int) -> int:
    """Algorithmic bytes of one dense FFN call with the residual tail: every
    weight byte once, x read, residual read and written."""
    w = 2 * weight_bytes(fmt, inter, hidden) + weight_bytes(fmt, hidden, inter)
    return w + m * hidden * 2 + 2 * m * hidden * 2


def gu_bytes(hidden: int, inter: int, fmt: int, m: int) -> int:
    """Algorithmic bytes of the gate/up kernel: gate and up weights once, x read.
    (The fp32 activation it hands to the down kernel is an intermediate.)"""
    return 2 * weight_bytes(fmt, inter, hidden) + m * hidden * 2


def sources_sha() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def read_traffic():
    """Measured HBM bytes per gate/up launch at M=1, if still valid for these sources."""
    path = os.path.join(ROOT, TRAFFIC_FILE)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith((" ", "#", "|")):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("sources_sha256") != sources_sha():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def setup(m: int, copies: int, tiled: bool = True):
    import torch
    import gen
    import moe_expert_dequant_amd as fq

    c = gen.CONFIGS[1]
    inp = gen.config_inputs(1, m)
    base = {n: fq.to_device(inp["ffn"][n]) for n in ("gate", "up", "down")}
    layers = []
    for i in range(copies):   # each copy is packed into its own tiled buffer (model-load time, not timed)
        d = {n: fq.pack(base[n]) for n in base} if tiled else \
            {n: {kk: (v.clone() if isinstance(v, torch.Tensor) else v) for kk, v in base[n].items()} for n in base}
        layers.append((d, fq.ffn_struct(d)))
    del base
    torch.cuda.synchronize()
    x = torch.from_numpy(inp["x"].view(np.int16)).cuda()
    resid = torch.from_numpy(inp["resid"].view(np.int16)).cuda()
    ws = fq.Workspace()
    stream = torch.cuda.current_stream()

    def step(i):   # on the current stream (the capture stream while a graph is recorded)
        fq.dense(layers[i % copies][1], c["hidden"], c["inter"], m, c["act"], c["tail"], x, resid, ws=ws)

    return c, step, stream


def run_gpu(m: int, steps: int, warmup: int, copies: int, tiled: bool = True):
    """Headline pass: wall clock over `steps` back-to-back calls, plus HIP
    events around each call."""
    import torch

    c, step, stream = setup(m, copies, tiled)
    for i in range(warmup):
        step(i)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record(stream)
        step(i)
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_call_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    return wall, per_call_ms, layer_bytes(c["hidden"], c["inter"], c["fmt"], m)


def run_graph(m: int, steps: int, warmup: int, copies: int, tiled: bool = True):
    """Headline pass: one HIP graph holds `copies` back-to-back calls (one per
    weight copy); it is replayed until `steps` calls have run, with the wall
    clock around the replays.  The kernels are the eager ones; the graph only
    removes the host's per-launch cost, as a serving loop would."""
    import torch

    c, step, stream = setup(m, copies, tiled)
    for i in range(max(warmup, copies)):
        step(i)                       # also sizes the workspace before capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(copies):
            step(i)
    g.replay()
    torch.cuda.synchronize()
    reps = max(1, (steps + copies - 1) // copies)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, reps * copies, e0.elapsed_time(e1) * 1e-3 / (reps * copies)


def run_phases(m: int, steps: int, warmup: int, copies: int, tiled: bool = True):
    """Per-kernel pass: the library records events before/after its kernels."""
    import torch
    import moe_expert_dequant_amd as fq

    c, step, stream = setup(m, copies, tiled)
    for i in range(warmup):
        step(i)
    evs = [fq.PhaseEvents(stream) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        with evs[i]:
            step(i)
    torch.cuda.synchronize()
    d = np.array([e.durations() for e in evs])   # ms: gate/up kernel, down kernel
    return d.mean(axis=0), gu_bytes(c["hidden"], c["inter"], c["fmt"], m)


# Steady-state timing of every workload shape: weight copies rotated so that the
# bytes a call touches, over all copies, exceed twice the 256 MB Infinity Cache
# (the 256x704 INT8 layer is L2-resident whatever is done, and is reported as a
# latency).  Routed layers time the whole layer from the router logits
# (ffnq_moe_layer_logits): router top-k and plan, shared expert (config 3),
# routed phases 1 and 2.
CONFIG_COPIES = {0: 1, 2: 6, 3: 6}


def _clone_mats(d: dict) -> dict:
    import torch
    return {n: {k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in m.items()} for n, m in d.items()}


def _dev16(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).cuda()


def run_config(c: int, m: int, steps: int, warmup: int) -> dict:
    import torch
    import gen
    import moe_expert_dequant_amd as fq

    cfg = gen.CONFIGS[c]
    inp = gen.config_inputs(c, m)
    hidden = cfg["hidden"]
    ws = fq.Workspace()
    x = _dev16(inp["x"])
    resid = _dev16(inp["resid"])
    if cfg["kind"] in ("dense", "shared"):
        inter = cfg["inter"]
        base = {n: fq.pack(fq.to_device(inp["ffn"][n])) for n in ("gate", "up", "down")}
        copies = CONFIG_COPIES.get(c, 6)
        layers = [base] + [_clone_mats(base) for _ in range(copies - 1)]
        structs = [fq.ffn_struct(d) for d in layers]
        wbytes = 2 * weight_bytes(cfg["fmt"], inter, hidden) + weight_bytes(cfg["fmt"], hidden, inter)
        if cfg["kind"] == "dense":
            io = 2 * m * hidden + 4 * m * hidden                          # x; residual read and written
            call = lambda i: fq.dense(structs[i % copies], hidden, inter, m, cfg["act"], cfg["tail"], x, resid, ws=ws)
        else:
            out = torch.zeros((m, hidden), dtype=torch.int16, device="cuda")
            nw = _dev16(inp["norm_w"])
            io = 2 * m * hidden + 2 * m * hidden + 2 * hidden            # x; norm output; norm weight
            call = lambda i: fq.shared_expert(structs[i % copies], hidden, inter, m, cfg["act"], cfg["tail"], x, out,
                                              nw, cfg["eps"], ws=ws)
        extra = {}
        bytes_of = lambda: wbytes + io
    else:
        E, inter, k, cap = cfg["n_experts"], cfg["moe_inter"], cfg["top_k"], cfg["cap"]
        sandwich = cfg["kind"] == "sandwich"
        sh_fmt = cfg.get("shared_fmt", cfg["fmt"])
        ex = {n: fq.pack(fq.to_device(inp["experts"][n]), E) for n in ("gate", "up", "down")}
        ebytes = 2 * weight_bytes(cfg["fmt"], inter, hidden) + weight_bytes(cfg["fmt"], hidden, inter)
        sh = None
        if cfg["shared_inter"]:
            sh = {n: fq.pack(fq.to_device(inp["shared"][n])) for n in ("gate", "up", "down")}
        logits = torch.from_numpy(np.ascontiguousarray(inp["logits"], dtype=np.float32)).cuda()
        ids = torch.zeros((m, k), dtype=torch.int32, device="cuda")
        w = torch.zeros((m, k), dtype=torch.float32, device="cuda")
        plan = torch.zeros((fq.plan_ints(m, k),), dtype=torch.int32, device="cuda")
        escale = torch.from_numpy(inp["expert_scale"]).cuda() if sandwich else None
        fq.moe_route(logits, m, E, k, cap, ids, w, plan, escale)
        torch.cuda.synchronize()
        p = plan.cpu().numpy()
        n_sub = min(max(int(p[0]), 0), m)
        union = min(max(int(p[m + 2 + n_sub]), 0), m * k)           # union entries of all sub-batches
        touched = union * ebytes + (0 if sh is None else 2 * weight_bytes(sh_fmt, cfg["shared_inter"], hidden)
                                    + weight_bytes(sh_fmt, hidden, cfg["shared_inter"]))
        copies = max(2, -(-2 * 256 * 1000 * 1000 // max(touched, 1)))
        exs = [ex] + [_clone_mats(ex) for _ in range(copies - 1)]
        ex_st = [fq.ffn_struct(d) for d in exs]
        # the copies' tensors stay referenced for as long as their structs are used (a struct holds raw pointers)
        sh_copies = None if sh is None else [sh] + [_clone_mats(sh) for _ in range(copies - 1)]
        shs = None if sh is None else [fq.ffn_struct(d) for d in sh_copies]
        gv = _dev16(inp["gate_vec"]) if (sh is not None and not sandwich) else None

        if sandwich:
            n1, n2 = _dev16(inp["shared_norm_w"]), _dev16(inp["post_norm_w"])

            def call(i):   # route (expert scale), shared branch + its norm, unseeded routed half, sandwich tail
                fq.moe_layer_sandwich(ex_st[i % copies], E, hidden, inter, m, k, cfg["act"], shs[i % copies],
                                      cfg["shared_inter"], n1, n2, cfg["eps"], x, logits, cap, ids, w, plan, resid,
                                      expert_scale=escale, ws=ws)
        else:
            def call(i):   # router top-k + plan, the gated shared expert and the routed half: one call
                fq.moe_layer_logits(ex_st[i % copies], E, hidden, inter, m, k, cfg["act"],
                                    None if shs is None else shs[i % copies], cfg["shared_inter"] or 0, gv, x,
                                    logits, cap, ids, w, plan, resid, ws=ws)
        counts = np.bincount(ids.cpu().numpy().ravel(), minlength=E)
        extra = dict(union=union, sub_batches=n_sub, tokens_per_expert_min=int(counts[counts > 0].min()),
                     tokens_per_expert_max=int(counts.max()))
        extra["router_gemv_us"] = time_router_gemv(x, m, hidden, E)
        io = 2 * m * hidden + 4 * m * E + 4 * m * hidden                 # x; logits; residual read and written
        if sandwich:
            io += 4 * hidden + 4 * E                                     # the two norm weights; the expert scale
        bytes_of = lambda: touched + io
    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    # per-kernel figures for the layers whose gate/up and down each run in one launch
    phases = kernel_phases(c, m, cfg, call, min(steps, 50), extra.get("union")) if cfg["kind"] != "sandwich" else []
    graph_us = graph_call_us(call, max(copies, 8), steps)
    st = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    en = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        st[i].record()
        call(i)
        en[i].record()
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in zip(st, en)]) * 1e-3   # s
    med = float(np.median(t))
    nb = bytes_of()
    return dict(call_us_median=med * 1e6, call_us_p10=float(np.percentile(t, 10)) * 1e6,
                call_us_p90=float(np.percentile(t, 90)) * 1e6, tokens_per_s=m / med, bytes_per_call=nb,
                achieved_GBs=nb / med / 1e9, frac_of_peak=nb / med / 1e9 / HBM_PEAK_GBS, weight_copies=copies,
                graph_call_us=graph_us, graph_tokens_per_s=m / (graph_us * 1e-6),
                graph_frac_of_peak=nb / (graph_us * 1e-6) / 1e9 / HBM_PEAK_GBS, kernels=phases, **extra)


# The kernels the library launches for the gate/up and down phases of each
# workload shape (its dispatch at these sizes; the rocprofv3 kernel traces
# under profiles/ list the same names).
def kernel_names(c: int, m: int):
    dense_gu = {0: "INT8", 1: "INT4", 2: "INT8"}
    if c in dense_gu:
        f = dense_gu[c]
        r_gu = m if m <= 4 else 8
        down = f"down_burst_kernel<{f},{2 * m if m <= 2 else 8}>" if m <= 4 else f"down_tiled_kernel<{f},...>"
        return f"gu_burst_kernel<{f},{r_gu}>", down
    if c == 3:
        return (f"gu_burst_kernel<INT4,{m}> (shared + routed gate/up{', routing' if m * 128 <= 128 else ''})",
                f"moe_down_kernel<INT4,{2 * m if m <= 2 else 8},1> (shared + routed down, seeded reduce, residual)")
    if m == 1:
        return ("gu_burst_kernel<INT4,1> (routed gate/up, routing)",
                "moe_down_kernel<INT4,2,1> (routed down, reduce, residual)")
    return ("prefill_kernel<12 waves, gate+up> (grouped bf16-MFMA gate/up + SiLU, staged K chunks)",
            "prefill_kernel<8 waves, down> (grouped bf16-MFMA down, fp32 partials per K range; the reduction "
            "with the residual is a launch of its own)")


def kernel_phases(c: int, m: int, cfg: dict, call, n: int, union) -> list:
    """Average duration of the gate/up and of the down launch of one call (HIP
    events that the library attaches to those kernel dispatches) and each
    one's algorithmic bytes: the weights it must read (the union's experts for
    a routed layer), x for gate/up, the residual read and write when the tail
    runs in the down kernel.  FLOPs are 2 per weight per token (per pair)."""
    import torch
    import moe_expert_dequant_amd as fq

    hidden, fmt = cfg["hidden"], cfg["fmt"]
    if cfg["kind"] in ("dense", "shared"):
        inter = cfg["inter"]
        gu_b = 2 * weight_bytes(fmt, inter, hidden) + 2 * m * hidden
        dn_b = weight_bytes(fmt, hidden, inter) + (4 * m * hidden if cfg["kind"] == "dense" else 0)
        gu_f, dn_f = 2 * m * 2 * inter * hidden, 2 * m * hidden * inter
    else:
        inter, k, si = cfg["moe_inter"], cfg["top_k"], cfg["shared_inter"] or 0
        gu_b = union * 2 * weight_bytes(fmt, inter, hidden) + 2 * m * hidden
        dn_b = union * weight_bytes(fmt, hidden, inter) + 4 * m * hidden
        gu_f, dn_f = 2 * m * k * 2 * inter * hidden, 2 * m * k * hidden * inter
        if si:
            gu_b += 2 * weight_bytes(fmt, si, hidden) + 2 * hidden      # shared gate/up; its gate vector
            dn_b += weight_bytes(fmt, hidden, si)
            gu_f += 2 * m * 2 * si * hidden
            dn_f += 2 * m * hidden * si
    evs = [fq.PhaseEvents() for _ in range(n)]
    torch.cuda.synchronize()
    for i in range(n):
        with evs[i]:
            call(i)
    torch.cuda.synchronize()
    d = np.array([e.durations() for e in evs]).mean(axis=0) * 1e-3   # s: gate/up, down
    names = kernel_names(c, m)
    out = []
    for name, phase, b, f, t in ((names[0], "gate_up", gu_b, gu_f, d[0]), (names[1], "down", dn_b, dn_f, d[1])):
        gbs = b / t / 1e9
        e = dict(workload=cfg["name"], m=m, phase=phase, kernel=name, bound="hbm", achieved=gbs, peak=HBM_PEAK_GBS,
                 unit="GB/s", frac=gbs / HBM_PEAK_GBS, algorithmic_bytes_per_launch=b, avg_launch_us=t * 1e6,
                 flops_per_launch=f, tflops=f / t / 1e12)
        if m * (cfg.get("top_k") or 1) >= 64:   # the grouped prefill GEMMs run on bf16 MFMA
            e["mfma_frac"] = f / t / 1e12 / BF16_MFMA_PEAK_TFLOPS
        out.append(e)
    return out


def graph_call_us(call, ncalls: int, steps: int) -> float:
    """Per-call time of `ncalls` calls captured in one HIP graph and replayed
    (the launches of a layer without the host's per-launch cost)."""
    import torch

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(ncalls):
            call(i)
    g.replay()
    torch.cuda.synchronize()
    reps = max(2, steps // ncalls)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (reps * ncalls)


def time_router_gemv(x, m: int, hidden: int, E: int, calls: int = 50) -> float:
    """Time per call (us) of the router GEMV in front of the top-k (ffnq_router_logits) on a seeded bf16
    router weight [E][hidden] (N(0,1)/sqrt(hidden)): `calls` back-to-back calls between two HIP events, so
    that the events' own cost is spread (a single short kernel between two events mostly times the events).
    Not part of the layer figures, whose workload takes the logits as input."""
    import torch
    import gen
    import moe_expert_dequant_amd as fq

    rng = np.random.default_rng(1000 + E)
    w = _dev16(gen.bf16_bits(rng.standard_normal((E, hidden)) / np.sqrt(hidden)))
    lg = torch.empty((m, E), dtype=torch.float32, device="cuda")
    for _ in range(5):
        fq.router_logits(x, w, m, hidden, E, lg)
    st, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    st.record()
    for _ in range(calls):
        fq.router_logits(x, w, m, hidden, E, lg)
    en.record()
    torch.cuda.synchronize()
    return st.elapsed_time(en) * 1e3 / calls


def run_streamed(c: int, m: int, steps: int, warmup: int) -> dict:
    """Workload c's routed half with its experts in pinned host memory (ffnq_moe_routed_streamed, slot cache of
    `cap` slots): `cold` empties the slot table before every call, so every union expert crosses PCIe (the
    expert-store case of a model larger than HBM); `warm` keeps it, so repeated routes copy nothing.  Each call
    reads the routes back to the host once, so the time is the wall clock of the call through a synchronize."""
    import torch
    import gen
    import moe_expert_dequant_amd as fq

    cfg = gen.CONFIGS[c]
    inp = gen.config_inputs(c, m)
    hidden, E, inter, k, cap = cfg["hidden"], cfg["n_experts"], cfg["moe_inter"], cfg["top_k"], cfg["cap"]
    d = {n: fq.pack(fq.to_device(inp["experts"][n]), E) for n in ("gate", "up", "down")}
    hx_d, hx = fq.host_experts(d)
    del d
    logits = torch.from_numpy(np.ascontiguousarray(inp["logits"], dtype=np.float32)).cuda()
    ids = torch.zeros((m, k), dtype=torch.int32, device="cuda")
    w = torch.zeros((m, k), dtype=torch.float32, device="cuda")
    plan = torch.zeros((fq.plan_ints(m, k),), dtype=torch.int32, device="cuda")
    fq.moe_route(logits, m, E, k, cap, ids, w, plan)
    x, resid = _dev16(inp["x"]), _dev16(inp["resid"])
    cache = fq.SlotCache(cap, hidden, inter)
    ws = fq.Workspace()
    torch.cuda.synchronize()
    union = len(set(ids.cpu().numpy().ravel().tolist()))
    ebytes = 2 * weight_bytes(cfg["fmt"], inter, hidden) + weight_bytes(cfg["fmt"], hidden, inter)

    def timed(cold: bool, n: int):
        t = []
        for _ in range(n):
            if cold:
                cache.expert[:] = -1
            t0 = time.perf_counter()
            fq.moe_routed_streamed(hx, E, hidden, inter, m, k, cfg["act"], x, ids, w, plan, None, resid, cache, ws=ws)
            torch.cuda.synchronize()
            t.append(time.perf_counter() - t0)
        return float(np.median(t))

    timed(True, warmup)
    copied0 = cache.copied
    cold = timed(True, steps)
    cold_copies = (cache.copied - copied0) / steps
    timed(False, 2)
    copied0 = cache.copied
    warm = timed(False, steps)
    return dict(union=union, expert_bytes=ebytes, slots=cap, cold_call_us=cold * 1e6, cold_tokens_per_s=m / cold,
                cold_experts_copied_per_call=cold_copies, pcie_GBs=union * ebytes / cold / 1e9,
                warm_call_us=warm * 1e6, warm_tokens_per_s=m / warm,
                warm_experts_copied_per_call=(cache.copied - copied0) / steps)


def run_configs(steps: int, warmup: int) -> dict:
    import gen
    out = {}
    for c in sorted(gen.CONFIGS):
        cfg = gen.CONFIGS[c]
        out[cfg["name"]] = {f"M={m}": run_config(c, m, steps, warmup) for m in cfg["ms"]}
        print(f"# config {c} done", file=sys.stderr, flush=True)
    # the Qwen-shaped routed half streamed from host memory through the slot cache
    out["qwen3-moe-int4-streamed-from-host"] = {f"M={m}": run_streamed(3, m, 30, 3) for m in (1, 4)}
    print("# streamed done", file=sys.stderr, flush=True)
    return out


READ_POOL = 1 << 30   # bytes swept by the read-rate probe before any byte is read again (4x the Infinity Cache)
READ_MIN_BYTES = 16 << 20   # kernels that stream less than this are L2/Infinity-Cache latency cases


def read_ceiling(sizes, steps: int = 30, warmup: int = 5) -> dict:
    """The read rate a plain streaming-read kernel (ffnq_stream_read) reaches for each byte count: each launch
    reads `size` bytes at the next offset of a 1 GiB sweep, timed by events the dispatch itself records.
    Returns {size: (median us, GB/s)}."""
    import torch
    import moe_expert_dequant_amd as fq

    sizes = sorted({int(b) // 16 * 16 for b in sizes if b >= 16})
    if not sizes:
        return {}
    buf = torch.ones(READ_POOL + sizes[-1], dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = {}
    for size in sizes:
        stride = (size + 65535) // 65536 * 65536
        slots = max(1, READ_POOL // stride)
        evs = [fq.PhaseEvents() for _ in range(steps)]
        for i in range(warmup + steps):
            view = buf[(i % slots) * stride:(i % slots) * stride + size]
            if i < warmup:
                fq.stream_read(view, sink)
                continue
            with evs[i - warmup]:
                fq.stream_read(view, sink)
        torch.cuda.synchronize()
        us = float(np.median([e.durations()[0] for e in evs])) * 1e3
        out[size] = (us, size / (us * 1e-6) / 1e9)
    del buf
    return out


def attach_read_ceiling(entries, rc: dict) -> None:
    """Adds the plain-read rate for the same bytes to each roofline entry that streams from HBM."""
    for e in entries:
        b = int(e.get("algorithmic_bytes_per_launch", 0)) // 16 * 16
        if b in rc:
            e["read_ceiling_GBs"] = rc[b][1]
            e["frac_of_read_ceiling"] = e["achieved"] / rc[b][1]


def copy_calibration(nbytes: int = 1 << 30, reps: int = 5):
    """A plain device copy of known size, for scaling FETCH_SIZE / WRITE_SIZE."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reps": reps}), flush=True)


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_dense_by_rows(inp, c, pool, nthr: int):
    """One token through the oracle's own step functions (gemv, act, residual),
    each projection partitioned by output rows over `nthr` threads (ctypes
    releases the GIL); the result is that of oracle.dense, bit for bit."""
    import gen
    import oracle

    hidden, inter = c["hidden"], c["inter"]

    def rows(mat, r0, r1):   # rows [r0, r1) of a row-major INT4 matrix (views, no copy)
        return dict(fmt=mat["fmt"], n=r1 - r0, k=mat["k"], q=mat["q"][r0:r1], s=mat["s"][r0:r1], z=mat["z"][r0:r1])

    def gemv_par(mat, x):
        n = mat["n"]
        b = [(n * i // nthr) // 16 * 16 for i in range(nthr)] + [n]
        parts = list(pool.map(lambda i: oracle.gemv(rows(mat, b[i], b[i + 1]), x), range(nthr)))
        return np.concatenate(parts)

    f = inp["ffn"]
    x = gen.bf16_to_f32(inp["x"][0]).astype(np.float64)
    g = gemv_par(f["gate"], x)
    u = gemv_par(f["up"], x)
    a = np.array([oracle.act(c["act"], float(gi), float(ui)) for gi, ui in zip(g, u)], dtype=np.float64)
    h = gemv_par(f["down"], a)
    return np.array([oracle.residual(int(r), float(v)) for r, v in zip(inp["resid"][0], h)], np.uint16)


def cpu_baseline(budget_s: float = 8.0):
    """The oracle as it stands on the Llama-shaped layer: single-threaded and pinned to one core (M = 1 and
    M = 4), then its step functions partitioned by output rows over every core this process may use (M = 1)."""
    from concurrent.futures import ThreadPoolExecutor
    import gen
    import oracle

    c = gen.CONFIGS[1]
    inp1 = gen.config_inputs(1, 1)
    inp4 = gen.config_inputs(1, 4)
    oracle.lib()
    cpus = sorted(os.sched_getaffinity(0))
    pinned = cpus[0]
    os.sched_setaffinity(0, {pinned})
    try:
        n1, t0 = 0, time.perf_counter()
        while True:
            ref1 = oracle.dense(inp1["ffn"], c["hidden"], c["inter"], c["act"], c["tail"], inp1["x"], inp1["resid"])
            n1 += 1
            el1 = time.perf_counter() - t0
            if el1 >= budget_s or n1 >= 64:
                break
        n4, t0 = 0, time.perf_counter()
        while True:
            oracle.dense(inp4["ffn"], c["hidden"], c["inter"], c["act"], c["tail"], inp4["x"], inp4["resid"])
            n4 += 1
            el4 = time.perf_counter() - t0
            if el4 >= budget_s / 2 or n4 >= 16:
                break
    finally:
        os.sched_setaffinity(0, set(cpus))
    nthr = len(cpus)
    with ThreadPoolExecutor(nthr) as pool:
        got = _oracle_dense_by_rows(inp1, c, pool, nthr)
        assert np.array_equal(got, ref1[0]), "row-partitioned oracle differs from the single-threaded one"
        nm, t0 = 0, time.perf_counter()
        while True:
            _oracle_dense_by_rows(inp1, c, pool, nthr)
            nm += 1
            elm = time.perf_counter() - t0
            if elm >= budget_s / 2 or nm >= 64:
                break
    return dict(value=n1 / el1, unit="tokens/s", cores=1, kind="oracle",
                sample=f"{n1} single-token calls (M=1) of the llama3-8b-shaped INT4 FFN layer, {el1:.1f} s, "
                       f"one thread pinned to CPU {pinned}",
                cpu_model=_cpu_model(), host_cpus=os.cpu_count(), usable_cpus=nthr, pinned_cpu=pinned,
                m4=dict(value=4 * n4 / el4, unit="tokens/s", cores=1, sample=f"{n4} calls at M=4, {el4:.1f} s"),
                row_partitioned=dict(value=nm / elm, unit="tokens/s", cores=nthr,
                                     sample=f"{nm} single-token calls, gate/up and down GEMVs split by output rows "
                                            f"over {nthr} threads, bit-identical to the single-threaded oracle, "
                                            f"{elm:.1f} s"))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--m", type=int, default=1, help="tokens per call for the headline value")
    ap.add_argument("--copies", type=int, default=8, help="distinct weight copies rotated over")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--single", action="store_true", help="time only --m, headline pass only (for profiling runs)")
    ap.add_argument("--copy-calibration", action="store_true", help="run a plain 1 GiB copy (counter calibration)")
    ap.add_argument("--rowmajor", action="store_true", help="stream the row-major weights instead of the tiled ones")
    ap.add_argument("--no-configs", action="store_true", help="skip the steady-state timing of every workload shape")
    ap.add_argument("--streamed", action="store_true",
                    help="time only the Qwen-shaped routed half streamed from host memory at --m tokens")
    ap.add_argument("--config", type=int, default=None,
                    help="time only workload shape CONFIG at --m tokens (steady state; for kernel traces)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU sharding is a "
              "design note, not a measured path", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.streamed:
        print(json.dumps({"config": 3, "m": args.m, "streamed": run_streamed(3, args.m, args.steps, args.warmup)}),
              flush=True)
        return
    if args.config is not None:
        r = run_config(args.config, args.m, args.steps, args.warmup)
        print(json.dumps({"config": args.config, "m": args.m, **r}), flush=True)
        return

    res = {}
    for m in ([args.m] if args.single else sorted({args.m, 1, 4})):
        wall, per_call, nbytes = run_gpu(m, args.steps, args.warmup, args.copies, not args.rowmajor)
        avg = float(np.mean(per_call)) * 1e-3
        res[m] = dict(wall=wall, avg_s=avg, med_s=float(np.median(per_call)) * 1e-3, bytes=nbytes,
                      p10_s=float(np.percentile(per_call, 10)) * 1e-3, p90_s=float(np.percentile(per_call, 90)) * 1e-3)
    phases = {}
    if not args.single:
        for m in res:
            ms, gb = run_phases(m, min(args.steps, 100), args.warmup, args.copies, not args.rowmajor)
            phases[m] = dict(gu_us=ms[0] * 1e3, down_us=ms[1] * 1e3, gu_bytes=gb)

    gwall, gcalls, gcall_s = run_graph(args.m, args.steps, args.warmup, args.copies, not args.rowmajor)
    h = res[args.m]
    value = args.m * gcalls / gwall
    out = {
        "metric": "quantized FFN layer tokens/s + achieved HBM GB/s (% of peak) at M=1 and M=4",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": gwall / gcalls * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"llama3-8b-shaped dense FFN layer, hidden 4096, inter 14336, INT4-affine g64, SiLU, "
                        f"residual tail, M={args.m}",
            "m": args.m,
            "weight_copies_rotated": args.copies,
            "weight_layout": "row-major" if args.rowmajor else "tiled (ffnq_pack, once per copy, untimed)",
            "launch": f"HIP graph of {args.copies} calls (one per weight copy), replayed; "
                      f"eager calls: {args.m * args.steps / h['wall']:.0f} tokens/s",
            "parallelism": "single GPU",
        },
    }
    if args.m in phases:
        p = phases[args.m]
        achieved = p["gu_bytes"] / (p["gu_us"] * 1e-6) / 1e9
        traffic = read_traffic() if args.m == 1 else None
        out["roofline"] = {
            "bound": "hbm",
            "kernel": ("gu_kernel<INT4,...>" if args.rowmajor else f"gu_burst_kernel<INT4,{args.m if args.m <= 4 else 8}>") +
                      " (gate+up dequant GEMV + SiLU gate-multiply)",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": p["gu_bytes"],
            "avg_launch_us": p["gu_us"],
        }
    out["graph_call_us"] = gcall_s * 1e6
    out["per_m"] = {str(m): {"tokens_per_s": m / r["avg_s"], "call_us_mean": r["avg_s"] * 1e6,
                             "call_us_median": r["med_s"] * 1e6, "call_us_p10": r["p10_s"] * 1e6,
                             "call_us_p90": r["p90_s"] * 1e6, "bytes_per_call": r["bytes"],
                             "achieved_GBs": r["bytes"] / r["avg_s"] / 1e9,
                             "frac_of_peak": r["bytes"] / r["avg_s"] / 1e9 / HBM_PEAK_GBS,
                             **({k: v for k, v in phases[m].items()} if m in phases else {})}
                    for m, r in res.items()}
    if not (args.no_configs or args.single):
        out["configs"] = run_configs(100, 10)
        # every workload shape's gate/up and down kernels against their roofline
        out["roofline_kernels"] = [k for cf in out["configs"].values() for r in cf.values() for k in r.get("kernels", [])]
    entries = ([out["roofline"]] if "roofline" in out else []) + out.get("roofline_kernels", [])
    big = [e["algorithmic_bytes_per_launch"] for e in entries if e.get("algorithmic_bytes_per_launch", 0) >= READ_MIN_BYTES]
    if big:
        rc = read_ceiling(big)
        attach_read_ceiling(entries, rc)
        out["read_ceiling"] = [{"bytes": b, "us": v[0], "GBs": v[1], "frac_of_peak": v[1] / HBM_PEAK_GBS,
                                "kernel": f"stream_read_kernel (256 x 512 threads, 16-byte loads)"}
                               for b, v in sorted(rc.items())]
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
