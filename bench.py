#!/usr/bin/env python3
"""Benchmark of the sparse-MoE layer on one MI355X.

One step = one whole MoE layer (router GEMM, top-k, grouping, gate/up grouped
GEMM with SwiGLU, down grouped GEMM writing each slot's output, weighted
combine) over one batch of T synthetic tokens, inputs and weights resident in
HBM.

Headline (``value``): prefill tokens/s of one layer at T=4096 (hidden 2048,
256 experts top-8 + 1 shared expert, expert intermediate 512, int4 group-64
weights).  Also reported: the layer's fraction of dense bf16 MFMA peak, the
dominant kernel's roofline (timed live with HIP events on the launch stream),
per-stage times, batch-1 decode over 40 stacked layers x 256 steps as HBM GB/s,
the GPU-resident vs host-synchronised routing ablation at T=512, a T=1..16
small-batch sweep, T=64 and T=512 as fractions of HBM bandwidth, the skewed
routing stress layer at T=16384 with its expert load, and the CPU oracle timed
on a bounded token sample of the same workload.

Prints exactly one JSON line on stdout; progress goes to stderr.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def layer_flops_per_token(d) -> int:
    """MFMA-eligible flops per token: (k routed + 1 shared) experts x 3 matrices."""
    return (d.top_k * 3 * 2 * d.hidden * d.inter) + 3 * 2 * d.hidden * d.shared_inter


def gate_up_flops(d, T) -> int:
    return 2 * (T * d.top_k * 2 * d.inter + T * 2 * d.shared_inter) * d.hidden


def expert_bytes(d) -> int:
    """int4 codes + fp16 scale + fp16 bias of one expert's three matrices."""
    n = 3 * d.hidden * d.inter
    return n // 2 + 2 * 2 * (n // d.group_size)


def decode_bytes_per_layer(d) -> int:
    shared = expert_bytes(synth_dims_shared(d))
    return (d.top_k * expert_bytes(d) + shared + d.n_experts * d.hidden * 4 + d.hidden * 4
            + 2 * d.hidden * 2)


def synth_dims_shared(d):
    import synth
    return synth.Dims(hidden=d.hidden, inter=d.shared_inter, n_experts=1, top_k=1, group_size=d.group_size,
                      shared_inter=d.shared_inter)


def device_layer(lay, d, moe, pack=True):
    import torch
    t = lambda a: None if a is None else a.to("cuda").contiguous()
    q = lambda m: tuple(t(a) for a in m)
    return moe.LayerWeights(moe.Dims(d.hidden, d.inter, d.n_experts, d.top_k, d.group_size, d.shared_inter),
                            q(lay.gate_up), q(lay.down), q(lay.sh_gate_up), q(lay.sh_down), t(lay.router_w),
                            t(lay.shared_gate_w), t(lay.router_bias), pack=pack)


def warm_graph(g, min_replays, min_seconds=0.025):
    """Untimed replays of graph g until the work runs at its steady rate: at
    least min_replays, and at least min_seconds of replays (the first ~20 ms
    of back-to-back work after a capture run several per cent slower)."""
    import torch
    t0 = time.perf_counter()
    n = 0
    while True:
        for _ in range(8):
            g.replay()
        n += 8
        torch.cuda.synchronize()
        if n >= min_replays and time.perf_counter() - t0 >= min_seconds:
            return n


def time_stages(moe, md, dl, x, y, ws, reps):
    """Average GPU time (us) of each stage of the layer, measured inside whole
    layers: HIP events recorded between the stages on the launch stream."""
    import torch
    n = len(moe.STAGES)
    s = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(n + 1)] for _ in range(reps)]
    moe.moe_forward(md, dl, x, y=y, workspace=ws)
    for r in range(reps):
        for i in range(n):
            ev[r][i].record(s)
            moe.moe_forward_stages(md, dl, x, y, ws, i, i)
        ev[r][n].record(s)
    torch.cuda.synchronize()
    return {name: sum(ev[r][i].elapsed_time(ev[r][i + 1]) for r in range(reps)) * 1000.0 / reps
            for i, name in enumerate(moe.STAGES)}


def bench_prefill(cfg, steps, warmup):
    import torch
    import sparse_moe_softmax_amd as moe
    import synth
    d = cfg.dims
    md = moe.Dims(d.hidden, d.inter, d.n_experts, d.top_k, d.group_size, d.shared_inter)
    log(f"prefill {cfg.name}: generating weights (seed {cfg.seed})")
    lay = synth.make_layer(d, cfg.seed, zipf_bias=cfg.zipf_bias, device="cuda")
    dl = device_layer(lay, d, moe)
    x_cpu = synth.activations(cfg.T, d.hidden, cfg.seed)
    x = x_cpu.cuda()
    T = cfg.T
    ws = moe.moe_workspace(md, T)
    y = torch.empty((T, d.hidden), dtype=torch.bfloat16, device="cuda")
    logits = torch.empty((T, d.n_experts), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, d.top_k), dtype=torch.int32, device="cuda")
    for _ in range(warmup):
        moe.moe_forward(md, dl, x, y=y, workspace=ws)
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # eager launches (one host call per layer, seven kernels)
    e0.record(s)
    for _ in range(steps):
        moe.moe_forward(md, dl, x, y=y, workspace=ws)
    e1.record(s)
    torch.cuda.synchronize()
    eager_ms = e0.elapsed_time(e1) / steps
    # the timed steps: the layer captured once as a HIP graph and replayed
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.moe_forward(md, dl, x, y=y, workspace=ws)
    warm_graph(g, max(48, warmup))   # untimed, until the layer runs at its steady rate
    t0 = time.perf_counter()
    e0.record(s)
    for _ in range(steps):
        g.replay()
    e1.record(s)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall_ms = (t1 - t0) * 1000.0 / steps
    gpu_ms = e0.elapsed_time(e1) / steps
    # the spread: the same replays again, an event between every two
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(s)
    for i in range(steps):
        g.replay()
        ev[i + 1].record(s)
    torch.cuda.synchronize()
    per = sorted(ev[i].elapsed_time(ev[i + 1]) * 1000.0 for i in range(steps))
    pct = {f"p{q}": round(per[min(steps - 1, int(q / 100 * steps))], 2) for q in (10, 50, 90)}
    log(f"prefill {cfg.name}: {wall_ms:.4f} ms/step wall, {gpu_ms:.4f} ms/step gpu events (HIP graph); "
        f"eager launches {eager_ms:.4f} ms/step")
    stages = time_stages(moe, md, dl, x, y, ws, reps=max(10, steps))
    log("stages (us):", {k: round(v, 2) for k, v in stages.items()})
    # final forward with routing outputs kept for the cross-check in the CPU leg
    moe.moe_forward(md, dl, x, y=y, logits_out=logits, ids_out=ids, workspace=ws)
    torch.cuda.synchronize()
    return {"cfg": cfg, "lay": lay, "x_cpu": x_cpu, "wall_ms": wall_ms, "gpu_ms": gpu_ms, "eager_ms": eager_ms,
            "pct_us": pct, "stages": stages, "y": y, "logits": logits, "ids": ids}


def bench_decode(cfg, n_steps, graph_chunk=32):
    import torch
    import sparse_moe_softmax_amd as moe
    import synth
    d = cfg.dims
    md = moe.Dims(d.hidden, d.inter, d.n_experts, d.top_k, d.group_size, d.shared_inter)
    log(f"decode: generating {cfg.layers} layers (seed {cfg.seed})")
    layers = []
    for l in range(cfg.layers):
        lay = synth.make_layer(d, cfg.seed, layer=l, device="cuda")
        layers.append(device_layer(lay, d, moe, pack=False))   # T == 1 reads the canonical layout
    xs = torch.stack([synth.activations(1, d.hidden, cfg.seed, step=s)[0] for s in range(n_steps)]).cuda()
    ws = moe.moe_workspace(md, 1)
    ys = torch.empty((cfg.layers, d.hidden), dtype=torch.bfloat16, device="cuda")

    def step(s):
        xi = xs[s:s + 1]
        for l, dl in enumerate(layers):
            moe.moe_forward(md, dl, xi, y=ys[l:l + 1], workspace=ws)

    step(0)
    torch.cuda.synchronize()
    graphs = []
    for c0 in range(0, n_steps, graph_chunk):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for s in range(c0, min(n_steps, c0 + graph_chunk)):
                step(s)
        graphs.append(g)
    torch.cuda.synchronize()
    for g in graphs[:1]:
        g.replay()                # warm
    torch.cuda.synchronize()
    s_ = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(s_)
    for g in graphs:
        g.replay()
    e1.record(s_)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    flags = moe.moe_workspace_errors(ws)   # a fused-layer wait that gave up would be flagged here
    gpu_s = e0.elapsed_time(e1) / 1000.0
    bytes_step = cfg.layers * decode_bytes_per_layer(d)
    gbs = n_steps * bytes_step / gpu_s / 1e9
    log(f"decode: {n_steps} steps x {cfg.layers} layers in {gpu_s * 1000:.2f} ms (wall {(t1 - t0) * 1000:.2f}), "
        f"{gbs:.1f} GB/s")
    return {"metric": "batch-1 decode HBM GB/s (algorithmic bytes)", "value": round(gbs, 2), "unit": "GB/s",
            "frac_of_peak": round(gbs / PEAK_HBM_GBS, 4), "us_per_step": round(gpu_s * 1e6 / n_steps, 2),
            "us_per_layer": round(gpu_s * 1e6 / n_steps / cfg.layers, 3), "steps": n_steps, "layers": cfg.layers,
            "bytes_per_layer": decode_bytes_per_layer(d), "launch": "HIP graphs of 32 steps",
            "workload": "decode T=1, 40 layers distinct seeded int4 weights, fresh x per step",
            "device_error_flags": flags}


def bench_routing_ablation(cfg, steps, warmup):
    """GPU-resident grouping (moe_forward) against the variant that takes the
    expert counts through the host and builds offsets and block map there
    (moe_forward_host_routing), eager launches, wall clock per layer."""
    import torch
    import sparse_moe_softmax_amd as moe
    import synth
    d = cfg.dims
    md = moe.Dims(d.hidden, d.inter, d.n_experts, d.top_k, d.group_size, d.shared_inter)
    lay = synth.make_layer(d, cfg.seed, zipf_bias=cfg.zipf_bias, device="cuda")
    dl = device_layer(lay, d, moe)
    x = synth.activations(cfg.T, d.hidden, cfg.seed).cuda()
    ws = moe.moe_workspace(md, cfg.T)
    hb = torch.empty(moe.moe_host_routing_bytes(md, cfg.T), dtype=torch.uint8, pin_memory=True)
    y = torch.empty((cfg.T, d.hidden), dtype=torch.bfloat16, device="cuda")
    y2 = torch.empty_like(y)
    runs = {"gpu_resident": lambda: moe.moe_forward(md, dl, x, y=y, workspace=ws),
            "host_synchronised": lambda: moe.moe_forward_host_routing(md, dl, x, y=y2, workspace=ws, host_buf=hb)}
    out = {}
    for name, fn in runs.items():
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        out[name] = (time.perf_counter() - t0) * 1e6 / steps
    same = bool(torch.equal(y, y2))
    log(f"routing ablation {cfg.name}: gpu-resident {out['gpu_resident']:.1f} us, host-synchronised "
        f"{out['host_synchronised']:.1f} us per layer; outputs equal {same}")
    return {"workload": f"moe_layer_prefill_{cfg.name}", "tokens": cfg.T,
            "gpu_resident_us": round(out["gpu_resident"], 2), "host_synchronised_us": round(out["host_synchronised"], 2),
            "speedup_of_gpu_resident": round(out["host_synchronised"] / out["gpu_resident"], 3),
            "outputs_bitwise_equal": same, "timing": f"eager launches, wall clock, mean of {steps} layers"}


def bench_skewed(cfg, reps=10):
    """The skewed-routing stress layer (per-expert Zipf logit bias, T=16384):
    throughput and MFMA fraction of the whole layer (HIP graph replays), the
    two grouped GEMMs' stage times, and the expert load it produced (max/mean
    rows, empty experts, routed tiles of the block map)."""
    import torch
    import sparse_moe_softmax_amd as moe
    import synth
    d = cfg.dims
    md = moe.Dims(d.hidden, d.inter, d.n_experts, d.top_k, d.group_size, d.shared_inter)
    log(f"skewed {cfg.name}: generating weights (seed {cfg.seed})")
    lay = synth.make_layer(d, cfg.seed, zipf_bias=cfg.zipf_bias, device="cuda")
    dl = device_layer(lay, d, moe)
    x = synth.activations(cfg.T, d.hidden, cfg.seed).cuda()
    ws = moe.moe_workspace(md, cfg.T)
    y = torch.empty((cfg.T, d.hidden), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((cfg.T, d.top_k), dtype=torch.int32, device="cuda")
    moe.moe_forward(md, dl, x, y=y, ids_out=ids, workspace=ws)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.moe_forward(md, dl, x, y=y, workspace=ws)
    warm_graph(g, 8)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1000.0 / reps
    stages = time_stages(moe, md, dl, x, y, ws, reps=reps)
    counts = torch.bincount(ids.flatten().cpu().long(), minlength=d.n_experts)
    bm = moe.moe_block_m()
    tiles = int(((counts + bm - 1) // bm).sum())
    tflops = layer_flops_per_token(d) * cfg.T / (us * 1e-6) / 1e12
    log(f"skewed {cfg.name}: {us:.1f} us per layer, max/mean load {counts.max().item() / counts.float().mean().item():.1f}")
    return {"workload": f"moe_layer_prefill_{cfg.name}", "tokens": cfg.T, "us_per_layer": round(us, 2),
            "tokens_per_s": round(cfg.T / (us * 1e-6), 1), "layer_tflops": round(tflops, 2),
            "frac_of_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
            "gate_up_us": round(stages["gate_up"], 2), "down_us": round(stages["down"], 2),
            "max_over_mean_load": round(counts.max().item() / counts.float().mean().item(), 2),
            "empty_experts": int((counts == 0).sum()), "experts_above_10x_mean":
                int((counts > 10 * counts.float().mean()).sum()), "routed_tiles": tiles, "block_m": bm,
            "launch": f"whole layer as one HIP graph, mean of {reps} replays"}


def bench_small_t(cfg, Ts=(1, 2, 4, 8, 16), n_layers=8, reps=20, seeds=None):
    """Memory-bound batch sizes: one pass of T tokens over n_layers distinct
    layers per replay (a HIP graph), algorithmic bytes = the experts the tokens
    touch + shared expert + router + activations, per layer.  seeds: per-T
    activation seeds (default: the configuration's seed, step T)."""
    import numpy as np
    import torch
    import sparse_moe_softmax_amd as moe
    import synth
    d = cfg.dims
    md = moe.Dims(d.hidden, d.inter, d.n_experts, d.top_k, d.group_size, d.shared_inter)
    layers = [device_layer(synth.make_layer(d, cfg.seed, layer=l, device="cuda"), d, moe) for l in range(n_layers)]
    eb, sb = expert_bytes(d), expert_bytes(synth_dims_shared(d))
    out = []
    for T in Ts:
        x = synth.activations(T, d.hidden, seeds[T] if seeds else cfg.seed, step=0 if seeds else T).cuda()
        ws = moe.moe_workspace(md, T)
        ys = torch.empty((n_layers, T, d.hidden), dtype=torch.bfloat16, device="cuda")
        ids = torch.empty((n_layers, T, d.top_k), dtype=torch.int32, device="cuda")

        def one_pass():
            for l, dl in enumerate(layers):
                moe.moe_forward(md, dl, x, y=ys[l], ids_out=ids[l], workspace=ws)

        one_pass()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            one_pass()
        warm_graph(g, 8)
        s_ = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s_)
        for _ in range(reps):
            g.replay()
        e1.record(s_)
        torch.cuda.synchronize()
        us_layer = e0.elapsed_time(e1) * 1000.0 / reps / n_layers
        touched = [len(np.unique(ids[l].cpu().numpy())) for l in range(n_layers)]
        bytes_layer = (float(np.mean(touched)) * eb + sb + d.n_experts * d.hidden * 4 + d.hidden * 4
                       + 2 * T * d.hidden * 2)
        gbs = bytes_layer / (us_layer * 1e-6) / 1e9
        out.append({"T": T, "us_per_layer": round(us_layer, 3), "experts_touched": round(float(np.mean(touched)), 2),
                    "bytes_per_layer": int(bytes_layer), "GBs": round(gbs, 1),
                    "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
                    "path": "fused layer, one launch" if T <= 4 else "router GEMM, grouping, grouped GEMMs"})
        log(f"T={T}: {us_layer:.2f} us/layer, {out[-1]['experts_touched']} experts, {gbs:.0f} GB/s "
            f"({100 * gbs / PEAK_HBM_GBS:.1f}% of HBM)")
    return {"layers": n_layers, "launch": f"HIP graph of one pass over {n_layers} layers, {reps} replays",
            "points": out}


def bench_gqa_decode(n_layers=10, B=1, Hq=16, Hkv=2, D=256, S=32768, reps=20, seed=109):
    """Grouped-query decode attention at 32K context, one query row per head:
    a HIP graph of one call per attention layer (n_layers distinct key/value
    caches, together larger than the 256 MB Infinity Cache), replayed; packed
    (each key/value row loaded once per group) and unpacked (once per query
    head).  Algorithmic bytes per call: the K and V rows in use, q and out."""
    import torch
    import sparse_moe_softmax_amd as moe
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    draw = lambda *shape: torch.randn(*shape, generator=gen, device="cuda").to(torch.bfloat16)
    qs = [draw(B, Hq, D) for _ in range(n_layers)]
    ks = [draw(B, Hkv, S, D) for _ in range(n_layers)]
    vs = [draw(B, Hkv, S, D) for _ in range(n_layers)]
    lens = torch.full((B,), S, dtype=torch.int32, device="cuda")
    ws = torch.empty(moe.moe_gqa_decode_workspace_bytes(B, Hq, Hkv, D, S), dtype=torch.uint8, device="cuda")
    outs = torch.empty((n_layers, B, Hq, D), dtype=torch.bfloat16, device="cuda")
    us = {}
    for pack in (True, False):
        def one_pass():
            for l in range(n_layers):
                moe.moe_gqa_decode_attention(qs[l], ks[l], vs[l], lens, pack_heads=pack, out=outs[l], workspace=ws)

        one_pass()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            one_pass()
        warm_graph(g, 8)
        s_ = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s_)
        for _ in range(reps):
            g.replay()
        e1.record(s_)
        torch.cuda.synchronize()
        us[pack] = e0.elapsed_time(e1) * 1000.0 / reps / n_layers
    nbytes = 2 * B * Hkv * S * D * 2 + 2 * B * Hq * D * 2
    gbs = nbytes / (us[True] * 1e-6) / 1e9
    log(f"gqa decode S={S}: packed {us[True]:.2f} us ({gbs:.0f} GB/s), unpacked {us[False]:.2f} us")
    return {"workload": f"GQA decode attention, batch {B}, {Hq} query heads on {Hkv} key/value heads, "
                        f"head_dim {D}, context {S}",
            "layers": n_layers, "launch": f"HIP graph of one call per layer, {reps} replays",
            "us_per_call": round(us[True], 3), "bytes_per_call": nbytes, "GBs": round(gbs, 1),
            "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
            "unpacked_us_per_call": round(us[False], 3),
            "packing_speedup": round(us[False] / us[True], 3)}


GEMM_SOURCES = ("sparse_moe_softmax_amd/csrc/gemm.hip", "sparse_moe_softmax_amd/csrc/internal.hpp")
TRAFFIC_PROFILE = "profiles/gemm_gate_up_t4096_hbm_traffic.md"


def gemm_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per gate/up launch from the committed counter profile, if it
    was taken on the current GEMM source (else None)."""
    path = os.path.join(ROOT, TRAFFIC_PROFILE)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and line.startswith("- "):
            k, v = line[2:].split(":", 1)
            vals[k.strip()] = v.strip().strip("`")
    if vals.get("gemm_source_sha256_16") != gemm_source_hash():
        return None
    try:
        return int(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def profile_stage(cfg, stage, reps):
    """Run the layer once, then one stage `reps` times, then a 256 MiB device
    copy that calibrates the byte counters (profiling runs only)."""
    import torch
    import sparse_moe_softmax_amd as moe
    import synth
    d = cfg.dims
    md = moe.Dims(d.hidden, d.inter, d.n_experts, d.top_k, d.group_size, d.shared_inter)
    lay = synth.make_layer(d, cfg.seed, zipf_bias=cfg.zipf_bias, device="cuda")
    dl = device_layer(lay, d, moe)
    x = synth.activations(cfg.T, d.hidden, cfg.seed).cuda()
    ws = moe.moe_workspace(md, cfg.T)
    y = torch.empty((cfg.T, d.hidden), dtype=torch.bfloat16, device="cuda")
    moe.moe_forward(md, dl, x, y=y, workspace=ws)
    i = moe.STAGES.index(stage)
    for _ in range(reps):
        moe.moe_forward_stages(md, dl, x, y, ws, i, i)
    a = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"profiled {stage} x{reps} on {cfg.name}, then {reps} copies of 256 MiB")


def host_cpu_info() -> dict:
    """The host the oracle runs on: logical CPUs the OS reports, CPUs this
    process may run on, and what /proc/cpuinfo and lscpu say about the part."""
    import subprocess
    info = {"logical_cpus": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0))}
    try:
        with open("/proc/cpuinfo") as f:
            first = f.read().split("\n\n")[0]
        kv = dict((l.split(":", 1)[0].strip(), l.split(":", 1)[1].strip()) for l in first.splitlines() if ":" in l)
        info.update({"model_name": kv.get("model name"), "cpu_family": kv.get("cpu family"), "model": kv.get("model"),
                     "stepping": kv.get("stepping")})
    except OSError:
        pass
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        kv = dict((l.split(":", 1)[0].strip(), l.split(":", 1)[1].strip()) for l in out.splitlines() if ":" in l)
        for key, name in (("Socket(s)", "sockets"), ("Core(s) per socket", "cores_per_socket"),
                          ("Thread(s) per core", "threads_per_core"), ("CPU max MHz", "max_mhz"),
                          ("Model name", "lscpu_model_name")):
            if key in kv:
                info[name] = kv[key]
    except (OSError, subprocess.SubprocessError):
        pass
    return info


def cpu_extra_legs(threads: int, decode_steps: int = 8) -> dict:
    """Two more oracle timings: the 64-token layer on one thread, and batch-1
    decode over the 40 distinct layers for the first `decode_steps` steps on
    `threads` threads, scaled to the 256-step run (weights copied to the host
    outside the timed region)."""
    import numpy as np
    import torch
    import oracle
    import synth
    out = {}
    c1 = synth.CONFIGS["t64"]
    d = c1.dims
    od = oracle.Dims(d.hidden, d.inter, d.n_experts, d.top_k, d.group_size, d.shared_inter)

    def ow_of(lay):
        ln = synth.layer_numpy(lay)
        return oracle.LayerWeights(ln["gate_up"], ln["down"], ln["sh_gate_up"], ln["sh_down"], ln["router_w"],
                                   ln["shared_gate_w"], ln["router_bias"])
    ow = ow_of(synth.make_layer(d, c1.seed, device="cuda"))
    xb = synth.bf16_bits_numpy(synth.activations(c1.T, d.hidden, c1.seed))
    log(f"cpu baseline: oracle on the {c1.T}-token layer, one thread")
    t0 = time.perf_counter()
    oracle.layer(od, xb, ow, threads=1)
    secs = time.perf_counter() - t0
    out["single_thread_t64"] = {"value": round(c1.T / secs, 3), "unit": "tokens/s", "threads": 1,
                                "seconds": round(secs, 2), "sample": f"all {c1.T} tokens of the 64-token layer"}
    del ow
    c4 = synth.CONFIGS["decode"]
    xs = [synth.bf16_bits_numpy(synth.activations(1, d.hidden, c4.seed, step=s)) for s in range(decode_steps)]
    log(f"cpu baseline: oracle decode, {decode_steps} steps x {c4.layers} layers, {threads} threads")
    secs = 0.0
    for l in range(c4.layers):
        owl = ow_of(synth.make_layer(d, c4.seed, layer=l, device="cuda"))
        t0 = time.perf_counter()
        for s in range(decode_steps):
            oracle.layer(od, xs[s], owl, threads=threads)
        secs += time.perf_counter() - t0
        del owl
        torch.cuda.empty_cache()
    per_step = secs / decode_steps
    out["decode_40_layers"] = {"us_per_step": round(per_step * 1e6, 1),
                               "tokens_per_s": round(1.0 / per_step, 4), "threads": threads,
                               "sample": f"the first {decode_steps} of 256 steps x {c4.layers} layers, "
                                         f"scaled x{256 // decode_steps} to the 256-step run "
                                         f"({secs * 256 / decode_steps:.1f} s)",
                               "seconds_measured": round(secs, 2)}
    return out


def cpu_baseline(res, sample, threads, min_secs=10.0, max_passes=8):
    """The oracle, as it stands, on `sample` tokens of the same workload; also
    cross-checks those tokens' GPU outputs (shared-logits protocol)."""
    import numpy as np
    import oracle
    import synth
    cfg, lay = res["cfg"], res["lay"]
    d = cfg.dims
    od = oracle.Dims(d.hidden, d.inter, d.n_experts, d.top_k, d.group_size, d.shared_inter)
    ln = synth.layer_numpy(lay)
    ow = oracle.LayerWeights(ln["gate_up"], ln["down"], ln["sh_gate_up"], ln["sh_down"], ln["router_w"],
                             ln["shared_gate_w"], ln["router_bias"])
    rng = np.random.default_rng(cfg.seed)
    sample = min(sample, cfg.T)
    tok = np.sort(rng.choice(cfg.T, sample, replace=False)).astype(np.int32)
    xb = synth.bf16_bits_numpy(res["x_cpu"])[tok]
    log(f"cpu baseline: oracle on {sample} of {cfg.T} tokens, {threads} threads, repeated to >= {min_secs} s")
    passes = 0
    t0 = time.perf_counter()
    while True:
        r = oracle.layer(od, xb, ow, threads=threads)
        passes += 1
        if time.perf_counter() - t0 >= min_secs or passes >= max_passes:
            break
    secs = time.perf_counter() - t0
    # cross-check against the GPU: logits, ids given the GPU logits, and the outputs
    g_logits = res["logits"].cpu().numpy()[tok]
    g_ids = res["ids"].cpu().numpy()[tok]
    logit_err = float(np.abs(g_logits - r["logits"]).max())
    o_ids, o_w = oracle.topk(g_logits, d.top_k)
    ids_equal = bool(np.array_equal(o_ids, g_ids))
    out, _, _, _ = oracle.moe_tokens(od, xb, o_ids, o_w, oracle.sigmoid(r["s"]), ow, threads=threads)
    gy = res["y"].cpu().view(__import__("torch").int16).numpy().view(np.uint16)[tok]
    g = oracle.bf16_to_double(gy)
    o = oracle.bf16_to_double(out)
    max_rel = float(np.abs(g - o).max() / np.abs(o).max())
    l1_rel = float(np.abs(g - o).sum() / np.abs(o).sum())
    log(f"cpu baseline: {secs:.2f} s; parity max_rel {max_rel:.2e} l1_rel {l1_rel:.2e} ids_equal {ids_equal}")
    host = host_cpu_info()
    return ({"value": round(passes * sample / secs, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
             "cores_note": "threads the oracle ran on: the host's CPU share for one GPU (at most 16), "
                           "not its core count (see host)",
             "host": host, "cpu_model": host.get("model_name"),
             "sample": f"{sample} of the {cfg.T} tokens of the same layer (router, top-k, experts incl. "
                       f"dequantisation of the experts they touch, combine), {passes} pass(es), {secs:.1f} s"},
            {"tokens": sample, "logit_max_abs_err": logit_err, "ids_equal_given_gpu_logits": ids_equal,
             "max_rel": max_rel, "l1_rel": l1_rel, "pass": bool(logit_err <= 1e-4 and ids_equal and
                                                                   max_rel <= 1e-2 and l1_rel <= 2e-3)})


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="t4096", choices=["t64", "t512", "t4096", "skew16k"])
    ap.add_argument("--decode-steps", type=int, default=256)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the routing ablation and the small-T sweep")
    ap.add_argument("--cpu-sample", type=int, default=4096)
    ap.add_argument("--cpu-threads", type=int, default=0)
    ap.add_argument("--cpu-decode-steps", type=int, default=8,
                    help="decode steps the oracle's 40-layer decode timing covers (scaled to 256)")
    ap.add_argument("--profile-stage", default=None,
                    help="profiling run: one stage repeated, no JSON line (gqa_decode: the attention leg alone; "
                         "decode: the 40-layer decode leg alone; small_t: the 8- and 16-token layers alone)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py times the MoE layer on one GPU; --gpus {args.gpus} (world size {world}) is not "
              f"supported: the layer is timed on a single MI355X", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    cfg = synth.CONFIGS[args.workload]
    d = cfg.dims
    if args.profile_stage == "gqa_decode":
        print(json.dumps({"gqa_decode_attention": bench_gqa_decode(reps=args.steps)}), flush=True)
        a = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")   # counter calibration, as profile_stage
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        return
    if args.profile_stage == "decode":
        # the 40-layer decode leg alone (args.steps steps), then the counter-calibration copies
        print(json.dumps({"decode": bench_decode(synth.CONFIGS["decode"], args.steps, graph_chunk=8)}), flush=True)
        a = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        return
    if args.profile_stage == "small_t":
        # the 8- and 16-token points of the small-batch sweep alone (args.steps graph replays each)
        print(json.dumps({"small_t": bench_small_t(synth.CONFIGS["decode"], Ts=(8, 16), reps=args.steps)}), flush=True)
        return
    if args.profile_stage:
        profile_stage(cfg, args.profile_stage, args.steps)
        return
    res = bench_prefill(cfg, args.steps, args.warmup)
    T = cfg.T
    tok_s = T / (res["wall_ms"] / 1000.0)
    layer_tflops = layer_flops_per_token(d) * T / (res["gpu_ms"] / 1000.0) / 1e12
    gu_us = res["stages"]["gate_up"]
    gu_tflops = gate_up_flops(d, T) / (gu_us * 1e-6) / 1e12
    out = {
        "metric": "MoE-layer prefill tokens/s at T=4096 + % bf16 MFMA peak; decode HBM GB/s",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["wall_ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded: x~N(0,1) bf16, router N(0,1/H) fp32, int4 codes uniform, fp16 scales "
                "U(.005,.02), bias=-8*scale)",
        "config": {"workload": f"moe_layer_prefill_{cfg.name}", "tokens": T, "hidden": d.hidden,
                   "expert_inter": d.inter, "experts": d.n_experts, "top_k": d.top_k, "shared_experts": 1,
                   "shared_inter": d.shared_inter, "quant": "int4 affine, group 64, fp16 scale+bias",
                   "skewed_routing": cfg.zipf_bias, "seed": cfg.seed},
        "layer_mfma": {"flops_per_token": layer_flops_per_token(d), "achieved_tflops": round(layer_tflops, 2),
                       "frac_of_bf16_peak": round(layer_tflops / PEAK_BF16_TFLOPS, 4),
                       "gpu_ms_per_step": round(res["gpu_ms"], 5),
                       "launch": "whole layer as one HIP graph, replayed",
                       "eager_ms_per_step": round(res["eager_ms"], 5),
                       "us_per_replay_percentiles": res["pct_us"]},
        "stages_us": {k: round(v, 2) for k, v in res["stages"].items()},
        "roofline": {"bound": "mfma", "achieved": round(gu_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(gu_tflops / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic(),
                     "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                     "kernel": "k_gemm_q4<0> (gate/up grouped GEMM, SwiGLU epilogue, + shared expert)",
                     "flops_per_launch": gate_up_flops(d, T), "us_per_launch": round(gu_us, 2)},
    }
    if not args.no_decode:
        out["decode"] = bench_decode(synth.CONFIGS["decode"], args.decode_steps)
    if not args.no_extras:
        out["routing_ablation"] = bench_routing_ablation(synth.CONFIGS["t512"], max(20, args.steps), args.warmup)
        out["small_t"] = bench_small_t(synth.CONFIGS["decode"])
        # the memory-bound prefill sizes (64 and 512 tokens, one layer each in
        # its own configuration) on the same footing: algorithmic bytes / time
        mid = {c.T: c.seed for c in (synth.CONFIGS["t64"], synth.CONFIGS["t512"])}
        out["hbm_bound_prefill"] = bench_small_t(synth.CONFIGS["t512"], Ts=tuple(sorted(mid)), seeds=mid)
        if cfg.name != "skew16k":
            out["skewed_routing"] = bench_skewed(synth.CONFIGS["skew16k"])
        out["gqa_decode_attention"] = bench_gqa_decode()
    if not args.no_cpu_baseline:
        threads = args.cpu_threads or min(16, len(os.sched_getaffinity(0)) or 1)
        out["cpu_baseline"], out["parity_sample"] = cpu_baseline(res, args.cpu_sample, threads)
        if not args.no_extras:
            out["cpu_baseline"].update(cpu_extra_legs(threads, args.cpu_decode_steps))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
