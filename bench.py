#!/usr/bin/env python3
"""Benchmark of one decode step of fused masked multi-head attention over a
KV cache on one MI355X.

A step is one pass of the whole path (bias add, append, q.K, softmax, P.V,
and the combine when the sequence is split) over one batch: one layer's
ftm_decode_mha call, or all layers back-to-back for the 32-layer sizing
workload.  Inputs are seeded synthetic tensors already resident in HBM; the
layer caches rotate so that the working set exceeds the 256 MB last-level
cache.  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--config NAME] [--graph]

With no --config the line's value is the 7b workload (the configuration the
metric is quoted on), and the tiny, sizing32, gqa and int8 workloads are
reported beside it under "configs", each with its own roofline and CPU
baseline.

--graph records the calls into HIP graphs (ftm_graph_*), each holding at
least 32 layer calls (one 32-layer step, or 32 one-layer steps), and times
graph replays instead of one library call per layer.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from decode_step_attention_amd import workloads as W  # noqa: E402

METRIC = "decode-MHA KV read GB/s (% of HBM peak) + attention tokens/s at batch×ctx"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
CSRC = os.path.join(ROOT, "decode_step_attention_amd", "csrc")


# The sources each kernel is built and launched from: a counter summary
# stays valid while none of them changes.
SHARED_SOURCES = ("gfx950.hpp", "ftm_internal.hpp", "ftm_api.cpp")
KERNEL_SOURCES = {
    "attention_kernel": ("decode_attention.hip",),
    "gqa_kernel": ("decode_attention.hip",),
    "qkv_proj_kernel": ("qkv_proj.hip",),
    "qkv_split_kernel": ("qkv_proj.hip",),
    "prefill_attn_kernel": ("prefill.hip",),
}


def kernel_source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for f in sorted(KERNEL_SOURCES[kernel] + SHARED_SOURCES):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def dominant_kernel(case: W.Case) -> str:
    """The kernel that streams the cache for this workload: grouped heads
    (3 or more per KV head) over fp16/bf16 caches run on the matrix cores
    (batch up to 256), everything else on the vector-ALU pass."""
    if (case.kv_dtype in ("f16", "bf16") and case.group >= 3 and case.batch <= 256
            and os.environ.get("FTM_GQA_VALU") != "1"):
        return "gqa_kernel"
    return "attention_kernel"


def read_traffic(kernel: str, config: str):
    """HBM bytes per launch of the dominant kernel from the committed
    rocprofv3 counter summary, if it was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{config}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_hash") != kernel_source_hash(kernel):
        return None
    return t


def describe(case: W.Case) -> str:
    lens = (f"L in U[{case.lens[0]}, {case.lens[1]}]" if case.lens else f"ctx {case.ctx}")
    grp = f"{case.n_heads}q/{case.n_kv_heads}kv heads" if case.group > 1 else f"{case.n_heads} heads"
    return (f"{case.name}: batch {case.batch}, {grp} x {case.head_dim}, {case.kv_dtype} cache, {lens}"
            + (f", {case.layers} layers" if case.layers > 1 else ""))


# Threads the oracle may use: the host CPUs this process may run on, capped
# at the 16-CPU share one GPU of the box is given.
CPU_SHARE = 16


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(case, inputs, lens, budget_s: float, threads: int = 0):
    """The CPU oracle, as it stands, on the host cores: a bounded sample of the
    same workload (whole sequences of layer 0), timed like the GPU step.
    threads 0: every CPU of the affinity mask up to the 16-CPU share."""
    import oracle
    affinity = len(os.sched_getaffinity(0))
    ncores = threads if threads > 0 else min(affinity, CPU_SHARE)
    inp = inputs[0]
    act, kvd = case.act_dtype, case.kv_dtype
    per_seq = case.n_kv_heads * 2 * case.max_seq_len * case.head_dim * W.ELEM_BYTES[kvd]
    nb = int(max(1, min(case.batch, (512 << 20) // per_seq)))
    paged = case.page_size > 0

    def host(t, dt):
        t = t.detach().contiguous().cpu()
        return t.view(torch.int16).numpy().view(np.uint16).copy() if dt == "bf16" else t.numpy().copy()

    H, Hkv, D = case.n_heads, case.n_kv_heads, case.head_dim
    q = host(inp["q"][:nb], act)
    kn = host(inp["k_new"][:nb], act)
    vn = host(inp["v_new"][:nb], act)
    bias = host(inp["bias"], act)
    if paged:
        kc0 = host(inp["k_pages"], kvd)
        vc0 = host(inp["v_pages"], kvd)
        table = host(inp["block_table"][:nb], "i32")
        sc0 = host(inp["kv_scales"], "f32") if kvd == "i8" else None
    else:
        kc0 = host(inp["k_cache"][:nb], kvd)
        vc0 = host(inp["v_cache"][:nb], kvd)
        sc0 = host(inp["kv_scales"][:, :nb], "f32") if kvd == "i8" else None
    sl = np.ascontiguousarray(lens[:nb].astype(np.int32))
    step = int(sl.max())
    sample_bytes = int(W.kv_bytes(case.with_(batch=nb), sl.tolist()))
    runs, total = 0, 0.0
    best = float("inf")
    while runs < 3 or (total < budget_s and runs < 1000):
        kc, vc = kc0.copy(), vc0.copy()
        sc = sc0.copy() if sc0 is not None else None
        t0 = time.perf_counter()
        if paged:
            oracle.decode_mha_paged(q, kn, vn, bias, kc, vc, table, sl, step, H, Hkv, D, kvd, sc,
                                    n_threads=ncores)
        else:
            oracle.decode_mha(q, kn, vn, bias, kc, vc, sl, step, H, Hkv, D, kvd, sc, n_threads=ncores)
        dt = time.perf_counter() - t0
        best = min(best, dt)
        total += dt
        runs += 1
    return {"value": sample_bytes / best / 1e9, "unit": "GB/s", "cores": ncores, "kind": "oracle",
            "tokens_per_s": nb / best, "affinity_cpus": affinity, "cpu_model": cpu_model(),
            "sample": f"layer 0, sequences 0..{nb - 1} of {case.batch} ({sample_bytes / 2**20:.3g} MiB "
                      f"of K/V), fp64 oracle on {ncores} threads, best of {runs} runs, {total:.1f} s in total"}


def device_copy_gbs(dev) -> float:
    """A plain device copy of known size (1 GiB, above the last-level cache):
    reference bandwidth, and the calibration dispatch for the HBM counters."""
    n_copy = 1 << 30
    src = torch.empty(n_copy, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    dst.copy_(src)
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbs = 2 * n_copy * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    return gbs


def run_projection(args, case):
    """The fused QKV projection alone, weights rotating over distinct sets:
    bound by the HBM stream of the weights."""
    from decode_step_attention_amd import ftm
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(dev) if args.graph else torch.cuda.current_stream(dev)
    print(f"# {case.name}: batch {case.batch}, hidden {case.hidden} -> {case.n_heads}q/{case.n_kv_heads}kv "
          f"heads x {case.head_dim}, {case.dtype}; {case.rotate} weight sets", file=sys.stderr, flush=True)
    sets = [W.make_proj_inputs(case, dev, layer=i) for i in range(case.rotate)]
    dt = W.TORCH_DTYPES[case.dtype]
    q = torch.empty((case.batch, case.n_heads, case.head_dim), dtype=dt, device=dev)
    k = torch.empty((case.batch, case.n_kv_heads, case.head_dim), dtype=dt, device=dev)
    v = torch.empty_like(k)
    calls = [ftm.ftm_qkv_proj_prepared(st["x"], st["w"], st["bias"], q, k, v, stream=stream.cuda_stream)
             for st in sets]
    nbytes = W.proj_bytes(case)
    copy_gbs = device_copy_gbs(dev)
    for i in range(args.warmup):
        calls[i % len(calls)]()
    torch.cuda.synchronize()
    graphs = []
    if args.graph:
        for c in calls:
            ftm.ftm_graph_begin(stream.cuda_stream)
            try:
                c()
            finally:
                graphs.append(ftm.ftm_graph_end(stream.cuda_stream))
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    r0.record(stream)
    for i in range(args.steps):
        if graphs:
            ftm.ftm_graph_launch(graphs[i % len(graphs)], stream.cuda_stream)
        else:
            calls[i % len(calls)]()
    r1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for g in graphs:
        ftm.ftm_graph_destroy(g)
    gpu_ms = r0.elapsed_time(r1)
    elapsed = t1 - t0
    avg_us = gpu_ms * 1e3 / args.steps
    achieved = nbytes / (avg_us * 1e-6) / 1e9
    traffic = read_traffic("qkv_proj_kernel", case.name)
    result = {
        "metric": "fused QKV projection GB/s (weights + x + outputs, % of HBM peak)",
        "value": round(nbytes * args.steps / elapsed / 1e9, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(elapsed * 1e3 / args.steps, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": case.dtype,
        "data": "synthetic (seeded, resident in HBM)",
        "config": {"workload": f"{case.name}: x [{case.batch}, {case.hidden}] times W "
                               f"[{case.n_out}, {case.hidden}] -> q/k_new/v_new",
                   "batch": case.batch, "hidden": case.hidden, "n_heads": case.n_heads,
                   "n_kv_heads": case.n_kv_heads, "head_dim": case.head_dim, "weight_sets_rotated": case.rotate,
                   "launch": "HIP graph replay" if graphs else "one library call"},
        "pct_hbm_peak": round(100 * nbytes * args.steps / elapsed / 1e9 / HBM_PEAK_GBS, 2),
        "bytes_per_step": nbytes, "gpu_ms_per_step": round(gpu_ms / args.steps, 5),
        "device_copy_GBs": round(copy_gbs, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic["hbm_bytes_per_launch"] if traffic else None,
                     "kernel": "qkv_proj_kernel", "avg_launch_us": round(avg_us, 2),
                     "timing": "events bracketing the timed region / launches",
                     "algorithmic_bytes_per_launch": nbytes,
                     "flops_per_launch": 2 * case.batch * case.n_out * case.hidden},
    }
    if args.cpu_budget > 0:
        import oracle
        host = {kk: vv.cpu() for kk, vv in sets[0].items()}
        hn = {kk: (vv.view(torch.int16).numpy().view(np.uint16) if case.dtype == "bf16" else vv.numpy())
              for kk, vv in host.items()}
        runs, total, best = 0, 0.0, float("inf")
        while runs < 3 or (total < args.cpu_budget and runs < 50):
            c0 = time.perf_counter()
            oracle.qkv_proj(hn["x"], hn["w"], hn["bias"], case.n_heads, case.n_kv_heads, case.head_dim,
                            case.dtype)
            dtm = time.perf_counter() - c0
            best, total, runs = min(best, dtm), total + dtm, runs + 1
        result["cpu_baseline"] = {"value": round(nbytes / best / 1e9, 3), "unit": "GB/s",
                                  "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
                                  "sample": f"the whole projection (weight set 0), float64 numpy, best of {runs} runs"}
    print(json.dumps(result), flush=True)


MFMA_PEAK_TFLOPS = 2500.0    # MI355X dense fp16/bf16 matrix peak, published


def run_prefill(args, case):
    """Prefill of the whole prompts: compute-bound on the matrix cores."""
    from decode_step_attention_amd import ftm
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    print(f"# {case.name}: batch {case.batch} x {case.prompt}-token prompts, {case.n_heads}q/{case.n_kv_heads}kv "
          f"heads x {case.head_dim}, {case.dtype}", file=sys.stderr, flush=True)
    inp = W.make_prefill_inputs(case, dev, poison=False)
    i8 = case.dtype == "i8"                 # INT8 cache: fp16 activations, int8 codes + fp32 row scales
    out = torch.empty((case.batch, case.prompt, case.n_heads, case.head_dim),
                      dtype=W.TORCH_DTYPES["f16" if i8 else case.dtype], device=dev)
    if case.page_size:
        inp = W.prefill_to_paged(inp, case, case.page_size)
        call = ftm.ftm_prefill_mha_paged_prepared(inp["q"], inp["k_new"], inp["v_new"], inp["bias"], inp["k_pages"],
                                                  inp["v_pages"], inp["block_table"], inp["seq_lens"], out,
                                                  stream=stream.cuda_stream, kv_scales=inp.get("kv_scales"))
    else:
        call = ftm.ftm_prefill_mha_prepared(inp["q"], inp["k_new"], inp["v_new"], inp["bias"], inp["k_cache"],
                                            inp["v_cache"], inp["seq_lens"], out, stream=stream.cuda_stream,
                                            kv_scales=inp.get("kv_scales"))
    lens = inp["seq_lens"].cpu().tolist()
    flops = W.prefill_flops(case, lens)
    copy_gbs = device_copy_gbs(dev)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    r0.record(stream)
    for _ in range(args.steps):
        call()
    r1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    gpu_ms = r0.elapsed_time(r1) / args.steps
    elapsed = t1 - t0
    # timed region 2: the same steps with a HIP event pair recorded around
    # each of the two kernels, on the launch stream (kind 0: the attention,
    # kind 1: the append)
    ftm.ftm_timing_enable(args.steps + 8)
    torch.cuda.synchronize()
    for _ in range(args.steps):
        call()
    torch.cuda.synchronize()
    n_att, ms_att = ftm.ftm_timing_read(0)
    n_app, ms_app = ftm.ftm_timing_read(1)
    ftm.ftm_timing_disable()
    att_us = ms_att * 1e3 / max(n_att, 1)
    app_us = ms_app * 1e3 / max(n_app, 1)
    tflops = flops / (att_us * 1e-6) / 1e12
    traffic = read_traffic("prefill_attn_kernel", case.name)
    result = {
        "metric": "prefill attention TFLOP/s (causal q.k + p.v, % of the dense fp16/bf16 matrix peak)",
        "value": round(flops * args.steps / elapsed / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(elapsed * 1e3 / args.steps, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16" if i8 else case.dtype,
        "data": "synthetic (seeded, resident in HBM)",
        "config": {"workload": f"{case.name}: batch {case.batch} x {case.prompt} tokens, {case.n_heads}q/"
                               f"{case.n_kv_heads}kv heads x {case.head_dim}",
                   "batch": case.batch, "prompt": case.prompt, "n_heads": case.n_heads,
                   "n_kv_heads": case.n_kv_heads, "head_dim": case.head_dim,
                   "cache_layout": f"paged, {case.page_size}-token pages" if case.page_size else "contiguous",
                   "cache_dtype": case.dtype},
        "tokens_per_s": round(sum(lens) * args.steps / elapsed, 1),
        "gpu_ms_per_step": round(gpu_ms, 5), "flops_per_step": flops, "kernels_per_step": 2,
        "device_copy_GBs": round(copy_gbs, 1),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / MFMA_PEAK_TFLOPS, 4),
                     "traffic": traffic["hbm_bytes_per_launch"] if traffic else None,
                     "kernel": "prefill_attn_kernel", "avg_launch_us": round(att_us, 2),
                     "timing": "event pair around every attention launch in timed region 2",
                     "launches": n_att, "flops_per_launch": flops,
                     "append_kernel_avg_us": round(app_us, 2),
                     "append_bytes_per_launch": W.prefill_append_bytes(case, lens)},
    }
    if args.cpu_budget > 0:
        import oracle
        hc = {k: (v.cpu().view(torch.int16).numpy().view(np.uint16) if case.dtype == "bf16" else v.cpu().numpy())
              for k, v in inp.items() if k not in ("seq_lens", "block_table")}
        # one sequence, the first head group only: a bounded sample
        G = case.n_heads // case.n_kv_heads
        D = case.head_dim
        qh = np.ascontiguousarray(hc["q"][:1, :, :G])
        kn = np.ascontiguousarray(hc["k_new"][:1, :, :1])
        vn = np.ascontiguousarray(hc["v_new"][:1, :, :1])
        H, Hkv = case.n_heads, case.n_kv_heads
        bb = hc["bias"]
        sb = np.concatenate([bb[:G * D], bb[H * D:(H + 1) * D], bb[(H + Hkv) * D:(H + Hkv + 1) * D]])
        runs, total, best = 0, 0.0, float("inf")
        while runs < 2 or (total < args.cpu_budget and runs < 20):
            kc = np.zeros((1, 1, case.max_seq_len, D), dtype=np.int8 if i8 else qh.dtype)
            vc = kc.copy()
            sc = np.zeros((2, 1, 1, case.max_seq_len), dtype=np.float32) if i8 else None
            c0 = time.perf_counter()
            oracle.prefill_mha(qh, kn, vn, sb, kc, vc, None, G, 1, D, case.dtype, sc)
            dtm = time.perf_counter() - c0
            best, total, runs = min(best, dtm), total + dtm, runs + 1
        sample_flops = W.prefill_flops(case.with_(batch=1, n_heads=G, n_kv_heads=1))
        result["cpu_baseline"] = {"value": round(sample_flops / best / 1e12, 4), "unit": "TFLOP/s",
                                  "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
                                  "sample": f"sequence 0, query heads 0..{G - 1} (one KV head), float64 numpy, "
                                            f"best of {runs} runs"}
    print(json.dumps(result), flush=True)


def run_decode(args, case: W.Case, cpu_budget: float) -> dict:
    """One decode workload: the whole path timed over args.steps steps after
    args.warmup untimed ones, with its roofline and the CPU oracle beside it."""
    from decode_step_attention_amd import ftm

    dev = torch.device("cuda:0")
    layers = case.layers
    rotate = max(case.rotate, layers)
    lens = W.seq_lens(case)
    print(f"# {describe(case)}; {rotate} cache sets; generating inputs", file=sys.stderr, flush=True)
    make = W.make_paged_inputs if case.page_size else W.make_inputs
    inputs = [make(case, dev, layer=i, poison=False, lens=lens) for i in range(rotate)]
    outs = [torch.empty((case.batch, case.n_heads, case.head_dim),
                        dtype=W.TORCH_DTYPES[case.act_dtype], device=dev) for _ in range(2)]
    step = int(lens.max())
    lens_np = lens.numpy()
    kv_layer = W.kv_bytes(case, lens_np.tolist())
    kv_step = kv_layer * layers
    # graph capture needs a created stream (the null stream cannot be captured)
    stream = torch.cuda.Stream(dev) if args.graph else torch.cuda.current_stream(dev)

    # one prepared call per (cache set, output buffer): the per-step host work
    # is a single C call, so the GPU is never waiting on Python
    def prepare(inp, out):
        if case.page_size:
            return ftm.ftm_decode_mha_paged_prepared(inp["q"], inp["k_new"], inp["v_new"], inp["bias"],
                                                     inp["k_pages"], inp["v_pages"], inp["block_table"],
                                                     inp["seq_lens"], step, out, inp.get("kv_scales"),
                                                     stream=stream.cuda_stream)
        return ftm.ftm_decode_mha_prepared(inp["q"], inp["k_new"], inp["v_new"], inp["bias"],
                                           inp["k_cache"], inp["v_cache"], inp["seq_lens"], step,
                                           out, inp.get("kv_scales"), stream=stream.cuda_stream)

    calls = [[prepare(inp, outs[o]) for o in range(2)] for inp in inputs]

    def call(i):
        calls[i % rotate][i & 1]()

    copy_gbs = device_copy_gbs(dev)

    k = 0
    for _ in range(args.warmup):
        for _l in range(layers):
            call(k)
            k += 1
    torch.cuda.synchronize()

    # kernels one step launches (the attention pass, plus the combine when
    # the sequences are split)
    ftm.ftm_timing_enable(layers + 8)
    for _l in range(layers):
        call(k)
        k += 1
    torch.cuda.synchronize()
    kernels_per_step = ftm.ftm_timing_read(0)[0] + ftm.ftm_timing_read(1)[0]
    ftm.ftm_timing_disable()

    # graph mode: one graph holds at least --graph-calls layer calls (by
    # default GRAPH_CALLS: a whole decode step of a 32-layer model, or 32
    # consecutive steps of a one-layer workload), so that its launch is
    # amortised over that much work; the timed steps are rounded up to
    # whole graphs
    spg = max(1, args.graph_calls // layers) if args.graph else 1     # steps per graph
    steps = -(-args.steps // spg) * spg
    graphs = []
    if args.graph:
        # captured after the warm-up has sized the stream's workspace; calls
        # cycle over the cache sets and the two output buffers as eager
        # steps do
        n_graphs = max(1, rotate // (spg * layers))
        for gi in range(n_graphs):
            ftm.ftm_graph_begin(stream.cuda_stream)
            try:
                for c in range(spg * layers):
                    kk = gi * spg * layers + c
                    calls[kk % rotate][kk & 1]()
            finally:
                graphs.append(ftm.ftm_graph_end(stream.cuda_stream))
        for gi in range(min(args.warmup, len(graphs) * 4)):
            ftm.ftm_graph_launch(graphs[gi % len(graphs)], stream.cuda_stream)
        torch.cuda.synchronize()

    def run_unit(i):
        """Unit i of the timed loops: one graph (spg steps) or one step."""
        nonlocal k
        if graphs:
            ftm.ftm_graph_launch(graphs[i % len(graphs)], stream.cuda_stream)
            return
        for _l in range(layers):
            call(k)
            k += 1

    units = steps // spg
    # timed region 1: the whole path, nothing else on the stream; a HIP event
    # pair on the launch stream brackets the region
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    r0.record(stream)
    for i in range(units):
        run_unit(i)
    r1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    region_gpu_ms = r0.elapsed_time(r1)
    n_att = n_cmb = 0
    ms_att = ms_cmb = 0.0
    t2 = t3 = 0.0
    if not graphs:
        # timed region 2: the same steps with a HIP event pair recorded around
        # every kernel launch, on the launch stream, for per-kernel durations
        ftm.ftm_timing_enable(steps * layers + 8)
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        for i in range(units):
            run_unit(i)
        torch.cuda.synchronize()
        t3 = time.perf_counter()
        n_att, ms_att = ftm.ftm_timing_read(0)
        n_cmb, ms_cmb = ftm.ftm_timing_read(1)
        ftm.ftm_timing_disable()
    # timed region 3: an event pair around every step (graph mode: every
    # graph, divided by its steps), for the distribution of step times (each
    # pair adds its own dispatch and release, a few us)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(units)]
    torch.cuda.synchronize()
    for i in range(units):
        ev[i][0].record(stream)
        run_unit(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    step_us = np.sort(np.array([a.elapsed_time(b) * 1e3 / spg for a, b in ev]))
    for g in graphs:
        ftm.ftm_graph_destroy(g)
    elapsed = t1 - t0
    ms_step = elapsed * 1e3 / steps
    gbs = kv_step * steps / elapsed / 1e9
    per_launch_us = ms_att * 1e3 / max(n_att, 1)
    if n_cmb == 0:
        # one kernel per step: its average duration is the event-bracketed
        # region time over the launches (an event pair around every launch
        # adds its own dispatch and release time, a few us)
        avg_att_us = region_gpu_ms * 1e3 / (steps * layers)
        timing = ("events bracketing timed region 1 (graph replays) / layer launches" if graphs
                  else "events bracketing timed region 1 / launches (one kernel per step)")
    else:
        avg_att_us = per_launch_us
        timing = "event pair around every attention launch in timed region 2"
    achieved = kv_layer / (avg_att_us * 1e-6) / 1e9
    kernel = dominant_kernel(case)
    traffic = read_traffic(kernel, case.name)
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic["hbm_bytes_per_launch"] if traffic else None,
            "kernel": kernel, "avg_launch_us": round(avg_att_us, 2),
            "avg_launch_us_per_launch_events": round(per_launch_us, 2), "timing": timing,
            "launches": n_att if n_att else steps * layers,
            "algorithmic_bytes_per_launch": kv_layer}
    result = {
        "metric": METRIC, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": case.kv_dtype, "data": "synthetic (seeded, resident in HBM)",
        "config": {"workload": describe(case), "batch": case.batch, "n_heads": case.n_heads,
                   "n_kv_heads": case.n_kv_heads, "head_dim": case.head_dim,
                   "context": step, "kv_dtype": case.kv_dtype, "act_dtype": case.act_dtype,
                   "layers_per_step": layers, "cache_sets_rotated": rotate,
                   "cache_layout": f"paged, {case.page_size}-token pages" if case.page_size else "contiguous",
                   "launch": (f"HIP graph replay, {spg * layers} layer calls ({spg} steps) per graph" if graphs
                              else "one library call per layer")},
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(case.batch * steps / elapsed, 1),
        "kv_bytes_per_step": kv_step,
        "ms_per_step_with_kernel_events": round((t3 - t2) * 1e3 / steps, 5) if not graphs else None,
        "kernels_per_step": kernels_per_step,
        "gpu_ms_per_step": round(region_gpu_ms / steps, 5),
        "combine_avg_launch_us": round(ms_cmb * 1e3 / n_cmb, 2) if n_cmb else None,
        "step_us_per_step_events": {"p50": round(float(np.percentile(step_us, 50)), 2),
                                    "p99": round(float(np.percentile(step_us, 99)), 2),
                                    "mean": round(float(step_us.mean()), 2),
                                    "note": "timed region 3: an event pair around every step, which adds "
                                            "its own dispatch and release time"},
        "device_copy_GBs": round(copy_gbs, 1),
        "roofline": roof,
    }
    if cpu_budget > 0:
        print(f"# timing the CPU oracle on {case.name}", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(case, inputs, lens_np, cpu_budget)
        if case.name in ONE_THREAD_CONFIGS:
            one = cpu_baseline(case, inputs, lens_np, 0.0, threads=1)
            result["cpu_baseline"]["one_thread"] = {"value": one["value"], "unit": "GB/s",
                                                    "tokens_per_s": one["tokens_per_s"], "sample": one["sample"]}
    del inputs, calls
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return result


# Layer calls one graph holds in graph mode.
GRAPH_CALLS = 32

# The headline workload, and the others reported beside it in the same line.
HEADLINE = "7b"
SECONDARY = ("tiny", "sizing32", "gqa", "int8")
# Workloads whose oracle is also timed on one thread.
ONE_THREAD_CONFIGS = ("tiny", "7b")
SUMMARY_KEYS = ("value", "unit", "pct_hbm_peak", "tokens_per_s", "ms_per_step", "gpu_ms_per_step", "dtype",
                "kernels_per_step", "step_us_per_step_events", "roofline", "cpu_baseline")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--config", default=None,
                    choices=sorted(W.CASES) + sorted(W.PROJ_CASES) + sorted(W.PREFILL_CASES),
                    help="one workload only (default: the 7b headline, with tiny, sizing32, gqa and int8 "
                         "reported beside it under \"configs\")")
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of oracle time for the CPU baseline of the headline (0 skips it)")
    ap.add_argument("--cpu-budget-others", type=float, default=5.0,
                    help="seconds of oracle time for each other workload's CPU baseline")
    ap.add_argument("--graph", action="store_true",
                    help="replay HIP graphs of layer calls instead of one call per layer")
    ap.add_argument("--graph-calls", type=int, default=GRAPH_CALLS,
                    help="layer calls one graph holds (rounded to whole steps; default 32)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (the attention "
              "shards by batch or KV-head group with no exchange). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.config in W.PROJ_CASES:
        run_projection(args, W.PROJ_CASES[args.config])
        return
    if args.config in W.PREFILL_CASES:
        run_prefill(args, W.PREFILL_CASES[args.config])
        return
    if args.config is not None:
        print(json.dumps(run_decode(args, W.CASES[args.config], args.cpu_budget)), flush=True)
        return
    t_start = time.perf_counter()
    result = run_decode(args, W.CASES[HEADLINE], args.cpu_budget)
    others = {}
    for name in SECONDARY:
        r = run_decode(args, W.CASES[name], args.cpu_budget_others if args.cpu_budget > 0 else 0.0)
        others[name] = {"workload": r["config"]["workload"], **{key: r[key] for key in SUMMARY_KEYS if key in r}}
    result["configs"] = others
    result["bench_wall_s"] = round(time.perf_counter() - t_start, 1)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
