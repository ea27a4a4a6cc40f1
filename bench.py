#!/usr/bin/env python3
"""Sparse MLA decode benchmark (one MI355X).

A step is one pass of the whole hot path on one batch: the tile plan, the
decode kernel and the split-KV combine, for b=64 query tokens, 128 heads,
topk=2048 slots into a paged FP8 cache of 32768 tokens per sequence.  Steps
rotate over --layers independent layers (own cache, Q and indices each) so
the gathered rows of one step are not still cached in the 256 MB Infinity
Cache when that layer comes round again.  With a per-request scheduler cost
of zero (the default here) the plan is passed as NULL and every work-group
evaluates its own partition in closed form, so a step is two launches;
--plan sched launches the scheduler kernel in every step instead.  Inputs are
resident in HBM before the timed region starts.  Before the --warmup steps,
untimed steps run for --prewarm-s seconds so the GPU clocks have ramped up
(the first milliseconds of work on an idle GPU run slower).  The kernels of a step are
launched one by one (--graph replays a captured HIP graph of each layer's step instead, which
on this stack costs more per step than the launches it saves); the decode
kernel's duration comes from HIP events around eager launches of the same
steps.

Prints one JSON line.  With --gpus N > 1 it exits: this build runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-decode query-tokens/s at b=64,h=128,topk=2048; % of MFMA/HBM roofline"
METRIC_SOA = ("sparse-decode query-tokens/s at b=64,h=128,topk=2048 on the {} cache (d_qk 512); "
              "% of MFMA/HBM roofline")
METRIC_HALFHEAD = ("sparse-decode query-tokens/s at b=128,h=64,topk=2048 (13 of 128 requests hold 1500 valid "
                   "slots); % of HBM roofline")
METRIC_PREFILL = ("sparse-prefill query-tokens/s at s_q=4096,h=128,topk=2048 over a bf16 cache of 8192 tokens; "
                  "% of MFMA roofline")
PEAK_BF16_TFLOPS = 2500.0        # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0            # MI355X HBM3E

# HBM bytes per launch of the decode kernel at this workload, from two rocprofv3
# --pmc runs of this script (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch),
# each scaled by what the same counter reads for a plain 1 GiB device copy
# (bench.py --copy-calibration 1024: FETCH_SIZE reads 524301.3 KiB -> x2.0,
# WRITE_SIZE 1048576 KiB -> x1.0).  Valid only for the kernel sources they were
# taken on (sha256 below); for any other source the traffic is reported null.
DECODE_KERNEL_SOURCES = ("sparse_mla_attention_decode_amd/csrc/decode_h128.hip",
                         "sparse_mla_attention_decode_amd/csrc/device_common.h",
                         "sparse_mla_attention_decode_amd/csrc/mla_internal.h")
DECODE_TRAFFIC = {"sources_sha256": "ec72c735b050720b7c380e04e5f809359d37947662c2598559cb0e678b54d4fd",
                  "fetch_scale": 2.0, "write_scale": 1.0,
                  # workload: (FETCH_SIZE KiB, WRITE_SIZE KiB) per decode dispatch
                  "kib": {"decode": (54055.7, 32896.0), "halfhead": (100990.4, 16448.0),
                          "v4": (51776.3, 32896.0), "v41": (44524.8, 32896.0),
                          "prefill": (2331126.8, 541269.6)}}

INDEXER_KERNEL_SOURCES = ("sparse_mla_attention_decode_amd/csrc/indexer.hip",
                          "sparse_mla_attention_decode_amd/csrc/indexer_internal.h",
                          "sparse_mla_attention_decode_amd/csrc/device_common.h")
INDEXER_TRAFFIC = {"sources_sha256": "43a82353eb4f8e99b5d4f8faf4e90e5f4c4b50b042e65242dcd76bdb3f4d4c26",
                   "fetch_kib": 137458.8, "fetch_scale": 2.0, "write_kib": 4223.3, "write_scale": 1.0}


def traffic_of(sources, t):
    """HBM bytes per launch from stored counters, if they match the sources."""
    import hashlib
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest() != t["sources_sha256"]:
        return None
    return t["fetch_kib"] * 1024 * t["fetch_scale"] + t["write_kib"] * 1024 * t["write_scale"]


def measured_traffic(workload):
    """HBM bytes per decode launch of this workload if the counters match the
    current kernel sources."""
    import hashlib
    h = hashlib.sha256()
    for f in DECODE_KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    t = DECODE_TRAFFIC
    if h.hexdigest() != t["sources_sha256"] or workload not in t["kib"]:
        return None, None
    fetch_kib, write_kib = t["kib"][workload]
    fetch = fetch_kib * 1024 * t["fetch_scale"]
    write = write_kib * 1024 * t["write_scale"]
    return fetch + write, {"fetch_bytes": fetch, "write_bytes": write,
                           "counters": "FETCH_SIZE x2.0, WRITE_SIZE x1.0 (copy-calibrated)"}


def algorithmic(w, unique_rows: bool = False):
    """Flops of the two contractions over valid slots and compulsory HBM bytes
    (gathered rows + Q + out + indices + lse) of one decode of workload w.
    unique_rows: count each cache row once however many query tokens select
    it (the sparse prefill: 4096 query tokens share an 8192-row cache, so
    repeated rows come from the caches, not from HBM)."""
    import numpy as np
    valid = (w.indices >= 0) & (w.indices < w.num_kv_tokens)
    n_valid = int(valid.sum())
    d_qk = w.q_bits.shape[-1]                       # 576; 512 for the V4 / V4.1 caches
    flops = 2.0 * w.h_q * n_valid * (d_qk + 512)
    rows = len(np.unique(w.indices[valid])) if unique_rows else n_valid
    bytes_ = (rows * w.row_bytes + w.b * w.s_q * w.h_q * d_qk * 2 + w.b * w.s_q * w.h_q * 512 * 2
              + w.indices.size * 4 + w.b * w.s_q * w.h_q * 4)
    return flops, float(bytes_), n_valid


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(w, budget_s: float):
    """The CPU oracle, as it stands, on the query tokens of layer 0 in order
    (starting over after the last) until the time budget is spent; returns
    query-tokens/s and what was run."""
    from threadpoolctl import threadpool_info
    from oracle import mla_oracle as O
    kv = w.kv_host()
    n_q = w.b * w.s_q
    done = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        bi, sj = divmod(done % n_q, w.s_q)
        O.sparse_mla_decode(w.q_bits, kv, w.indices, w.sm_scale, w.kv_format, w.page_block_size,
                            queries=[(bi, sj)])
        done += 1
    dt = time.perf_counter() - t0
    threads = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    return {"value": done / dt, "unit": "query-tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{done} query-token decodes of the same workload (layer 0's {n_q} query tokens in order, "
                      f"repeated), {dt:.1f} s, numpy float64 with {threads} BLAS threads"}


def bench_indexer(args, torch, np, M, W, dev):
    """Lightning indexer + top-k ("FlashMLA 与 DSA" sections 4.1, 5.3, 5.5) for 64
    requests of one query token at a 32768-token context (512 pages of 64), 64
    indexer heads, K = 2048: one step = the score kernel + the top-k kernel."""
    b, heads, pages, K = 64, 64, 512, 2048
    lens = np.full(b, pages * 64, dtype=np.int32)
    # steps rotate over independent layers (key cache, q, weights, page table:
    # 277 MB of keys each) so a step's keys are not still in the 256 MB
    # Infinity Cache when its layer comes round again
    n_layers = max(2, min(args.layers, 4))
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    sets = []
    for l in range(n_layers):
        q, w, kc, pt, lens = W.indexer_inputs(21 + 1000 * l, b, heads, lens, max_pages=pages)
        scores = torch.empty((b, pages * 64), dtype=torch.bfloat16, device=dev)
        idx = torch.empty((b, K), dtype=torch.int32, device=dev)
        q_d, w_d, kc_d, pt_d, len_d = d(q), d(w), d(kc), d(pt), d(lens)
        sets.append((M.indexer_args(q_d, w_d, kc_d, pt_d, len_d, K, scores, idx),
                     (q_d, w_d, kc_d, pt_d, len_d, scores, idx)))
        if l == 0:
            q0, w0_, kc0, pt0 = q, w, kc, pt
    st = torch.cuda.current_stream()
    sp = st.cuda_stream

    def step(i, ev=None):
        a = sets[i % n_layers][0]
        if ev is not None:
            ev[0].record(st)
        M.mla_indexer_scores(a, sp)
        if ev is not None:
            ev[1].record(st)
        M.mla_indexer_topk(a, sp)
        if ev is not None:
            ev[2].record(st)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i, e in enumerate(evs):
        step(i, e)
    torch.cuda.synchronize()
    score_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    topk_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    n_tok = int(lens.sum())
    # algorithmic bytes: every key row (128 codes + 4-byte scale), q, w, the page
    # table and the bf16 scores written once; top-k reads the scores once and
    # writes K ids per request
    score_bytes = n_tok * (132 + 2) + b * heads * (128 + 4) + b * pages * 4
    topk_bytes = n_tok * 2 + b * K * 4
    achieved = score_bytes / (score_ms * 1e-3) / 1e9
    res = {"metric": "indexer query-tokens/s at b=64, 32K context, K=2048 (scores + top-k)",
           "value": b / dt, "unit": "query-tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": dt * 1e3, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "fp8", "data": "synthetic",
           "config": {"workload": "indexer_b64_h64_ctx32k_k2048", "b": b, "indexer_heads": heads,
                      "context": pages * 64, "topk": K, "key_cache": "fp8 128 B + fp32 scale per token, page 64",
                      "layers_rotated": n_layers},
           "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": achieved / PEAK_HBM_GBS,
                        "traffic": traffic_of(INDEXER_KERNEL_SOURCES, INDEXER_TRAFFIC), "kernel": "indexer_score_kernel",
                        "kernel_ms": score_ms, "algorithmic_bytes_per_launch": score_bytes},
           "topk_kernel": {"kernel": "indexer_topk_kernel", "kernel_ms": topk_ms,
                           "algorithmic_bytes_per_launch": topk_bytes,
                           "achieved_GBs": topk_bytes / (topk_ms * 1e-3) / 1e9}}
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_info
        from oracle import indexer_oracle as X
        q, w, kc, pt = q0, w0_, kc0, pt0
        rows, t1 = 0, time.perf_counter()
        while rows < b and time.perf_counter() - t1 < args.cpu_budget:
            sc = X.indexer_scores(q[rows:rows + 1], w[rows:rows + 1], kc, pt[rows:rows + 1], lens[rows:rows + 1])
            X.topk_select(sc[0], int(lens[rows]), K, pt[rows], kc.shape[0])
            rows += 1
        cpu_s = time.perf_counter() - t1
        threads = max([t.get("num_threads", 1) for t in threadpool_info()] + [1])
        res["cpu_baseline"] = {"value": rows / cpu_s, "unit": "query-tokens/s", "cores": threads, "kind": "oracle",
                               "cpu_model": cpu_model(),
                               "sample": f"{rows} of {b} requests of the same workload (layer 0), {cpu_s:.1f} s, "
                                         f"numpy float64 with {threads} BLAS threads"}
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--prewarm-s", type=float, default=0.25,
                    help="untimed steps for at least this many seconds before the warm-up steps, "
                         "so the GPU clocks have ramped up (a cold GPU runs the first milliseconds "
                         "of work at lower clocks)")
    ap.add_argument("--layers", type=int, default=4)
    ap.add_argument("--split-granularity", type=int, default=32)
    ap.add_argument("--fixed-overhead", type=int, default=0)
    ap.add_argument("--plan", choices=("auto", "closed", "sched"), default="auto",
                    help="closed: NULL plan, the kernels evaluate the greedy plan in closed form "
                         "(fixed_overhead 0 only); sched: launch the scheduler kernel every step; "
                         "auto: closed when fixed_overhead is 0")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", choices=("decode", "halfhead", "indexer", "v4", "v41", "prefill"),
                    default="decode",
                    help="decode: the sparse MLA decode step at b=64, h=128, topk=2048 (default); "
                         "halfhead: b=128, h=64, topk=2048 over 65536-token contexts with 10%% of the "
                         "requests holding 1500 valid slots (HBM-bound); indexer: the lightning "
                         "indexer scores + top-k that select the decode's tokens; v4 / v41: the "
                         "decode step's shape on the V4 (584 B/token) / V4.1 (528 B/token) cache; prefill: "
                         "the sparse prefill, 4096 query tokens of one sequence selecting 2048 of an "
                         "8192-token bf16 cache each (MFMA-bound)")
    ap.add_argument("--graph", action="store_true",
                    help="replay a captured HIP graph of each layer's step instead of launching "
                         "its kernels one by one")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB five times (the reference "
                         "kernel for scaling HBM byte counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(sparse decode shards by query token with no exchange); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import sparse_mla_attention_decode_amd as M
    from sparse_mla_attention_decode_amd import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    if args.workload == "indexer":
        return bench_indexer(args, torch, np, M, W, dev)
    if args.copy_calibration > 0:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty(n, dtype=torch.uint8, device=dev)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "repeats": 5}), flush=True)
        return
    M.load_library()

    cfg = {"halfhead": 2, "prefill": 3}.get(args.workload, 1)
    kv_format = {"v4": W.KV_V4_584, "v41": W.KV_V41_528}.get(args.workload, W.KV_FP8_656)
    soa = kv_format != W.KV_FP8_656
    wl_name = W.CONFIG_NAMES[cfg] + (f"_{args.workload}kv" if soa else "")
    # the 64-head workload's cache is 5.4 GB per layer: two layers already
    # exceed the 256 MB Infinity Cache many times over
    # (the prefill: 1.2 GB of Q and out per step, far past that cache, and a
    # 9 MB cache that every step reads anyway)
    n_layers = args.layers if cfg == 1 else 1 if cfg == 3 else min(args.layers, 2)
    print(f"[bench] building {n_layers} layers of {wl_name}", file=sys.stderr, flush=True)
    layers = []
    for l in range(n_layers):
        if l == 0 and not soa:
            w = W.make_config(cfg)             # (the prefill: one layer)
        elif cfg == 1:
            w = W.paged_decode(f"{wl_name}_layer{l}", W.BASE_SEED + 1 + 1000 * l, b=64, s_q=1, h_q=128,
                               topk=2048, tokens_per_seq=32768, kv_format=kv_format)
        else:
            w = W.paged_decode(f"{W.CONFIG_NAMES[2]}_layer{l}", W.BASE_SEED + 2 + 1000 * l, b=128, s_q=1, h_q=64,
                               topk=2048, tokens_per_seq=65536, short_frac=0.1, short_len=1500)
        layers.append((w, w.q_device(dev), w.kv_device(dev), w.indices_device(dev)))
    w0 = layers[0][0]
    shape = M.make_shape(w0.b, w0.s_q, w0.h_q, w0.topk, w0.num_kv_tokens, w0.kv_format,
                         w0.page_block_size, split_granularity=args.split_granularity,
                         fixed_overhead=args.fixed_overhead)
    closed = args.plan == "closed" or (args.plan == "auto" and args.fixed_overhead == 0)
    plan = M.DecodePlan(shape, device=dev, closed_form=closed)
    argsets = [plan.args(q, kv, idx, w.sm_scale) for (w, q, kv, idx) in layers]
    stream = torch.cuda.current_stream(dev)

    def step(i, ev=None):
        a = argsets[i % len(argsets)]
        plan.get_sched_meta()
        if ev is not None:
            ev[0].record(stream)
        M.mla_sparse_decode_fwd(a)
        if ev is not None:
            ev[1].record(stream)
        M.mla_splitkv_combine(a)

    t_pre = time.perf_counter()
    n_pre = 0
    while time.perf_counter() - t_pre < args.prewarm_s:
        for i in range(20):
            step(n_pre + i)
        n_pre += 20
        torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # With --graph, one HIP graph per layer holding that layer's whole step
    # (plan, decode, combine), replayed.  The library calls only launch
    # kernels on the current stream (no allocation, no memset), which is what
    # capture needs.
    graphs = []
    if args.graph:
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for i in range(len(argsets)):
                step(i)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        for i in range(len(argsets)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(i)
            graphs.append(g)
        for i in range(args.warmup):
            graphs[i % len(graphs)].replay()
        torch.cuda.synchronize()

    # ---- timed region: exactly `steps` steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if graphs:
        for i in range(args.steps):
            graphs[i % len(graphs)].replay()
    else:
        for i in range(args.steps):
            step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    # ---- decode kernel duration: HIP events on the launch stream around each
    # decode of `steps` eager steps (the same work, launched one by one)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    decode_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))

    flops, bytes_, n_valid = algorithmic(w0, unique_rows=cfg == 3)
    traffic, traffic_detail = measured_traffic(args.workload)
    achieved_tflops = flops / (decode_ms * 1e-3) / 1e12
    achieved_gbs = bytes_ / (decode_ms * 1e-3) / 1e9
    t_roof_ms = max(flops / (PEAK_BF16_TFLOPS * 1e12), bytes_ / (PEAK_HBM_GBS * 1e9)) * 1e3
    mfma_bound = flops / (PEAK_BF16_TFLOPS * 1e12) >= bytes_ / (PEAK_HBM_GBS * 1e9)
    q_tokens = w0.b * w0.s_q
    value = q_tokens / (ms_per_step * 1e-3)
    if mfma_bound:
        roof = {"bound": "mfma", "achieved": achieved_tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved_tflops / PEAK_BF16_TFLOPS}
    else:
        roof = {"bound": "hbm", "achieved": achieved_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved_gbs / PEAK_HBM_GBS}
    roof.update({"traffic": traffic, "traffic_detail": traffic_detail,
                 "kernel": "decode_kernel" if cfg == 3 else "decode_fp8_h128_kernel", "kernel_ms": decode_ms,
                 "algorithmic_flop_per_launch": flops, "algorithmic_bytes_per_launch": bytes_,
                 "mfma_achieved_TFLOPs": achieved_tflops, "hbm_achieved_GBs": achieved_gbs})

    res = {
        "metric": (METRIC_SOA.format({"v4": "V4", "v41": "V4.1"}[args.workload]) if soa
                   else {1: METRIC, 2: METRIC_HALFHEAD, 3: METRIC_PREFILL}[cfg]), "value": value,
        "unit": "query-tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "prewarm_steps": n_pre, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl_name, "b": w0.b, "s_q": w0.s_q, "h_q": w0.h_q,
                   "topk": w0.topk, "valid_slots": n_valid,
                   "kv_cache": (f"bf16 {w0.row_bytes} B/token, flat, {w0.num_kv_tokens} tokens" if cfg == 3 else
                                f"fp8 {w0.row_bytes} B/token, page 64, {w0.num_kv_tokens // w0.b} tokens/seq"),
                   "layers_rotated": n_layers, "split_granularity": args.split_granularity,
                   "fixed_overhead": args.fixed_overhead, "num_parts": plan.shape.num_parts,
                   "step": ("decode (closed-form plan in-kernel) + combine" if closed
                            else "sched + decode + combine"),
                   "launch": "eager" if not graphs else "hip graph per layer"},
        "roofline": roof,
        "step_roofline_frac": t_roof_ms / ms_per_step,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w0, args.cpu_budget)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
