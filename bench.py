"""Benchmark of one paged MLA decode step on one MI355X.

A step is the whole hot path over one batch: the split-KV decode kernel and
the log-sum-exp combine (the scheduler metadata is computed once per batch of
sequence lengths and timed separately).  Inputs are seeded synthetic bf16
tensors resident in HBM before timing starts.  Successive steps alternate
between independent KV pools whose total exceeds the 256 MB Infinity Cache,
so every step streams its cache from HBM.

Prints one JSON line.  `value` is achieved algorithmic bandwidth (GB/s) of the
whole step; `roofline` rates the dominant kernel (the decode kernel) against
MI355X's 8 TB/s HBM or 2.5 PFLOP/s dense bf16 MFMA peak, with its duration
measured by HIP events that the kernel's dispatch records at its start and
end (mla_decode_splitkv_timed).

    python bench.py [--steps K] [--warmup W] [--workload mem_bound] [--no-cpu-baseline]
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
METRIC = "paged MLA decode: achieved HBM GB/s & TFLOPS (bf16), % of MI355X roofline"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
MALL_BYTES = 256 << 20
BOUND = {"mem_bound": "hbm", "var_len": "hbm", "skewed": "hbm", "causal_sq2": "mfma", "tiny": "hbm"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # Until a few hundred launches have gone through, the gaps between
    # back-to-back kernels are ~20 us longer (mem_bound step 121 us after 10
    # warmup steps, 98.6 after 100, 94.6 after 300 and 95.0 after 1000; the
    # kernels' own durations do not change), so the default warmup is 300
    # steps (about 30 ms).
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--workload", default="mem_bound")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=15.0)
    ap.add_argument("--op", choices=["decode", "append", "absorb"], default="decode",
                    help="append: time the cache append of the workload's new tokens instead; absorb: the "
                         "per-head projections before and after the decode (each prints its own JSON line)")
    ap.add_argument("--append-tokens", type=int, default=0,
                    help="new tokens per sequence for --op append (default: the workload's s_q)")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="before the timed steps, run one plain device copy of this many MiB: the known-size "
                         "kernel that scales the decode kernel's HBM counters in a rocprofv3 --pmc run")
    return ap.parse_args()


KERNEL_SOURCES = {
    "mla_decode_kernel": ("mla_decode.hip", "mla_decode_common.h", "mla_kernels.h"),
    "mla_decode_wide_kernel": ("mla_decode_wide.hip", "mla_decode_common.h", "mla_kernels.h"),
    "mla_append_kernel": ("mla_append.hip", "mla_append.h", "mla_kernels.h"),
    "mla_absorb_kernel": ("mla_absorb.hip", "mla_absorb.h"),
}


def kernel_source_hash(kernel: str) -> str:
    """First 16 hex digits of the sha256 of the sources one decode kernel is
    built from: a traffic record counts only for the source it was taken on."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "paged_mla_decode_03_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def decode_kernel_name(w) -> str:
    """The decode kernel a workload runs: 128-row workgroups above 128 query
    rows per latent head, else 64-row ones."""
    return "mla_decode_wide_kernel" if w.s_q * w.h_q // w.h_kv > 128 else "mla_decode_kernel"


def measured_traffic(w, kernel=None, workload=None):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel source (else None)."""
    kernel = kernel or decode_kernel_name(w)
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload or w.name}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash(kernel):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(inp, budget_s: float) -> dict:
    """The CPU oracle, untuned, on a bounded sample of the same workload:
    whole sequences, in order, until the time budget is spent."""
    from threadpoolctl import threadpool_info

    from oracle.mla_oracle import mla_decode_ref
    from workloads import algorithmic_counts

    w = inp.workload
    L = inp.cache_seqlens.numpy()
    bt = inp.block_table.numpy()
    done, t0 = [], time.perf_counter()
    for b in range(w.batch):
        mla_decode_ref(inp.q, inp.kvcache, bt, L, 512, causal=w.causal, batch_subset=[b])
        done.append(b)
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    sub = algorithmic_counts(w, L[done], bt.shape[1])
    threads = max([t.get("num_threads", 1) for t in threadpool_info()] + [1])
    return {"value": round(sub["total_bytes"] / dt / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle", "tflops": round(sub["flops"] / dt / 1e12, 6), "seconds": round(dt, 3),
            "sample": f"{len(done)} of {w.batch} sequences ({int(L[done].sum())} cached tokens), float64 numpy"}


def bench_append(args):
    """The cache append of one step's new tokens (or of --append-tokens per
    sequence, as a prefill writes them), launched back to back between two
    events on its stream; algorithmic bytes = the new rows read and written
    plus the lengths and block-table entries read."""
    import torch

    sys.path.insert(0, ROOT)
    from paged_mla_decode_03_amd import kvcache_append
    from workloads import WORKLOADS, make_append_inputs

    dev = torch.device("cuda", 0)
    w = WORKLOADS[args.workload]
    s_new = args.append_tokens or w.s_q
    print(f"[bench] generating append inputs for {args.workload}, {s_new} new tokens (seed {args.seed})",
          file=sys.stderr, flush=True)
    inp, kv_new = make_append_inputs(w, args.seed, s_new)
    kv, new = inp.kvcache.to(dev), kv_new.to(dev)
    bt, L = inp.block_table.to(dev), inp.cache_seqlens.to(dev)
    rows = w.batch * s_new * w.h_kv
    nbytes = 2 * rows * 576 * 2 + w.batch * 4 + w.batch * s_new * 4
    for _ in range(args.warmup):
        kvcache_append(new, kv, bt, L)
    torch.cuda.synchronize()
    if args.copy_mb > 0:              # the counters' calibration copy, as for the decode
        src = torch.empty(args.copy_mb << 20, dtype=torch.uint8, device=dev)
        torch.empty_like(src).copy_(src)
        torch.cuda.synchronize()
        del src
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        kvcache_append(new, kv, bt, L)
    e1.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    ev_ms = e0.elapsed_time(e1) / args.steps
    # Through the Python binding a launch costs more host time than a
    # decode-size append takes on the GPU, so the eager loop above measures
    # the host.  The roofline takes the GPU's own rate: the same launches
    # captured once into a HIP graph and replayed (each replay rewrites the
    # same rows, so the cache is checked against the eager result after it).
    want = kv.clone()
    n_graph = 50
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(n_graph):
            kvcache_append(new, kv, bt, L)
    reps = max(1, args.steps // n_graph)
    graph.replay()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    if not torch.equal(kv, want):
        raise RuntimeError("graph replays of the append changed the cache")
    graph_ms = e0.elapsed_time(e1) / (reps * n_graph)
    print(f"[bench] append: {ev_ms * 1e3:.2f} us per launch (events, back to back, host-bound at small sizes), "
          f"{wall_ms * 1e3:.2f} us wall, {graph_ms * 1e3:.2f} us per launch replayed from a graph",
          file=sys.stderr, flush=True)
    gbs = nbytes / (wall_ms * 1e-3) / 1e9
    achieved = nbytes / (graph_ms * 1e-3) / 1e9
    out = {"metric": "paged MLA cache append: achieved HBM GB/s", "value": round(gbs, 2), "unit": "GB/s",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall_ms, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": f"{args.workload} append", "batch": w.batch, "new_tokens": s_new, "h_kv": w.h_kv,
                      "d_qk": 576, "page_size": 64, "seed": args.seed},
           "append_eager_us": round(ev_ms * 1e3, 2), "append_graph_us": round(graph_ms * 1e3, 3),
           "roofline": {"kernel": "mla_append_kernel", "bound": "hbm", "achieved": round(achieved, 2),
                        "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                        "traffic": measured_traffic(w, "mla_append_kernel", f"{args.workload}_append{s_new}"),
                        "per_launch": {"bytes": nbytes}}}
    print(json.dumps(out), flush=True)


def bench_absorb(args):
    """The per-head projections around the decode for the workload's
    B * s_q tokens and h_q heads (random bf16 weights of the model's shape):
    the query absorption W^UK^T q^C and the output projection W^UV o, each
    captured 50 times into a HIP graph and replayed, so the time is the GPU's
    own.  Algorithmic bytes: each operand read once and each result written
    once; flops 2 * tokens * h_q * 128 * 512 per projection."""
    import torch

    sys.path.insert(0, ROOT)
    from paged_mla_decode_03_amd import absorb_o, absorb_q
    from workloads import WORKLOADS, bf16_normal

    dev = torch.device("cuda", 0)
    w = WORKLOADS[args.workload]
    T, H = w.batch * w.s_q, w.h_q
    rng = np.random.Generator(np.random.PCG64(args.seed))
    qn, qr = bf16_normal(rng, (T, H, 128)).to(dev), bf16_normal(rng, (T, H, 64)).to(dev)
    w_uk_t, w_uv = bf16_normal(rng, (H, 512, 128)).to(dev), bf16_normal(rng, (H, 128, 512)).to(dev)
    o = bf16_normal(rng, (T, H, 512)).to(dev)
    q_out = torch.empty((T, H, 576), dtype=torch.bfloat16, device=dev)
    u_out = torch.empty((T, H, 128), dtype=torch.bfloat16, device=dev)
    bytes_q = 2 * (T * H * (128 + 64 + 576) + H * 512 * 128)
    bytes_o = 2 * (T * H * (512 + 128) + H * 128 * 512)
    flops = 2 * T * H * 128 * 512
    if args.copy_mb > 0:              # the counters' calibration copy, as for the decode
        src = torch.empty(args.copy_mb << 20, dtype=torch.uint8, device=dev)
        torch.empty_like(src).copy_(src)
        torch.cuda.synchronize()
        del src
    times = {}
    for name, fn in (("absorb_q", lambda: absorb_q(qn, qr, w_uk_t, q_out)), ("absorb_o", lambda: absorb_o(o, w_uv, u_out))):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        graph, n_graph = torch.cuda.CUDAGraph(), 50
        with torch.cuda.graph(graph):
            for _ in range(n_graph):
                fn()
        reps = max(1, args.steps // n_graph)
        graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        times[name] = e0.elapsed_time(e1) / (reps * n_graph)
    tq, to = times["absorb_q"], times["absorb_o"]
    print(f"[bench] absorb: query {tq * 1e3:.2f} us ({bytes_q / tq / 1e6:.0f} GB/s), "
          f"output {to * 1e3:.2f} us ({bytes_o / to / 1e6:.0f} GB/s) per launch, graph replay", file=sys.stderr, flush=True)
    total = bytes_q + bytes_o
    achieved = total / ((tq + to) * 1e-3) / 1e9
    out = {"metric": "MLA per-head projections around the decode: achieved HBM GB/s", "value": round(achieved, 2),
           "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(tq + to, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16", "data": "synthetic",
           "config": {"workload": f"{args.workload} absorb", "tokens": T, "h_q": H, "d_h": 128, "d_c": 512,
                      "seed": args.seed},
           "absorb_q_us": round(tq * 1e3, 3), "absorb_o_us": round(to * 1e3, 3),
           "tflops": round(2 * flops / ((tq + to) * 1e-3) / 1e12, 2),
           "roofline": {"kernel": "mla_absorb_kernel", "bound": "hbm", "achieved": round(achieved, 2),
                        "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                        "traffic": measured_traffic(w, "mla_absorb_kernel", f"{args.workload}_absorb"),
                        "per_launch": {"bytes_q": bytes_q, "bytes_o": bytes_o, "flops_each": flops}}}
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU; a sharded path is not built "
                          "(the decode shards by sequence with no exchange, see the design notes)",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if args.op == "append":
        bench_append(args)
        return
    if args.op == "absorb":
        bench_absorb(args)
        return

    import torch

    sys.path.insert(0, ROOT)
    from paged_mla_decode_03_amd import (DecodeBuffers, get_mla_metadata, mla_combine_splits, mla_decode_paged,
                                         mla_decode_splitkv, mla_decode_splitkv_timed)
    from workloads import WORKLOADS, algorithmic_counts, make_inputs

    dev = torch.device("cuda", 0)
    w = WORKLOADS[args.workload]
    print(f"[bench] generating {args.workload} (seed {args.seed})", file=sys.stderr, flush=True)
    inp = make_inputs(w, args.seed)
    L = inp.cache_seqlens.numpy()
    counts = algorithmic_counts(w, L, inp.block_table.shape[1])

    q = inp.q.to(dev)
    bt = inp.block_table.to(dev)
    seqlens = inp.cache_seqlens.to(dev)
    kv_bytes = inp.kvcache.numel() * 2
    n_pools = max(2, -(-2 * MALL_BYTES // kv_bytes) + 1)
    pools = [inp.kvcache.to(dev)]
    for i in range(1, n_pools):
        pools.append(pools[0].clone())
    rows = w.s_q * w.h_q // w.h_kv

    # Scheduler metadata (once per batch of lengths), timed on its own.
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    meta, ns = get_mla_metadata(seqlens, rows, w.h_kv)
    e0.record()
    for _ in range(10):
        meta, ns = get_mla_metadata(seqlens, rows, w.h_kv)
    e1.record()
    torch.cuda.synchronize()
    metadata_us = e0.elapsed_time(e1) / 10 * 1e3
    W = meta.shape[0]
    buf = DecodeBuffers(q, pools[0], 512, W)

    # One step: mla_decode_paged, one call that launches the decode and the
    # combine kernel on torch's current stream (which the binding launches on).
    def step(i):
        mla_decode_paged(q, pools[i % n_pools], bt, seqlens, 512, meta, ns, causal=w.causal, buffers=buf)

    # The same two launches through their own entry points, each bracketed by
    # events (used only outside the timed loop: an event between launches
    # widens the gap).
    def split_step(i, evs):
        kv = pools[i % n_pools]
        evs[0].record()
        mla_decode_splitkv(q, kv, bt, seqlens, 512, meta, ns, causal=w.causal, buffers=buf)
        evs[1].record()
        mla_combine_splits(ns, w.s_q, w.h_q, w.h_kv, 512, W, buf)
        evs[2].record()

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    if args.copy_mb > 0:
        src = torch.empty(args.copy_mb << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # The timed steps: launches only, between a synchronize and a pair of
    # events on each side.
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    g0.record()
    for i in range(args.steps):
        step(i)
    g1.record()
    launch_ms = (time.perf_counter() - t_start) * 1e3      # host time to issue the steps
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t_start) * 1e3
    ms_per_step = wall_ms / args.steps
    event_ms_per_step = g0.elapsed_time(g1) / args.steps

    # Per-launch split of a step, from separate steps with events between the
    # launches (outside the timed loop).
    n_split = min(args.steps, 10)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_split)]
    for i in range(n_split):
        split_step(i, evs[i])
    torch.cuda.synchronize()
    decode_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    combine_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])

    # The decode kernel alone, launched back to back between two events on
    # its stream: the average is the kernel's own duration plus one dispatch
    # gap, the closest event-based match to a profiler's per-kernel time.
    n_dec = max(args.steps, 10)
    d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    d0.record()
    for i in range(n_dec):
        mla_decode_splitkv(q, pools[i % n_pools], bt, seqlens, 512, meta, ns, causal=w.causal, buffers=buf)
    d1.record()
    torch.cuda.synchronize()
    decode_b2b_ms = d0.elapsed_time(d1) / n_dec

    # The decode kernel alone, each launch bracketed by its own pair of
    # events recorded on the stream with the stream idle before it.
    iso_ms = []
    for i in range(n_dec):
        a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        mla_decode_splitkv(q, pools[i % n_pools], bt, seqlens, 512, meta, ns, causal=w.causal, buffers=buf)
        z.record()
        z.synchronize()
        iso_ms.append(a.elapsed_time(z))
    decode_iso_ms = float(np.mean(iso_ms))

    # The decode kernel's own duration: HIP events that the dispatch records
    # at the kernel's start and end, back-to-back launches.  This is the
    # duration the roofline uses.
    kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_dec)]
    torch.cuda.synchronize()
    for i in range(n_dec):
        mla_decode_splitkv_timed(q, pools[i % n_pools], bt, seqlens, 512, meta, ns, kev[i][0], kev[i][1],
                                 causal=w.causal, buffers=buf)
    torch.cuda.synchronize()
    kernel_ms = np.array([a.elapsed_time(z) for a, z in kev])
    decode_kernel_ms = float(kernel_ms.mean())
    print(f"[bench] {args.steps} steps: {ms_per_step * 1e3:.1f} us/step (wall), "
          f"{event_ms_per_step * 1e3:.1f} us/step (events), host issue {launch_ms / args.steps * 1e3:.1f} us/step, decode kernel "
          f"{decode_ms.mean() * 1e3:.1f} us in step, {decode_b2b_ms * 1e3:.1f} us back to back, "
          f"{decode_iso_ms * 1e3:.1f} us launched alone, {decode_kernel_ms * 1e3:.1f} us kernel (dispatch events), "
          f"combine {combine_ms.mean() * 1e3:.1f} us", file=sys.stderr, flush=True)

    gbs = counts["total_bytes"] / (ms_per_step * 1e-3) / 1e9
    tflops = counts["flops"] / (ms_per_step * 1e-3) / 1e12
    dec_s = decode_kernel_ms * 1e-3
    bound = BOUND.get(args.workload, "hbm")
    if bound == "hbm":
        achieved, peak, unit = counts["total_bytes"] / dec_s / 1e9, HBM_PEAK_GBS, "GB/s"
    else:
        achieved, peak, unit = counts["flops"] / dec_s / 1e12, MFMA_BF16_PEAK_TFLOPS, "TFLOP/s"
    traffic = measured_traffic(w)
    out = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": w.batch, "s_q": w.s_q, "h_q": w.h_q, "h_kv": w.h_kv,
                   "d_qk": 576, "dv": 512, "page_size": 64, "causal": w.causal,
                   "seqlen_total": int(L.sum()), "seqlen_max": int(L.max()), "seed": args.seed,
                   "kv_pools": n_pools, "num_workers": W},
        "tflops": round(tflops, 2),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "mfma_frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
        "decode_kernel_us": round(decode_kernel_ms * 1e3, 2),
        "decode_launched_alone_us": round(decode_iso_ms * 1e3, 2),
        "decode_back_to_back_us": round(decode_b2b_ms * 1e3, 2),
        "decode_in_step_us": round(decode_ms.mean() * 1e3, 2),
        "combine_kernel_us": round(combine_ms.mean() * 1e3, 2),
        "step_event_us": round(event_ms_per_step * 1e3, 2),
        "metadata_us": round(metadata_us, 2),
        "algorithmic_bytes": counts["total_bytes"],
        "algorithmic_flops": counts["flops"],
        "roofline": {"kernel": decode_kernel_name(w), "bound": bound, "achieved": round(achieved, 2),
                     "peak": peak, "unit": unit, "frac": round(achieved / peak, 4),
                     "traffic": traffic,
                     "per_launch": {"bytes": counts["total_bytes"], "flops": counts["flops"]}},
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_budget_s)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
