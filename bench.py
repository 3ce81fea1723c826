"""Benchmark of the paged MLA decode hot path on one MI355X.

A step is the whole hot path over one batch of sequences: the split-KV
decode kernel and the log-sum-exp combine (the scheduler metadata is
computed once per batch of sequence lengths; a "full step" that recomputes
it is timed too).  Inputs are seeded synthetic bf16 tensors resident in HBM
before timing starts.  Successive steps alternate between independent KV
pools whose total exceeds the 256 MB Infinity Cache, so every step streams
its cache from HBM.

The headline is the largest single-GPU workload, causal_sq2 (B=132, s_q=2
causal, h_q=128, L=8192), which the bf16 matrix cores bound: `value` is its
whole-step throughput in TFLOP/s, and `roofline` rates its decode kernel
against the 2.5 PFLOP/s dense bf16 MFMA peak, the kernel's duration the
average over K back-to-back launches of the decode kernel alone, between
two HIP events on the stream it runs on (the kernel-trace average of the
same command agrees with it; the durations its own dispatches record in
the timed steps, mla_decode_splitkv_timed, carry some 5-12 us of event
overhead and are reported as a distribution).  `per_config` holds the same
measurements for every workload but tiny (kept off the GPU), each with both
roofline fractions (HBM 8 TB/s and MFMA).

Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--workload causal_sq2] [--configs all|none]
                    [--no-cpu-baseline]
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
# Workloads kept off the GPU (an input that faulted an earlier decode kernel;
# see the design notes' fault history) until the cause is shown on the CPU.
OFF_GPU = {"tiny"}


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
    ap.add_argument("--workload", default="causal_sq2",
                    help="the headline workload (the largest one by default)")
    ap.add_argument("--configs", default="all",
                    help="'all': also measure the other workloads into per_config; 'none': the headline only")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=15.0)
    ap.add_argument("--op", choices=["decode", "append", "absorb", "outproj", "fp8", "lds"], default="decode",
                    help="append: time the cache append of the workload's new tokens instead; absorb: the "
                         "per-head projections before and after the decode (each prints its own JSON line); "
                         "lds: the LDS read rate of one wave, by read kind, at one and two waves per SIMD")
    ap.add_argument("--append-tokens", type=int, default=0,
                    help="new tokens per sequence for --op append (default: the workload's s_q)")
    ap.add_argument("--cache", choices=["streamed", "resident"], default="streamed",
                    help="resident: remap every sequence's pages into the first 64 pages of one pool (4.7 MB, "
                         "held in L2 / MALL), the same decode without HBM streaming, to separate its cost; "
                         "streamed (default): the workload as generated, over pools rotated per step")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="before the timed steps, run one plain device copy of this many MiB: the known-size "
                         "kernel that scales the decode kernel's HBM counters in a rocprofv3 --pmc run")
    return ap.parse_args()


KERNEL_SOURCES = {
    "mla_decode_kernel": ("mla_decode.hip", "mla_decode_common.h", "mla_kernels.h"),
    "mla_decode_wide_kernel": ("mla_decode_wide.hip", "mla_decode_common.h", "mla_kernels.h"),
    "mla_append_kernel": ("mla_append.hip", "mla_append.h", "mla_kernels.h"),
    "mla_absorb_kernel": ("mla_absorb.hip", "mla_absorb.h"),
    "mla_outproj_kernel": ("mla_outproj.hip", "mla_outproj.h"),
    "mla_decode_fp8_kernel": ("mla_decode.hip", "mla_decode_common.h", "mla_kernels.h"),
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


def bench_outproj(args):
    """The output projection over all heads, u = W^O [o_1; ...; o_h], for
    the workload's B * s_q tokens, h_q = 128 heads of d_h = 128 and
    d_model = h_q * d_h = 16384 (the multi-head convention that each head is
    d_model / n_h wide), random bf16 weights; 20 launches captured into a
    HIP graph and replayed.  Algorithmic bytes: W^O and the per-head outputs
    read once, u written once; flops 2 * tokens * d_model * h_q * d_h."""
    import torch

    sys.path.insert(0, ROOT)
    from paged_mla_decode_03_amd import outproj
    from paged_mla_decode_03_amd.binding import library
    from workloads import WORKLOADS, bf16_normal

    dev = torch.device("cuda", 0)
    w = WORKLOADS[args.workload]
    T, H = w.batch * w.s_q, w.h_q
    K, N = H * 128, H * 128
    rng = np.random.Generator(np.random.PCG64(args.seed))
    o = bf16_normal(rng, (T, H, 128)).to(dev)
    wo = bf16_normal(rng, (N, K)).to(dev)
    out = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
    need = int(library().mla_outproj_workspace_bytes(T, K, N))
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    nbytes = 2 * (N * K + T * K + T * N)
    flops = 2 * T * N * K
    fn = lambda: outproj(o, wo, out, ws)
    for _ in range(args.warmup):
        fn()
    torch.cuda.synchronize()
    if args.copy_mb > 0:
        src = torch.empty(args.copy_mb << 20, dtype=torch.uint8, device=dev)
        torch.empty_like(src).copy_(src)
        torch.cuda.synchronize()
        del src
    graph, n_graph = torch.cuda.CUDAGraph(), 20
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
    ms = e0.elapsed_time(e1) / (reps * n_graph)
    gbs = nbytes / (ms * 1e-3) / 1e9
    print(f"[bench] outproj: {ms * 1e3:.2f} us per call ({gbs:.0f} GB/s, {flops / ms / 1e9:.0f} TFLOP/s), "
          f"split-K workspace {need} B", file=sys.stderr, flush=True)
    out_line = {"metric": "MLA output projection over all heads: achieved HBM GB/s", "value": round(gbs, 2),
                "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
                "dtype": "bf16", "data": "synthetic",
                "config": {"workload": f"{args.workload} outproj", "tokens": T, "h_q": H, "d_h": 128,
                           "d_model": N, "seed": args.seed},
                "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
                "roofline": {"kernel": "mla_outproj_kernel", "bound": "hbm", "achieved": round(gbs, 2),
                             "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                             "traffic": measured_traffic(w, "mla_outproj_kernel", f"{args.workload}_outproj"),
                             "per_launch": {"bytes": nbytes, "flops": flops}}}
    print(json.dumps(out_line), flush=True)


def _fp8_codes(latents, kv_scale):
    """E4M3 codes of latents / kv_scale by torch's float8 cast (round to
    nearest even; the values are clamped to +-448 first): the fp8 cache a
    quantising append would leave for the benchmark's latents."""
    import torch
    x = (latents.float() * (1.0 / kv_scale)).clamp_(-448.0, 448.0)
    return x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def bench_fp8(args):
    """The decode over an fp8 cache (one byte per cached value, OCP E4M3 codes
    with one scale) against the same step over the bf16 cache, on the
    workloads with up to 128 query rows per head (mem_bound, var_len,
    skewed): median step time (decode + combine, events around each step,
    pools rotated past the Infinity Cache) and the step's algorithmic rate,
    the fp8 cache counted at one byte per value."""
    import torch

    sys.path.insert(0, ROOT)
    from paged_mla_decode_03_amd import DecodeBuffers, get_mla_metadata, mla_decode_paged, mla_decode_paged_fp8
    from workloads import FP8_KV_SCALE, WORKLOADS, algorithmic_counts, make_fp8_inputs, make_inputs

    dev = torch.device("cuda", 0)
    if args.copy_mb > 0:              # the counters' calibration copy, as for the decode
        src = torch.empty(args.copy_mb << 20, dtype=torch.uint8, device=dev)
        torch.empty_like(src).copy_(src)
        torch.cuda.synchronize()
        del src
    res = {}
    for name in ("mem_bound", "var_len", "skewed"):
        w = WORKLOADS[name]
        out = {}
        for kind in ("bf16", "fp8"):
            print(f"[bench] fp8 op: {name} {kind}", file=sys.stderr, flush=True)
            inp = make_fp8_inputs(w, args.seed, encode=_fp8_codes) if kind == "fp8" else make_inputs(w, args.seed)
            L = inp.cache_seqlens.numpy()
            counts = algorithmic_counts(w, L, inp.block_table.shape[1])
            nbytes = counts["total_bytes"] - (counts["kv_bytes"] // 2 if kind == "fp8" else 0)
            q, bt, sl = inp.q.to(dev), inp.block_table.to(dev), inp.cache_seqlens.to(dev)
            kv_bytes = inp.kvcache.numel() * inp.kvcache.element_size()
            n_pools = max(2, -(-2 * MALL_BYTES // kv_bytes) + 1)
            pools = [inp.kvcache.to(dev)]
            for _ in range(1, n_pools):
                pools.append(pools[0].clone())
            meta, ns = get_mla_metadata(sl, w.s_q * w.h_q // w.h_kv, w.h_kv)
            buf = DecodeBuffers(q, pools[0] if kind == "bf16" else torch.empty((1, 64, w.h_kv, 576), device=dev,
                                                                                dtype=torch.bfloat16),
                                512, meta.shape[0])
            if kind == "fp8":
                sc = inp.extra["kv_scale"]
                fn = lambda i: mla_decode_paged_fp8(q, pools[i % n_pools], sc, bt, sl, 512, meta, ns, buffers=buf)
            else:
                fn = lambda i: mla_decode_paged(q, pools[i % n_pools], bt, sl, 512, meta, ns, buffers=buf)
            for i in range(args.warmup):
                fn(i)
            torch.cuda.synchronize()
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
            for i in range(args.steps):
                evs[i][0].record()
                fn(i)
                evs[i][1].record()
            torch.cuda.synchronize()
            us = np.array([a.elapsed_time(z) for a, z in evs]) * 1e3
            med = float(np.median(us))
            out[kind] = {"step_us_median": round(med, 2), "p10": round(_pct(us, 10), 2), "p90": round(_pct(us, 90), 2),
                         "algorithmic_bytes": int(nbytes), "gbs": round(nbytes / (med * 1e-6) / 1e9, 2),
                         "hbm_frac": round(nbytes / (med * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
            del pools, q, bt, sl, buf, inp
            torch.cuda.empty_cache()
        out["speedup_vs_bf16"] = round(out["bf16"]["step_us_median"] / out["fp8"]["step_us_median"], 3)
        print(f"[bench] fp8 op: {name}: bf16 {out['bf16']['step_us_median']} us, fp8 {out['fp8']['step_us_median']} us "
              f"({out['speedup_vs_bf16']}x)", file=sys.stderr, flush=True)
        res[name] = out
    head = res["mem_bound"]["fp8"]
    line = {"metric": "paged MLA decode over an fp8 cache: achieved HBM GB/s (fp8 bytes)", "value": head["gbs"],
            "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(head["step_us_median"] / 1e3, 5), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "fp8 cache, bf16 compute", "data": "synthetic",
            "config": {"workload": "mem_bound fp8 cache", "kv_scale": FP8_KV_SCALE, "seed": args.seed},
            "roofline": {"kernel": "mla_decode_fp8_kernel", "bound": "hbm", "achieved": head["gbs"],
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": head["hbm_frac"],
                         "traffic": measured_traffic(WORKLOADS["mem_bound"], "mla_decode_fp8_kernel", "mem_bound"),
                         "duration": "median step (decode + combine)"},
            "per_config": res}
    print(json.dumps(line), flush=True)


def _pct(a, q):
    return float(np.percentile(np.asarray(a), q))


def gpu_clock_mhz():
    """Current shader clock from sysfs (the entry marked '*' of
    pp_dpm_sclk), or None where it cannot be read."""
    import glob
    import re
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            for line in open(path).read().splitlines():
                if line.strip().endswith("*"):
                    m = re.search(r"(\d+)\s*Mhz", line, re.I)
                    if m:
                        return int(m.group(1))
        except OSError:
            continue
    return None


def achievable_bandwidth(dev, mib: int = 2048) -> dict:
    """Measured HBM rates beside the 8 TB/s spec: the library's plain
    streaming read of `mib` MiB (mla_stream_read) and a plain device copy of
    half of it (read + write), each the median of 10 event-timed runs after
    warmup."""
    import torch
    from paged_mla_decode_03_amd.binding import stream_read
    n = mib << 20
    src = torch.ones(n // 4, dtype=torch.float32, device=dev)
    half = src[: n // 8]
    dst = torch.empty_like(half)
    sink = torch.empty(4, dtype=torch.int32, device=dev)
    out = {}
    for name, fn, nbytes in (("read_gbs", lambda: stream_read(src, sink), n),
                             ("copy_gbs", lambda: dst.copy_(half), n)):
        for _ in range(3):
            fn()
        ts = []
        for _ in range(10):
            a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            z.record()
            z.synchronize()
            ts.append(a.elapsed_time(z))
        out[name] = round(nbytes / (float(np.median(ts)) * 1e-3) / 1e9, 1)
    del src, dst
    torch.cuda.empty_cache()
    return out


def measure_workload(name: str, args, dev, want_cpu: bool) -> dict:
    """All measurements of one workload (see the module docstring)."""
    import torch

    from paged_mla_decode_03_amd import (DecodeBuffers, get_mla_metadata, mla_combine_splits, mla_decode_paged,
                                         mla_decode_splitkv, mla_decode_splitkv_timed)
    from workloads import WORKLOADS, algorithmic_counts, make_inputs

    w = WORKLOADS[name]
    print(f"[bench] generating {name} (seed {args.seed})", file=sys.stderr, flush=True)
    inp = make_inputs(w, args.seed)
    L = inp.cache_seqlens.numpy()
    counts = algorithmic_counts(w, L, inp.block_table.shape[1])
    q = inp.q.to(dev)
    bt = inp.block_table.to(dev)
    seqlens = inp.cache_seqlens.to(dev)
    kv_bytes = inp.kvcache.numel() * 2
    n_pools = max(2, -(-2 * MALL_BYTES // kv_bytes) + 1)
    if getattr(args, "cache", "streamed") == "resident":
        # Same shapes and lengths; every page id folded into the pool's first
        # 64 pages, so the decode reads a cache that stays on chip.
        bt = torch.where(bt >= 0, bt % 64, bt)
        n_pools = 1
    pools = [inp.kvcache.to(dev)]
    for _ in range(1, n_pools):
        pools.append(pools[0].clone())
    rows = w.s_q * w.h_q // w.h_kv

    # Scheduler metadata (once per batch of lengths), timed on its own.
    torch.cuda.synchronize()
    meta, ns = get_mla_metadata(seqlens, rows, w.h_kv)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(20):
        meta, ns = get_mla_metadata(seqlens, rows, w.h_kv)
    e1.record()
    torch.cuda.synchronize()
    metadata_us = e0.elapsed_time(e1) / 20 * 1e3
    W = meta.shape[0]
    buf = DecodeBuffers(q, pools[0], 512, W)
    splits = np.diff(ns.cpu().numpy())
    # Bytes per kernel: the combine writes o and lse of split sequences.
    split_rows = int((splits > 1).sum()) * w.s_q * w.h_q
    combine_bytes = split_rows * (512 * 2 + 4)
    decode_bytes = counts["total_bytes"] - combine_bytes

    # One step: the decode kernel (its dispatch records two events, so the
    # kernel's own duration comes from the timed steps themselves) and the
    # combine, on torch's current stream.
    def step(i, evs=None):
        kv = pools[i % n_pools]
        if evs is None:
            mla_decode_paged(q, kv, bt, seqlens, 512, meta, ns, causal=w.causal, buffers=buf)
        else:
            mla_decode_splitkv_timed(q, kv, bt, seqlens, 512, meta, ns, evs[0], evs[1], causal=w.causal,
                                     buffers=buf)
            mla_combine_splits(ns, w.s_q, w.h_q, w.h_kv, 512, W, buf)

    K = args.steps
    kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    print(f"[bench] {name}: warmup {args.warmup}", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i, kev[i % K])
    torch.cuda.synchronize()
    if args.copy_mb > 0:
        src = torch.empty(args.copy_mb << 20, dtype=torch.uint8, device=dev)
        torch.empty_like(src).copy_(src)
        torch.cuda.synchronize()
        del src

    # The timed steps, launches only, between a synchronize and a pair of
    # events on each side.
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g0.record()
    for i in range(K):
        step(i, kev[i])
    g1.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    ms_per_step = wall_ms / K
    event_ms_per_step = g0.elapsed_time(g1) / K
    kernel_ms = np.array([a.elapsed_time(z) for a, z in kev])

    # Step-time distribution: each step bracketed by events on the stream
    # (plain mla_decode_paged); then the full step with the metadata.
    def timed_loop(fn):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
        torch.cuda.synchronize()
        for i in range(K):
            evs[i][0].record()
            fn(i)
            evs[i][1].record()
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(z) for a, z in evs]) * 1e3

    step_us = timed_loop(lambda i: step(i))

    def full(i):
        m, n = get_mla_metadata(seqlens, rows, w.h_kv)
        mla_decode_paged(q, pools[i % n_pools], bt, seqlens, 512, m, n, causal=w.causal, buffers=buf)

    full_us = timed_loop(full)

    # The decode kernel alone, K launches back to back (pools rotated as in
    # the steps) between two events on the stream it runs on: its average
    # duration, the roofline's denominator.  (The dispatch-recorded events of
    # the timed steps add some 5-12 us of event overhead per launch; they are
    # kept as a distribution.)
    torch.cuda.synchronize()
    d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    d0.record()
    for i in range(K):
        mla_decode_splitkv(q, pools[i % n_pools], bt, seqlens, 512, meta, ns, causal=w.causal, buffers=buf)
    d1.record()
    torch.cuda.synchronize()
    kernel_batch_us = d0.elapsed_time(d1) / K * 1e3
    clock = gpu_clock_mhz()

    kernel_mean_s = kernel_batch_us * 1e-6
    res = {
        "config": {"workload": name, "batch": w.batch, "s_q": w.s_q, "h_q": w.h_q, "h_kv": w.h_kv, "d_qk": 576,
                   "dv": 512, "page_size": 64, "causal": w.causal, "seqlen_total": int(L.sum()),
                   "seqlen_max": int(L.max()), "seed": args.seed, "kv_pools": n_pools, "num_workers": W,
                   "max_splits": int(splits.max()), "cache": getattr(args, "cache", "streamed")},
        "us_per_step": round(ms_per_step * 1e3, 2),
        "step_event_us": round(event_ms_per_step * 1e3, 2),
        "step_us": {"median": round(float(np.median(step_us)), 2), "p10": round(_pct(step_us, 10), 2),
                    "p90": round(_pct(step_us, 90), 2)},
        "full_step_with_metadata_us": {"median": round(float(np.median(full_us)), 2),
                                       "p10": round(_pct(full_us, 10), 2), "p90": round(_pct(full_us, 90), 2)},
        "metadata_us": round(metadata_us, 2),
        "decode_kernel_us": {"mean": round(kernel_mean_s * 1e6, 2),
                             "dispatch_events": {"mean": round(float(kernel_ms.mean()) * 1e3, 2),
                                                 "median": round(float(np.median(kernel_ms)) * 1e3, 2),
                                                 "p10": round(_pct(kernel_ms, 10) * 1e3, 2),
                                                 "p90": round(_pct(kernel_ms, 90) * 1e3, 2)}},
        "step": {"gbs": round(counts["total_bytes"] / (ms_per_step * 1e-3) / 1e9, 2),
                 "tflops": round(counts["flops"] / (ms_per_step * 1e-3) / 1e12, 2),
                 "hbm_frac": round(counts["total_bytes"] / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                 "mfma_frac": round(counts["flops"] / (ms_per_step * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)},
        "decode_kernel": {"kernel": decode_kernel_name(w), "bytes": decode_bytes, "flops": counts["flops"],
                          "gbs": round(decode_bytes / kernel_mean_s / 1e9, 2),
                          "tflops": round(counts["flops"] / kernel_mean_s / 1e12, 2),
                          "hbm_frac": round(decode_bytes / kernel_mean_s / 1e9 / HBM_PEAK_GBS, 4),
                          "mfma_frac": round(counts["flops"] / kernel_mean_s / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                          "traffic": measured_traffic(w) if getattr(args, "cache", "streamed") == "streamed" else None},
        "algorithmic_bytes": counts["total_bytes"],
        "algorithmic_flops": counts["flops"],
        "combine_bytes": combine_bytes,
        "gpu_clock_mhz_after": clock,
    }
    print(f"[bench] {name}: {res['us_per_step']} us/step (wall), step median {res['step_us']['median']} us, "
          f"decode kernel mean {res['decode_kernel_us']['mean']} us ({res['decode_kernel']['hbm_frac']:.3f} HBM, "
          f"{res['decode_kernel']['mfma_frac']:.3f} MFMA), full step {res['full_step_with_metadata_us']['median']} us",
          file=sys.stderr, flush=True)
    if want_cpu:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(inp, args.cpu_budget_s)
    del pools, q, bt, seqlens, buf, inp
    torch.cuda.empty_cache()
    return res


def bench_lds(args):
    """The rate at which one wave reads LDS (mla_lds_read_rate): for each read
    kind, one workgroup per CU of four waves (one per SIMD, as the 128-row
    decode workgroup) and of eight (two per SIMD, as the 64-row one); cycles
    are the shader clock's (s_memtime) over each workgroup's loop, median over
    the workgroups of the third of three launches.  A decode stream whose
    fragment reads per MFMA exceed this rate waits on LDS, not on the matrix
    core."""
    import torch
    sys.path.insert(0, ROOT)
    from paged_mla_decode_03_amd.binding import LDS_READ_KINDS, lds_read_rate
    dev = torch.device("cuda", 0)
    blocks = torch.cuda.get_device_properties(dev).multi_processor_count
    iters = 1024
    rates = {}
    for kind, (_, lane_bytes) in LDS_READ_KINDS.items():
        for waves in (4, 8):
            for _ in range(3):
                cyc = lds_read_rate(kind, waves, iters, blocks, dev)
            torch.cuda.synchronize()
            c = float(np.median(cyc.cpu().numpy()))
            reads = 64 * iters
            rates[f"{kind}/{waves}w"] = {"cycles_per_read": round(c / reads, 2),
                                         "bytes_per_cycle_per_wave": round(reads * 64 * lane_bytes / c, 2),
                                         "bytes_per_cycle_per_cu": round(waves * reads * 64 * lane_bytes / c, 1)}
    print(json.dumps({"metric": "LDS read rate of one wave", "unit": "cycles per read",
                      "config": {"workload": "lds_read_rate", "blocks": blocks, "reads_per_wave": 64 * iters,
                                 "in_flight_per_wave": 8},
                      "rates": rates}))


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
    if args.op == "outproj":
        bench_outproj(args)
        return
    if args.op == "fp8":
        bench_fp8(args)
        return
    if args.op == "lds":
        bench_lds(args)
        return

    import torch

    sys.path.insert(0, ROOT)
    from workloads import WORKLOADS

    if args.workload in OFF_GPU:
        print(json.dumps({"error": f"workload {args.workload} is kept off the GPU (see the design notes)"}))
        sys.exit(2)
    dev = torch.device("cuda", 0)
    head = measure_workload(args.workload, args, dev, not args.no_cpu_baseline)
    per_config = {args.workload: head}
    if args.configs == "all":
        for name in WORKLOADS:
            if name != args.workload and name not in OFF_GPU:
                per_config[name] = measure_workload(name, args, dev, False)
    achievable = achievable_bandwidth(dev)
    bound = BOUND.get(args.workload, "hbm")
    dk = head["decode_kernel"]
    if bound == "hbm":
        achieved, peak, unit = dk["gbs"], HBM_PEAK_GBS, "GB/s"
        value, vunit = head["step"]["gbs"], "GB/s"
    else:
        achieved, peak, unit = dk["tflops"], MFMA_BF16_PEAK_TFLOPS, "TFLOP/s"
        value, vunit = head["step"]["tflops"], "TFLOP/s"
    out = {
        "metric": METRIC,
        "value": value,
        "unit": vunit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["us_per_step"] / 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": head["config"],
        "gbs": head["step"]["gbs"],
        "tflops": head["step"]["tflops"],
        "us_per_step": head["us_per_step"],
        "hbm_frac": head["step"]["hbm_frac"],
        "mfma_frac": head["step"]["mfma_frac"],
        "roofline": {"kernel": dk["kernel"], "bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
                     "frac": round(achieved / peak, 4), "traffic": dk["traffic"],
                     "duration": "average of the decode kernel over K back-to-back launches, events on its stream",
                     "kernel_us": head["decode_kernel_us"]["mean"],
                     "per_launch": {"bytes": dk["bytes"], "flops": dk["flops"]},
                     "hbm_frac": dk["hbm_frac"], "mfma_frac": dk["mfma_frac"]},
        "achievable_hbm": achievable,
        "per_config": {k: {kk: vv for kk, vv in v.items() if kk != "cpu_baseline"} for k, v in per_config.items()},
    }
    if "cpu_baseline" in head:
        out["cpu_baseline"] = head["cpu_baseline"]
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
