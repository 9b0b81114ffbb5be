#!/usr/bin/env python3
"""Benchmark of the single-token GQA decode step on one MI355X.

A step is one prepared decode launch (attention kernel + log-sum-exp combine)
over one batch of synthetic, seeded inputs already resident in HBM. The
default (headline) workload is the largest one-GPU configuration: 16
requests, capacity 131072, lengths uniform in [65536, 131072], 32 query / 8
KV heads, head_dim 128, q bf16, an fp8_e4m3 cache with k_scale = v_scale =
1/64, bf16 output.

Printed: one JSON line with the whole-step KV-read throughput (GB/s of
algorithmic bytes: the valid K/V prefixes plus q, out and the lengths), the
attention kernel's roofline position (bytes per launch over its average
duration from HIP events recorded on the launch stream around every timed
launch, against 8 TB/s), cold-cache microseconds per call, the CPU oracle
timed on a bounded sample of the same workload, and under "configs" every
one of the five decode configurations (the headline's figures included),
each timed in this run as direct launches, as replays of a captured one-step
graph and as replays of a captured sixteen-step graph.

    python bench.py [--steps 50] [--warmup W] [--workload NAME] [--num-splits N]
"""

from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GQA decode: achieved KV-read HBM GB/s (% of peak) and µs/call at 1 GPU"
PEAK_HBM_GBPS = 8000.0
DEFAULT_WORKLOAD = "gqa_decode_b16_c131072_fp8kv_long"
# The five decode configurations, timed in every default run.
CONFIG_WORKLOADS = ["gqa_decode_b1_c64_f16", "gqa_decode_b1_c1024_f16",
                    "gqa_decode_b32_c8192_f16_ragged", "gqa_decode_b8_c65536_bf16_long",
                    "gqa_decode_b16_c131072_fp8kv_long"]
GRAPH_STEPS = 16    # steps captured in the multi-step graph
PROFILES = os.path.join(ROOT, "profiles")


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps first (default: at least 200 steps and at least "
                         "2 s of them; the clocks take some tens of milliseconds of steady "
                         "load to settle after the idle input setup, and right after other "
                         "GPU work the memory can read ~5%% slower for a second or more)")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--num-splits", type=int, default=0, help="0 = automatic")
    ap.add_argument("--fused-combine", action="store_true",
                    help="merge chunks in the last workgroup instead of a second kernel")
    ap.add_argument("--cold-calls", type=int, default=50,
                    help="calls timed one by one after a 512 MiB cache-flush write")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="CPU-oracle time budget for the cpu_baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip timing the five decode configurations besides the headline")
    ap.add_argument("--page-size", type=int, default=0,
                    help="paged workloads: override the page size (slots per page)")
    ap.add_argument("--q-tokens", type=int, default=0,
                    help="paged workloads: override the query tokens per request")
    ap.add_argument("--scales-by-position", action="store_true",
                    help="INT8 page pools: row scales indexed by position "
                         "([batch, 2, 8, max_pages * page_size]) instead of beside their rows")
    ap.add_argument("--page-order", choices=("random", "ordered"), default="random",
                    help="paged workloads: the block table as drawn (a random permutation "
                         "of the pool) or each request's pages in pool order, as an "
                         "allocator that hands out pages in turn gives them")
    ap.add_argument("--shape", default="",
                    help="override batch,capacity,len_lo,len_hi (e.g. 16,131072,65536,131072)")
    return ap.parse_args()


def algorithmic_bytes(lens, kv_dtype, batch, num_q_heads=32, q_tokens=1, page_size=0):
    """Valid K/V prefix bytes (an INT8 cache's bf16 row scales included) + q and
    out (16-bit, q_tokens rows per head) + int32 lengths (+ the block-table
    entries of the pages the prefixes occupy); no padding, no workspace."""
    from gqa_kv_cache_attn_amd.inputs import kv_slot_bytes
    table = 4 * sum(-(-int(L) // page_size) for L in lens) if page_size else 0
    return (int(sum(lens)) * 8 * kv_slot_bytes(kv_dtype)
            + batch * q_tokens * num_q_heads * 128 * (2 + 2) + 4 * batch + table)


def kernel_source_digest(kernel):
    from gqa_kv_cache_attn_amd.profile_summary import kernel_source_digest as digest
    return digest(kernel)


def read_traffic(kernel, workload, num_splits):
    """HBM bytes per attention launch from committed rocprofv3 --pmc summaries.

    The summary file is only used while its recorded kernel-source digest
    matches the current source; otherwise traffic is reported as null."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.lstrip().startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != kernel_source_digest(kernel):
        return None
    if int(kv.get("num_splits_requested", "0")) != num_splits:
        return None
    try:
        return int(float(kv["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def cpu_model() -> str:
    """The host CPU's model name (Linux /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline_paged(inp, w, budget_s):
    """Time the paged fp64 oracle (as it stands) one request at a time until the budget."""
    import numpy as np

    from gqa_kv_cache_attn_amd.inputs import kv_slot_bytes, storage_bits
    from oracle import decode_int8_rows, decode_storage
    from oracle.paged import gqa_decode_multi, gqa_decode_paged_reference, int8_rows_by_position

    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:   # pragma: no cover - threadpoolctl missing
        blas_threads = 1
    lens = inp["seq_lens"].cpu().numpy()
    P = w.page_size
    spent, nbytes, done = 0.0, 0, 0
    for b in range(w.batch):
        L = int(lens[b])
        n = -(-L // P)
        ids = inp["block_table"][b, :n].long()
        pages = storage_bits(inp["kv_pages"].index_select(0, ids))   # D2H copies are not timed
        by_pos = inp.get("scales_by_position", False)
        if w.kv_dtype != "int8":
            sc = None
        elif by_pos:
            sc = storage_bits(inp["kv_scales"][b:b + 1, :, :, :n * P])
        else:
            sc = storage_bits(inp["kv_scales"].index_select(0, ids))
        qb = storage_bits(inp["q"][b:b + 1])
        t0 = time.perf_counter()
        q = decode_storage(qb, w.q_dtype)
        if by_pos:
            rows = int8_rows_by_position(pages, sc, np.arange(n)[None, :], [L], P)
            out = gqa_decode_multi(q, rows, [L], w.q_scale, w.k_scale, w.v_scale)
        else:
            dec = decode_int8_rows(pages, sc) if sc is not None else decode_storage(pages, w.kv_dtype)
            out = gqa_decode_paged_reference(q, dec, np.arange(n)[None, :], [L], P, w.q_scale,
                                             w.k_scale, w.v_scale)
        spent += time.perf_counter() - t0
        assert np.all(np.isfinite(out))
        nbytes += L * 8 * kv_slot_bytes(w.kv_dtype) + w.q_tokens * w.num_q_heads * 128 * 4
        done += 1
        if spent >= budget_s:
            break
    return {
        "value": round(nbytes / spent / 1e9, 4),
        "unit": "GB/s",
        "cores": int(blas_threads),
        "kind": "oracle",
        "sample": f"{done} of {w.batch} requests of {w.name}, {nbytes / 1e6:.1f} MB of algorithmic "
                  f"bytes, {spent:.2f} s (fp64 numpy incl. decoding the stored pages and the "
                  f"slot-by-slot gather; D2H copy excluded)",
        "seconds": round(spent, 3),
        "affinity_cpus": len(os.sched_getaffinity(0)),
        "cpu_model": cpu_model(),
    }


def cpu_baseline(inp, w, budget_s):
    """Time the fp64 oracle (as it stands) on (request, KV head) pairs until the budget."""
    import numpy as np

    from gqa_kv_cache_attn_amd.inputs import kv_slot_bytes, storage_bits
    from oracle import decode_int8_rows, decode_storage, gqa_decode_head

    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:   # pragma: no cover - threadpoolctl missing
        blas_threads = 1
    lens = inp["seq_lens"].cpu().numpy()
    G = w.num_q_heads // 8
    int8 = w.kv_dtype == "int8"
    pairs = [(b, g) for g in range(8) for b in range(w.batch)]
    spent, nbytes, done = 0.0, 0, 0
    for (b, g) in pairs:
        L = int(lens[b])
        qb = storage_bits(inp["q"][b, G * g:G * g + G])          # D2H copies are not timed
        kb = storage_bits(inp["kv"][b, 0, g, :L])
        vb = storage_bits(inp["kv"][b, 1, g, :L])
        if int8:
            ksb = storage_bits(inp["kv_scales"][b, 0, g, :L])
            vsb = storage_bits(inp["kv_scales"][b, 1, g, :L])
        t0 = time.perf_counter()
        if int8:
            k, v = decode_int8_rows(kb, ksb), decode_int8_rows(vb, vsb)
        else:
            k, v = decode_storage(kb, w.kv_dtype), decode_storage(vb, w.kv_dtype)
        out = gqa_decode_head(decode_storage(qb, w.q_dtype), k, v, w.q_scale, w.k_scale, w.v_scale)
        spent += time.perf_counter() - t0
        assert np.all(np.isfinite(out))
        nbytes += L * kv_slot_bytes(w.kv_dtype) + G * 128 * 4
        done += 1
        if spent >= budget_s:
            break
    return {
        "value": round(nbytes / spent / 1e9, 4),
        "unit": "GB/s",
        "cores": int(blas_threads),
        "kind": "oracle",
        "sample": f"{done} of {len(pairs)} (request, KV head) pairs of {w.name}, "
                  f"{nbytes / 1e6:.1f} MB of algorithmic bytes, {spent:.2f} s "
                  f"(fp64 numpy incl. decoding the stored {w.kv_dtype} values; D2H copy excluded)",
        "seconds": round(spent, 3),
        "affinity_cpus": len(os.sched_getaffinity(0)),
        "cpu_model": cpu_model(),
    }


def _workload(args, name):
    """The named workload with the command line's shape and paging overrides."""
    import dataclasses

    from gqa_kv_cache_attn_amd.inputs import WORKLOADS_BY_NAME
    w = WORKLOADS_BY_NAME[name]
    if args.shape:
        B, C, lo, hi = (int(x) for x in args.shape.split(","))
        w = dataclasses.replace(w, batch=B, capacity=C, len_lo=lo, len_hi=hi,
                                name=f"{w.name}[B={B},C={C},L={lo}..{hi}]")
    if args.scales_by_position and not (w.page_size and w.kv_dtype == "int8"):
        print("--scales-by-position applies to INT8 paged workloads only", file=sys.stderr)
        sys.exit(2)
    if args.page_size or args.q_tokens or args.page_order != "random":
        if not w.page_size:
            print("--page-size / --q-tokens / --page-order apply to paged workloads only",
                  file=sys.stderr)
            sys.exit(2)
        w = dataclasses.replace(w, page_size=args.page_size or w.page_size,
                                q_tokens=args.q_tokens or w.q_tokens,
                                name=f"{w.name}[P={args.page_size or w.page_size},"
                                     f"T={args.q_tokens or w.q_tokens}]"
                                     + ("[pages in order]" if args.page_order == "ordered" else ""))
    if args.scales_by_position:
        w = dataclasses.replace(w, name=f"{w.name}[scales by position]")
    return w


class Case:
    """One workload's inputs in HBM and its prepared decode step."""

    def __init__(self, w, dev, num_splits=0, fused_combine=False, page_order="random",
                 scales_by_position=False):
        import torch

        from gqa_kv_cache_attn_amd import binding as b
        from gqa_kv_cache_attn_amd.inputs import make_inputs, make_paged_inputs, position_scales
        self.w, self.dev, self.b = w, dev, b
        self.paged = w.page_size > 0
        self.by_position = scales_by_position
        inp = make_paged_inputs(w, device=dev) if self.paged else make_inputs(w, device=dev)
        if self.paged and page_order == "ordered":
            B, max_pages = inp["block_table"].shape
            inp["block_table"] = torch.arange(B * max_pages, device=dev,
                                              dtype=torch.int32).reshape(B, max_pages)
        if scales_by_position:   # the same scales, moved to the slots that read them
            inp["kv_scales"] = position_scales(inp["kv_scales"], inp["block_table"], w.page_size)
            inp["scales_by_position"] = True
        self.inp = inp
        self.lens = inp["seq_lens"].cpu().tolist()
        self.nbytes = algorithmic_bytes(self.lens, w.kv_dtype, w.batch, w.num_q_heads,
                                        w.q_tokens, w.page_size)
        self.out = torch.empty_like(inp["q"])
        if self.paged:
            if fused_combine:
                print("the paged entry points have no one-launch merge", file=sys.stderr)
                sys.exit(2)
            self.prep = b.prepare_gqa_decode_paged(
                inp["q"], inp["kv_pages"], inp["block_table"], inp["seq_lens"], self.out,
                inp["q_scale"], num_splits=num_splits, k_scale=inp["k_scale"],
                v_scale=inp["v_scale"], kv_scales=inp["kv_scales"],
                scales_by_position=scales_by_position)
        elif w.kv_dtype == "int8":
            self.prep = b.prepare_gqa_decode_int8(
                inp["q"], inp["kv"], inp["kv_scales"], inp["seq_lens"], self.out, inp["q_scale"],
                num_splits=num_splits, k_scale=inp["k_scale"], v_scale=inp["v_scale"],
                fused_combine=fused_combine)
        else:
            self.prep = b.prepare_gqa_decode(
                inp["q"], inp["kv"], inp["seq_lens"], self.out, inp["q_scale"],
                num_splits=num_splits, k_scale=inp["k_scale"], v_scale=inp["v_scale"],
                fused_combine=fused_combine)
        self.plan = self.prep.plan

    def step(self):
        self.b.launch_gqa_decode_prepared(self.prep)

    def warm(self, seconds, min_steps=0):
        """Untimed steps for at least `seconds` and `min_steps`; returns the count."""
        import torch
        n, t0 = 0, time.perf_counter()
        while n < min_steps or time.perf_counter() - t0 < seconds:
            for _ in range(50):
                self.step()
            n += 50
            torch.cuda.synchronize()
        return n

    def destroy(self):
        self.prep.destroy()


def _event(stream):
    import torch
    e = torch.cuda.Event(enable_timing=True)
    e.record(stream)            # creates the underlying HIP event
    return e


def _marker(dev, k):
    """A tiny kernel between measurement passes, so a rocprofv3 kernel trace of
    this run can be split into its passes (outside every timed region). It is
    torch's negation of a 256-element tensor, which nothing else in this
    program launches (torch's graph replays launch small fills of their own)."""
    import torch
    torch.full((256,), float(k + 1), device=dev).neg_()
    torch.cuda.synchronize()


def time_direct(case, K, stream):
    """µs per step of K back-to-back prepared launches (events on the launch stream)."""
    import torch
    e0, e1 = _event(stream), _event(stream)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(K):
        case.step()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / K


def time_graph(case, K, stream, steps_per_graph):
    """Capture `steps_per_graph` prepared launches in one torch CUDA graph and
    replay it until at least K steps ran. Returns (µs per step on the GPU,
    host µs per replay call, steps timed)."""
    import torch
    dev = case.dev
    side = torch.cuda.Stream(dev)
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        case.step()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(steps_per_graph):
            case.step()
    # The first replays of a newly instantiated graph run slower; replay it
    # for at least 0.2 s and 10 launches before the timed replays.
    n, t0 = 0, time.perf_counter()
    while n < 10 or time.perf_counter() - t0 < 0.2:
        graph.replay()
        n += 1
        if n % 10 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    launches = -(-K // steps_per_graph)
    e0, e1 = _event(stream), _event(stream)
    torch.cuda.synchronize()
    e0.record(stream)
    h0 = time.perf_counter()
    for _ in range(launches):
        graph.replay()
    h1 = time.perf_counter()
    e1.record(stream)
    torch.cuda.synchronize()
    steps = launches * steps_per_graph
    del graph
    return e0.elapsed_time(e1) * 1e3 / steps, (h1 - h0) * 1e6 / launches, steps


def time_graph_floor(dev, K, stream):
    """The same replay loop over a graph of two one-block fill kernels: the
    runtime's own cost per graph launch, whatever the graph holds. Returns
    (GPU µs per replay, host µs per replay call)."""
    import torch
    t = torch.zeros(64, device=dev)
    side = torch.cuda.Stream(dev)
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        t.fill_(1.0)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        t.fill_(2.0)
        t.fill_(3.0)
    n, t0 = 0, time.perf_counter()
    while n < 10 or time.perf_counter() - t0 < 0.2:
        graph.replay()
        n += 1
        if n % 10 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    e0, e1 = _event(stream), _event(stream)
    torch.cuda.synchronize()
    e0.record(stream)
    h0 = time.perf_counter()
    for _ in range(K):
        graph.replay()
    h1 = time.perf_counter()
    e1.record(stream)
    torch.cuda.synchronize()
    del graph
    return e0.elapsed_time(e1) * 1e3 / K, (h1 - h0) * 1e6 / K


def config_entry(case, direct_us, graph1, graph16):
    gbps = case.nbytes / (direct_us * 1e-6) / 1e9
    return {
        "plan": case.plan,
        "algorithmic_bytes_per_step": case.nbytes,
        "us_per_call": round(direct_us, 2),
        "pct_of_peak": round(100 * gbps / PEAK_HBM_GBPS, 2),
        "us_per_call_graph_1step": round(graph1[0], 2),
        "host_us_per_graph_1step_launch": round(graph1[1], 2),
        "us_per_step_graph_16step": round(graph16[0], 2),
        "pct_of_peak_graph_16step": round(100 * case.nbytes / (graph16[0] * 1e-6) / 1e9
                                          / PEAK_HBM_GBPS, 2),
    }


def measure_config(name, args, dev, stream, phase):
    """Direct, one-step-graph and sixteen-step-graph µs per step of one configuration."""
    import torch
    from gqa_kv_cache_attn_amd.inputs import WORKLOADS_BY_NAME
    w = WORKLOADS_BY_NAME[name]      # as defined: the headline's overrides do not apply
    print(f"[bench] config {w.name}", file=sys.stderr, flush=True)
    case = Case(w, dev)
    _marker(dev, phase)
    case.warm(1.0, 100)
    K = max(args.steps, 48)
    _marker(dev, phase + 1)
    direct = time_direct(case, K, stream)
    _marker(dev, phase + 2)
    g1 = time_graph(case, K, stream, 1)
    _marker(dev, phase + 3)
    g16 = time_graph(case, K, stream, GRAPH_STEPS)
    entry = config_entry(case, direct, g1, g16)
    entry["steps_timed"] = K
    case.destroy()
    del case
    torch.cuda.empty_cache()
    return entry


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: the library "
              "runs the decode step on one GPU (sharding by request, KV head or sequence is a "
              "design, not code).", file=sys.stderr)
        sys.exit(2)

    import torch

    from gqa_kv_cache_attn_amd import binding as b

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    arch = torch.cuda.get_device_properties(dev).gcnArchName
    # Every pass runs on one non-default stream, as a serving loop's decode
    # steps do; graphs are replayed on it too.
    stream = torch.cuda.Stream(dev)
    with torch.cuda.stream(stream):
        result = run(args, dev, arch, stream)
    print(json.dumps(result), flush=True)


def run(args, dev, arch, stream):
    import torch

    from gqa_kv_cache_attn_amd import binding as b
    w = _workload(args, args.workload)

    # The other decode configurations first (each with its own short warm-up),
    # then the headline workload.
    configs = {}
    if not args.no_configs:
        for i, name in enumerate(n for n in CONFIG_WORKLOADS if n != args.workload):
            configs[name] = measure_config(name, args, dev, stream, 10 * (i + 1))

    print(f"[bench] device {arch}; workload {w.name}; generating inputs", file=sys.stderr, flush=True)
    case = Case(w, dev, args.num_splits, args.fused_combine, args.page_order,
                args.scales_by_position)
    paged, inp, out, nbytes, lens = case.paged, case.inp, case.out, case.nbytes, case.lens
    plan = dict(case.plan)
    if plan.get("fused_merge"):
        plan["combine"] = "one launch (the last workgroup of each head merges it)"
    elif plan["route"] != 2 and plan["num_splits"] == 1:
        plan["combine"] = "none (one chunk per head)"
    else:
        plan["combine"] = "separate kernel"

    K = args.steps
    _marker(dev, 99)
    if args.warmup is not None:
        W = args.warmup
        for _ in range(W):
            case.step()
    else:
        W = case.warm(2.0, 200)
    torch.cuda.synchronize()

    # Timed region: exactly K steps, synchronised on both sides, no other
    # work on the stream. `value` and ms_per_step come from here.
    _marker(dev, 100)
    t_begin, t_end = _event(stream), _event(stream)
    torch.cuda.synchronize()
    print(f"[bench] plan {plan}; timing {K} steps", file=sys.stderr, flush=True)
    wall0 = time.perf_counter()
    t_begin.record(stream)
    for _ in range(K):
        case.step()
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = t_begin.elapsed_time(t_end) / K

    # Kernel durations: K more steps with HIP events recorded on the launch
    # stream right before the attention kernel, between it and the combine,
    # and after the combine. (Event packets add a few microseconds between
    # launches, which is why the step time above is taken without them.)
    _marker(dev, 101)
    ev = [[_event(stream) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    for k in range(K):
        b.launch_gqa_decode_prepared_timed(case.prep, ev[k][0], ev[k][1], ev[k][2])
    torch.cuda.synchronize()
    attn_ms = [e[0].elapsed_time(e[1]) for e in ev]
    comb_ms = [e[1].elapsed_time(e[2]) for e in ev]
    attn_avg = statistics.fmean(attn_ms)
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = nbytes / (attn_avg * 1e-3) / 1e9

    # The same step replayed from captured graphs: one step per graph, and
    # sixteen steps per graph (a captured decode loop).
    _marker(dev, 102)
    g1 = time_graph(case, K, stream, 1)
    _marker(dev, 103)
    g16 = time_graph(case, K, stream, GRAPH_STEPS)
    _marker(dev, 104)
    if not args.no_configs or w.name in CONFIG_WORKLOADS:
        configs[w.name] = {**config_entry(case, ms_per_step * 1e3, g1, g16), "steps_timed": K}

    def convenience():
        if paged:
            b.gqa_decode_paged(inp["q"], inp["kv_pages"], inp["block_table"], inp["seq_lens"],
                               inp["q_scale"], out, k_scale=inp["k_scale"], v_scale=inp["v_scale"],
                               kv_scales=inp["kv_scales"],
                               scales_by_position=args.scales_by_position)
        elif w.kv_dtype == "int8":
            b.gqa_decode_int8(inp["q"], inp["kv"], inp["kv_scales"], inp["seq_lens"], inp["q_scale"],
                              out, k_scale=inp["k_scale"], v_scale=inp["v_scale"])
        else:
            b.gqa_decode(inp["q"], inp["kv"], inp["seq_lens"], inp["q_scale"], out,
                         k_scale=inp["k_scale"], v_scale=inp["v_scale"])
    # Warm up for 0.2 s (and at least 3 calls): the graph passes before leave
    # the clocks where their replays put them.
    n, t0 = 0, time.perf_counter()
    while n < 3 or time.perf_counter() - t0 < 0.2:
        convenience()
        n += 1
        if n % 10 == 0:
            torch.cuda.synchronize()
    c_begin, c_end = _event(stream), _event(stream)
    torch.cuda.synchronize()
    c_begin.record(stream)
    for _ in range(K):
        convenience()
    c_end.record(stream)
    torch.cuda.synchronize()
    convenience_us = c_begin.elapsed_time(c_end) / K * 1e3

    # KV append (the cache write before each step): the step's new tokens (one
    # per request, T for a paged verify pass) at slots L_b .. L_b + T - 1, past
    # the valid prefix, so the decode inputs are unchanged (slots past the
    # cache write nothing). An INT8 cache is quantised row by row on the way.
    _marker(dev, 105)
    shape = (w.batch, w.q_tokens, 8, 128) if paged else (w.batch, 8, 128)
    k_new = torch.randn(*shape, device=dev).to(inp["q"].dtype)
    v_new = torch.randn(*shape, device=dev).to(inp["q"].dtype)
    slots = inp["seq_lens"].clone()
    int8 = w.kv_dtype == "int8"
    if paged and int8:
        def append():
            b.gqa_kv_append_paged_int8(inp["kv_pages"], inp["kv_scales"], inp["block_table"],
                                       k_new, v_new, slots, inp["k_scale"], inp["v_scale"],
                                       num_q_heads=w.num_q_heads,
                                       scales_by_position=args.scales_by_position)
    elif paged:
        def append():
            b.gqa_kv_append_paged(inp["kv_pages"], inp["block_table"], k_new, v_new, slots,
                                  inp["k_scale"], inp["v_scale"], num_q_heads=w.num_q_heads)
    elif int8:
        def append():
            b.gqa_kv_append_int8(inp["kv"], inp["kv_scales"], k_new, v_new, slots,
                                 inp["k_scale"], inp["v_scale"], num_q_heads=w.num_q_heads)
    else:
        def append():
            b.gqa_kv_append(inp["kv"], k_new, v_new, slots, inp["k_scale"], inp["v_scale"])
    for _ in range(3):
        append()
    a_begin, a_end = _event(stream), _event(stream)
    torch.cuda.synchronize()
    a_begin.record(stream)
    for _ in range(K):
        append()
    a_end.record(stream)
    torch.cuda.synchronize()
    append_us = round(a_begin.elapsed_time(a_end) / K * 1e3, 2)

    # Cold-cache calls: a 512 MiB write evicts the caches before each timed call.
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cold = []
    for _ in range(args.cold_calls):
        flush.fill_(1)
        e0, e1 = _event(stream), _event(stream)
        e0.record(stream)
        case.step()
        e1.record(stream)
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1) * 1e3)
    del flush
    cold.sort()

    # Last, as it leaves the device mostly idle: the runtime's own cost per
    # graph launch (a graph of two one-block fill kernels).
    _marker(dev, 106)
    floor = time_graph_floor(dev, max(K, 48), stream)

    def pct(xs, p):
        return xs[min(len(xs) - 1, int(round(p / 100 * (len(xs) - 1))))] if xs else None

    if paged:
        kernel = "gqa_paged_balanced_kernel" if plan["route"] == 2 else "gqa_paged_attention_kernel"
    else:
        kernel = "gqa_balanced_attention_kernel" if plan["route"] == 2 else "gqa_attention_kernel"
    traffic = read_traffic(kernel, w.name, args.num_splits) if not args.fused_combine else None
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"fp8_e4m3": "fp8_e4m3->bf16", "int8": f"int8+bf16 row scales->{w.q_dtype}"}
                 .get(w.kv_dtype, w.kv_dtype),
        "data": "synthetic",
        "config": {**w.describe(), **({"page_order": args.page_order} if paged else {}),
                   **({"scales_by_position": True} if args.scales_by_position else {}),
                   "seq_lens_sum": int(sum(lens)),
                   "algorithmic_bytes_per_step": nbytes, "plan": plan},
        "pct_of_peak": round(100 * value / PEAK_HBM_GBPS, 2),
        "us_per_call": round(ms_per_step * 1e3, 2),
        "us_per_call_graph_replay": round(g1[0], 2),
        "us_per_step_graph_16step": round(g16[0], 2),
        "graph_launch_floor": {"us_per_replay": round(floor[0], 2),
                               "host_us_per_replay": round(floor[1], 2),
                               "graph": "two one-block fill kernels"},
        "us_per_call_convenience": round(convenience_us, 2),
        "us_per_call_cold": {"p10": round(pct(cold, 10), 2), "p50": round(pct(cold, 50), 2),
                             "p90": round(pct(cold, 90), 2)} if cold else None,
        "kv_append_us": append_us,
        "kernels_us": {"attention_avg": round(attn_avg * 1e3, 2),
                       "attention_min": round(min(attn_ms) * 1e3, 2),
                       "combine_avg": round(statistics.fmean(comb_ms) * 1e3, 2)},
        "roofline": {
            "bound": "hbm",
            "kernel": kernel,
            "achieved": round(achieved, 2),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBPS, 4),
            "traffic": traffic,
        },
        "configs": configs,
        "wall_s_timed": round(wall, 4),
        "device": arch,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = (cpu_baseline_paged if paged else cpu_baseline)(inp, w,
                                                                                args.cpu_seconds)
    case.destroy()
    return result


if __name__ == "__main__":
    main()
