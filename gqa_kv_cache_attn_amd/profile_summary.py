"""Summarise rocprofv3 CSV output into the short text files kept under profiles/.

    python -m gqa_kv_cache_attn_amd.profile_summary stats  --csv K_kernel_stats.csv \\
        --title T --command "C" --out profiles/X.txt
    python -m gqa_kv_cache_attn_amd.profile_summary traffic --workload W \\
        --fetch F_counter_collection.csv --write W_counter_collection.csv \\
        --copy-fetch CF.csv --copy-write CW.csv --copy-bytes N \\
        --algorithmic-bytes A --command "C" --out profiles/gqa_attention_kernel_W_traffic.txt
    python -m gqa_kv_cache_attn_amd.profile_summary counters --csv A.csv B.csv --elements E \\
        --title T --command "C" --out profiles/X.txt
    python -m gqa_kv_cache_attn_amd.profile_summary phases --trace K_kernel_trace.csv \\
        --names direct,graph1,... --title T --command "C" --out profiles/X.txt
    python -m gqa_kv_cache_attn_amd.profile_summary calibrate [--gib 1] [--iters 3]   (GPU)

`traffic` scales each counter by what it reads for a plain elementwise pass
of known size (`calibrate`: torch's bitwise_not over a 1 GiB uint8 tensor
into another, N bytes read, N bytes written per launch), so counter units
become bytes. It records the kernel-source digest the counters were taken
with, and bench.py only reports the figure while that digest still matches
the source.

`phases` splits a kernel trace of a bench.py run at the marker kernels bench
places between its measurement passes (a negation of a 256-element tensor) and
reports, per pass, the decode kernels' average durations, the gaps between
consecutive kernels and the time per step.
"""

from __future__ import annotations

import argparse
import csv
import hashlib
import os
import statistics

from .build import CSRC

COPY_MATCH = "bitwise_not"


# Sources each kernel family is compiled from (the digest covers all of them).
_SOURCES = {
    "contiguous": ("gqa_kernels.h", "gqa_device.h", "gqa_kernels.hip"),
    "paged": ("gqa_kernels.h", "gqa_device.h", "gqa_paged.hip"),
}


def _code_only(text: str) -> str:
    """Source text without comments and whitespace (string literals kept as
    they are), so an edit to comments alone leaves the digest unchanged."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        elif c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            if not c.isspace():
                out.append(c)
            i += 1
    return "".join(out)


def kernel_source_digest(kernel: str = "gqa_balanced_attention_kernel") -> str:
    """Digest of the code (comments and whitespace left out) of the sources
    the named kernel is built from."""
    h = hashlib.sha256()
    for name in _SOURCES["paged" if "paged" in kernel else "contiguous"]:
        with open(os.path.join(CSRC, name), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def _counter_avg(path, match):
    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(path)) if match in r["Kernel_Name"]]
    if not vals:
        raise SystemExit(f"no dispatch of {match} in {path}")
    return statistics.fmean(vals), len(vals)


def cmd_stats(a):
    rows = list(csv.DictReader(open(a.csv)))
    lines = [f"# {a.title}", "", f"command: {a.command}", "",
             "| kernel | calls | avg us | min us | max us | share % |", "|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"]
        if a.only_gqa and "gqa" not in name:
            continue
        lines.append(f"| `{name[:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.2f} |")
    lines.append("")
    lines.append(f"kernel_source_sha256_16 = {kernel_source_digest(a.kernel)}")
    with open(a.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cmd_traffic(a):
    match = f"::{a.kernel}<"            # exact kernel name within the demangled signature
    fetch, nf = _counter_avg(a.fetch, match)
    write, nw = _counter_avg(a.write, match)
    cfetch, _ = _counter_avg(a.copy_fetch, a.copy_match)
    cwrite, _ = _counter_avg(a.copy_write, a.copy_match)
    fscale = a.copy_bytes / cfetch          # bytes per FETCH_SIZE unit
    wscale = a.copy_bytes / cwrite          # bytes per WRITE_SIZE unit
    fb, wb = fetch * fscale, write * wscale
    lines = [
        f"# HBM traffic per launch of the attention kernel ({a.kernel}), workload {a.workload}",
        "#",
        f"# command (FETCH_SIZE pass; WRITE_SIZE pass identical but for the counter): {a.command}",
        f"# calibration: {a.copy_match} reads and writes {a.copy_bytes} bytes per launch; it reads "
        f"FETCH_SIZE={cfetch:.1f} and WRITE_SIZE={cwrite:.1f}",
        f"# -> {fscale:.4f} bytes per FETCH_SIZE unit, {wscale:.4f} bytes per WRITE_SIZE unit",
        f"# dispatches averaged: fetch {nf}, write {nw}",
        f"workload = {a.workload}",
        f"num_splits_requested = {a.num_splits}",
        f"fetch_size_raw = {fetch:.3f}",
        f"write_size_raw = {write:.3f}",
        f"fetch_bytes_per_launch = {fb:.0f}",
        f"write_bytes_per_launch = {wb:.0f}",
        f"hbm_bytes_per_launch = {fb + wb:.0f}",
        f"algorithmic_bytes_per_launch = {a.algorithmic_bytes}",
        f"fetch_over_algorithmic = {fb / a.algorithmic_bytes:.4f}",
        f"kernel_source_sha256_16 = {kernel_source_digest(a.kernel)}",
    ]
    with open(a.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cmd_phases(a):
    rows = sorted(csv.DictReader(open(a.trace)), key=lambda r: int(r["Start_Timestamp"]))
    # Passes: runs of decode kernels between marker kernels (bench places a
    # marker before each pass). Other kernels (input generation) are dropped.
    # A marker is the negation kernel bench launches between passes (torch's
    # graph replays launch small fills of their own, so fills cannot mark).
    # Passes with no decode kernel (the graph-launch floor) are dropped.
    passes, cur, seen_marker = [], [], False
    for r in rows:
        name = r["Kernel_Name"]
        if "gqa" in name and "append" not in name:
            if seen_marker:
                cur.append(r)
        elif a.marker in name:
            if cur:
                passes.append(cur)
            cur, seen_marker = [], True
    if cur:
        passes.append(cur)
    names = a.names.split(",")
    if len(names) != len(passes):
        raise SystemExit(f"{len(passes)} passes with decode kernels in the trace, {len(names)} names given")
    us = lambda r: (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    lines = [f"# {a.title}", "", f"command: {a.command}", "",
             "| pass | steps | attention avg us | combine avg us | gap attention->combine us "
             "(median) | gap combine->next attention us (median) | us per step (median start "
             "to start) |",
             "|---|---|---|---|---|---|---|"]
    for name, p in zip(names, passes):
        att = [r for r in p if "combine" not in r["Kernel_Name"]]
        com = [r for r in p if "combine" in r["Kernel_Name"]]
        g_ac, g_ca = [], []
        for x, y in zip(p, p[1:]):
            gap = (int(y["Start_Timestamp"]) - int(x["End_Timestamp"])) / 1e3
            (g_ac if "combine" in y["Kernel_Name"] else g_ca).append(gap)
        starts = [int(r["Start_Timestamp"]) for r in att]
        step = [(y - x) / 1e3 for x, y in zip(starts, starts[1:])]
        f = lambda xs: f"{statistics.fmean(xs):.2f}" if xs else "-"
        m = lambda xs: f"{statistics.median(xs):.2f}" if xs else "-"
        lines.append(f"| {name} | {len(att)} | {f([us(r) for r in att])} | {f([us(r) for r in com])} "
                     f"| {m(g_ac)} | {m(g_ca)} | {m(step)} |")
    lines.append("")
    lines.append(f"kernel_source_sha256_16 = {kernel_source_digest(a.kernel)}")
    with open(a.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _counters_by_name(path, match):
    """{counter name: mean per dispatch} over the dispatches of the matching kernel."""
    acc = {}
    for r in csv.DictReader(open(path)):
        if match in r["Kernel_Name"]:
            acc.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    return {k: statistics.fmean(v) for k, v in acc.items()}


def cmd_counters(a):
    """Instruction and busy-cycle counters of one kernel, with the ratios that
    say how much of the matrix and vector units the kernel keeps busy."""
    match = f"::{a.kernel}<"
    vals = {}
    for path in a.csv:
        vals.update(_counters_by_name(path, match))
    if not vals:
        raise SystemExit(f"no dispatch of {a.kernel} in {a.csv}")
    lines = [f"# {a.title}", "", f"command: {a.command}", "",
             f"kernel: {a.kernel}; counters averaged per dispatch; {a.elements} KV elements "
             f"(valid K and V values) per launch", "",
             "| counter | per launch |", "|---|---|"]
    for k in sorted(vals):
        lines.append(f"| {k} | {vals[k]:.6g} |")
    lines.append("")
    simds = a.cus * 4
    gui = vals.get("GRBM_GUI_ACTIVE")
    if gui:
        # GRBM_GUI_ACTIVE is summed over the XCDs; each counts the kernel's cycles.
        cycles = gui / a.xcds
        lines.append(f"GPU-busy cycles per XCD: {cycles:.6g} ({cycles / (a.clock_ghz * 1e3):.1f} us at "
                     f"{a.clock_ghz} GHz)")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in vals:
            lines.append(f"MFMA busy: {100 * vals['SQ_VALU_MFMA_BUSY_CYCLES'] / (cycles * simds):.2f}% "
                         f"of the {simds} SIMDs' cycles")
        if "SQ_ACTIVE_INST_VALU" in vals:
            # quad-cycles, summed over waves; at most `waves per SIMD` waves issue per SIMD
            lines.append(f"VALU active: {100 * 4 * vals['SQ_ACTIVE_INST_VALU'] / (cycles * simds):.2f}% "
                         f"of the SIMDs' cycles (summed over waves)")
    e = a.elements
    for k, label in (("SQ_INSTS_VALU", "VALU"), ("SQ_INSTS_MFMA", "MFMA"), ("SQ_INSTS_VMEM_RD", "VMEM read"),
                     ("SQ_INSTS_LDS", "LDS"), ("SQ_INSTS_SALU", "SALU")):
        if k in vals:
            lines.append(f"{label} instructions per 1000 KV elements: {1000 * vals[k] / e:.3f} "
                         f"(per lane-element: {vals[k] * 64 / e:.3f})")
    lines.append("")
    lines.append(f"kernel_source_sha256_16 = {kernel_source_digest(a.kernel)}")
    with open(a.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cmd_calibrate(a):
    """The calibration pass the traffic summaries scale by (run under
    rocprofv3 --pmc): torch's bitwise_not over an N GiB uint8 tensor into
    another, `iters` times, so each launch reads and writes N GiB."""
    import torch
    n = a.gib << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(0x5A)
    dst = torch.empty_like(src)
    for _ in range(a.iters):
        torch.bitwise_not(src, out=dst)
    torch.cuda.synchronize()
    assert int(dst[0]) == 0xA5 and int(dst[-1]) == 0xA5
    print(f"bitwise_not over {n} bytes x {a.iters}")


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("--csv", required=True)
    s.add_argument("--title", required=True)
    s.add_argument("--command", required=True)
    s.add_argument("--out", required=True)
    s.add_argument("--only-gqa", action="store_true")
    s.add_argument("--kernel", default="gqa_balanced_attention_kernel",
                   help="kernel whose source digest is recorded")
    t = sub.add_parser("traffic")
    for k in ("workload", "fetch", "write", "copy_fetch", "copy_write", "command", "out"):
        t.add_argument("--" + k.replace("_", "-"), required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--algorithmic-bytes", type=int, required=True)
    t.add_argument("--num-splits", type=int, default=0)
    t.add_argument("--kernel", default="gqa_balanced_attention_kernel")
    t.add_argument("--copy-match", default=COPY_MATCH,
                   help="substring naming the calibration kernel in the copy runs")
    ph = sub.add_parser("phases")
    for k in ("trace", "names", "title", "command", "out"):
        ph.add_argument("--" + k, required=True)
    ph.add_argument("--kernel", default="gqa_balanced_attention_kernel")
    ph.add_argument("--marker", default="neg_kernel",
                    help="substring naming the marker kernel between passes")
    c = sub.add_parser("counters")
    c.add_argument("--csv", nargs="+", required=True)
    for k in ("title", "command", "out"):
        c.add_argument("--" + k, required=True)
    c.add_argument("--kernel", default="gqa_balanced_attention_kernel")
    c.add_argument("--elements", type=int, required=True, help="valid K and V values per launch")
    c.add_argument("--cus", type=int, default=256)
    c.add_argument("--xcds", type=int, default=8)
    c.add_argument("--clock-ghz", type=float, default=2.4)
    k = sub.add_parser("calibrate")
    k.add_argument("--gib", type=int, default=1)
    k.add_argument("--iters", type=int, default=3)
    a = ap.parse_args()
    {"stats": cmd_stats, "traffic": cmd_traffic, "phases": cmd_phases,
     "counters": cmd_counters, "calibrate": cmd_calibrate}[a.cmd](a)


if __name__ == "__main__":
    main()
