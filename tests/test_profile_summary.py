"""Host logic of the rocprofv3 summariser (no GPU; synthetic rows): splitting a
kernel trace of a bench run into its measurement passes, turning FETCH_SIZE /
WRITE_SIZE readings into bytes by the copy of known size, the busy-cycle
ratios of the counter summaries, and the source digest that ties a summary to
the kernels it was taken on."""

import csv
import types

import pytest

from gqa_kv_cache_attn_amd import profile_summary as ps

FIELDS = ["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X"]
ATT = "void gqa::(anonymous namespace)::gqa_balanced_attention_kernel<1, 1, 4>(gqa::StepArgs)"
COMB = "void gqa::(anonymous namespace)::gqa_balanced_combine_kernel<1, 4>(gqa::StepArgs)"
FILL = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<float>>"
MARK = ("void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda("
        "at::TensorIteratorBase&)::{lambda()#1}::operator()() const::{lambda(float)#1}>")


def _trace(tmp_path, rows):
    path = tmp_path / "trace.csv"
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for name, start, end, grid in rows:
            w.writerow({"Kernel_Name": name, "Start_Timestamp": start, "End_Timestamp": end,
                        "Grid_Size_X": grid})
    return str(path)


def _steps(t0, n, att_ns, comb_ns, gap_ns):
    """n decode steps from t0: attention, gap, combine, gap."""
    rows, t = [], t0
    for _ in range(n):
        rows.append((ATT, t, t + att_ns, 131072))
        t += att_ns + gap_ns
        rows.append((COMB, t, t + comb_ns, 32768))
        t += comb_ns + gap_ns
    return rows, t


def _args(trace, names, out):
    return types.SimpleNamespace(trace=trace, names=names, title="t", command="c", out=str(out),
                                 kernel="gqa_balanced_attention_kernel", marker="neg_kernel")


def test_phases_splits_at_markers_only(tmp_path):
    rows = [("void at::native::distribution_elementwise_grid_stride_kernel", 0, 10, 10 ** 7)]
    steps, t = _steps(100, 3, 1000, 100, 0)      # before the first marker: dropped
    rows += steps
    rows.append((MARK, t + 10, t + 20, 256))
    steps, t = _steps(t + 100, 4, 2000, 200, 50)
    rows += steps
    rows.append((MARK, t + 10, t + 20, 256))      # then a pass with no decode kernel
    rows.append((FILL, t + 30, t + 40, 64))
    rows.append((MARK, t + 50, t + 60, 256))
    # A graph replay's own small fills between steps do not split the pass.
    steps, t = _steps(t + 100, 1, 3000, 300, 100)
    rows += steps
    rows.append((FILL, t + 10, t + 20, 256))
    rows.append((FILL, t + 30, t + 40, 256))
    steps, t = _steps(t + 100, 1, 3000, 300, 100)
    rows += steps
    # A cold call: a large fill (not a marker) before each step.
    rows.append((FILL, t + 10, t + 5000, 10 ** 8))
    steps, t = _steps(t + 6000, 1, 3000, 300, 100)
    rows += steps
    out = tmp_path / "phases.txt"
    ps.cmd_phases(_args(_trace(tmp_path, rows), "first,second", out))
    text = out.read_text()
    lines = [ln for ln in text.splitlines() if ln.startswith("| first") or ln.startswith("| second")]
    first = [c.strip() for c in lines[0].split("|")[1:-1]]
    second = [c.strip() for c in lines[1].split("|")[1:-1]]
    assert first[:4] == ["first", "4", "2.00", "0.20"]
    assert first[4] == "0.05" and first[5] == "0.05"
    assert first[6] == "2.30"                     # start to start: 2000 + 50 + 200 + 50 ns
    assert second[:4] == ["second", "3", "3.00", "0.30"]


def test_phases_rejects_a_name_count_that_does_not_match(tmp_path):
    rows = [(MARK, 0, 10, 256)]
    steps, _ = _steps(100, 2, 1000, 100, 0)
    rows += steps
    with pytest.raises(SystemExit, match="1 passes"):
        ps.cmd_phases(_args(_trace(tmp_path, rows), "a,b", tmp_path / "x.txt"))


# ------------------------------------------------------------------ traffic
CNT_FIELDS = ["Kernel_Name", "Counter_Name", "Counter_Value"]
COPY = ("void at::native::vectorized_elementwise_kernel<4, at::native::bitwise_not_kernel_cuda"
        "(at::TensorIteratorBase&)::{lambda(unsigned char)#1}>")


def _counters(tmp_path, name, rows):
    path = tmp_path / name
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=CNT_FIELDS)
        w.writeheader()
        for kernel, counter, value in rows:
            w.writerow({"Kernel_Name": kernel, "Counter_Name": counter, "Counter_Value": value})
    return str(path)


def _read_kv(path):
    kv = {}
    for line in open(path):
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    return kv


def test_traffic_scales_each_counter_by_the_copy_of_known_size(tmp_path):
    # The copy reads and writes 1 GiB and the counters read 2^19 and 2^20
    # units: 2048 bytes per FETCH unit, 1024 per WRITE unit. The attention
    # kernel's two dispatches average 1000 and 10 units; the combine kernel,
    # whose name shares a suffix, must not be counted.
    gib = 1 << 30
    fetch = _counters(tmp_path, "f.csv", [(ATT, "FETCH_SIZE", 900), (ATT, "FETCH_SIZE", 1100),
                                          (COMB, "FETCH_SIZE", 10 ** 9)])
    write = _counters(tmp_path, "w.csv", [(ATT, "WRITE_SIZE", 10), (ATT, "WRITE_SIZE", 10),
                                          (COMB, "WRITE_SIZE", 10 ** 9)])
    cf = _counters(tmp_path, "cf.csv", [(COPY, "FETCH_SIZE", 1 << 19)])
    cw = _counters(tmp_path, "cw.csv", [(COPY, "WRITE_SIZE", 1 << 20)])
    out = tmp_path / "t.txt"
    ps.cmd_traffic(types.SimpleNamespace(
        fetch=fetch, write=write, copy_fetch=cf, copy_write=cw, copy_bytes=gib, copy_match="bitwise_not",
        algorithmic_bytes=2_000_000, num_splits=0, kernel="gqa_balanced_attention_kernel",
        workload="w", command="c", out=str(out)))
    kv = _read_kv(out)
    assert kv["fetch_bytes_per_launch"] == str(1000 * 2048)
    assert kv["write_bytes_per_launch"] == str(10 * 1024)
    assert kv["hbm_bytes_per_launch"] == str(1000 * 2048 + 10 * 1024)
    assert kv["fetch_over_algorithmic"] == "1.0240"
    assert kv["kernel_source_sha256_16"] == ps.kernel_source_digest("gqa_balanced_attention_kernel")


def test_traffic_refuses_a_run_without_the_kernel(tmp_path):
    fetch = _counters(tmp_path, "f.csv", [(COMB, "FETCH_SIZE", 5)])
    with pytest.raises(SystemExit, match="no dispatch"):
        ps._counter_avg(fetch, "::gqa_balanced_attention_kernel<")
    # The chunked kernel's name is not a match for the balanced one, nor the reverse.
    assert "::gqa_attention_kernel<" not in ATT


def test_counters_ratios(tmp_path):
    # 8 XCDs x 1000 cycles; 1024 SIMDs; MFMA busy 102400 cycles -> 10%;
    # VALU active 51200 quad-cycles -> 20%.
    rows = [(ATT, "GRBM_GUI_ACTIVE", 8000), (ATT, "SQ_VALU_MFMA_BUSY_CYCLES", 102400),
            (ATT, "SQ_ACTIVE_INST_VALU", 51200), (ATT, "SQ_INSTS_VALU", 640),
            (COMB, "SQ_INSTS_VALU", 10 ** 9)]
    out = tmp_path / "c.txt"
    ps.cmd_counters(types.SimpleNamespace(
        csv=[_counters(tmp_path, "c.csv", rows)], kernel="gqa_balanced_attention_kernel",
        elements=6400, cus=256, xcds=8, clock_ghz=2.4, title="t", command="c", out=str(out)))
    text = out.read_text()
    assert "MFMA busy: 10.00%" in text
    assert "VALU active: 20.00%" in text
    assert "VALU instructions per 1000 KV elements: 100.000 (per lane-element: 6.400)" in text


# ------------------------------------------------------------------- digest
def test_the_digest_ignores_comments_and_whitespace_only():
    a = 'int f(int x) {\n  // add one\n  return x + 1; /* done */\n}\nconst char* s = "a // b";\n'
    b = 'int f(int x){return x+1;}\n// another comment\nconst char* s = "a // b";'
    c = 'int f(int x){return x+2;}\nconst char* s = "a // b";'
    d = 'int f(int x){return x+1;}\nconst char* s = "a  // b";'
    assert ps._code_only(a) == ps._code_only(b)
    assert ps._code_only(a) != ps._code_only(c)          # code changed
    assert ps._code_only(a) != ps._code_only(d)          # a string literal is code
    assert ps._code_only('x = "\\"//"; y') == 'x="\\"//";y'
