"""Host logic of the rocprofv3 summariser: splitting a kernel trace of a bench
run into its measurement passes (no GPU; synthetic trace rows)."""

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
