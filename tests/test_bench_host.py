"""Host logic of bench.py (no GPU): the one-GPU refusal, the algorithmic-byte
count behind every GB/s and roofline figure (checked against hand-computed
totals), the traffic lookup that reports HBM bytes only while the profiled
kernel source is unchanged, and the validation of workload overrides."""

import argparse
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("kv_dtype,kv_bytes", [
    # 3 valid slots x 8 KV heads x (K + V) rows of 128 elements
    ("bf16", 3 * 8 * 2 * 128 * 2),
    ("f16", 3 * 8 * 2 * 128 * 2),
    ("fp8_e4m3", 3 * 8 * 2 * 128 * 1),
    ("int8", 3 * 8 * 2 * (128 * 1 + 2)),   # int8 rows plus one bf16 scale per row
])
def test_algorithmic_bytes_by_hand(kv_dtype, kv_bytes):
    q_and_out = 2 * 32 * 128 * (2 + 2)      # batch 2, 32 query heads, 16-bit q and out
    lens = 2 * 4
    assert bench.algorithmic_bytes([1, 2], kv_dtype, 2) == kv_bytes + q_and_out + lens


def test_algorithmic_bytes_of_a_paged_verify_step():
    # 2 requests of 17 and 16 slots in 16-slot pages: 2 + 1 table entries;
    # 3 query tokens at 16 query heads; an int8 pool with its row scales.
    kv = (17 + 16) * 8 * 2 * (128 + 2)
    q_and_out = 2 * 3 * 16 * 128 * 4
    got = bench.algorithmic_bytes([17, 16], "int8", 2, num_q_heads=16, q_tokens=3, page_size=16)
    assert got == kv + q_and_out + 2 * 4 + 3 * 4


def test_the_headline_figure_counts_only_valid_prefixes():
    # Padding past a length is not counted: doubling the capacity changes nothing.
    assert bench.algorithmic_bytes([65536, 131072], "fp8_e4m3", 2) == \
        (65536 + 131072) * 8 * 256 + 2 * 32 * 128 * 4 + 8


def _traffic_file(directory, digest, splits=0, nbytes=123456789):
    path = os.path.join(directory, "k_w_traffic.txt")
    with open(path, "w") as f:
        f.write("# summary\n")
        f.write(f"kernel_source_sha256_16 = {digest}\n")
        f.write(f"num_splits_requested = {splits}\n")
        f.write(f"hbm_bytes_per_launch = {nbytes}\n")
    return path


def test_traffic_is_reported_only_for_the_profiled_source(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_digest", lambda kernel: "abcdef0123456789")
    assert bench.read_traffic("k", "w", 0) is None                 # no summary file
    _traffic_file(tmp_path, "abcdef0123456789")
    assert bench.read_traffic("k", "w", 0) == 123456789
    assert bench.read_traffic("k", "w", 4) is None                 # profiled with another split
    _traffic_file(tmp_path, "0000000000000000")
    assert bench.read_traffic("k", "w", 0) is None                 # kernel source changed since


def test_the_committed_headline_traffic_matches_the_current_kernels():
    """The headline's traffic summary was taken on the kernels as they are now;
    a kernel change has to be followed by new FETCH/WRITE passes."""
    got = bench.read_traffic("gqa_balanced_attention_kernel", bench.DEFAULT_WORKLOAD, 0)
    assert got is not None and got > 3_300_000_000


def _args(**kw):
    base = dict(shape="", scales_by_position=False, page_size=0, q_tokens=0, page_order="random")
    base.update(kw)
    return argparse.Namespace(**base)


def test_workload_overrides_are_validated():
    with pytest.raises(SystemExit) as e:
        bench._workload(_args(scales_by_position=True), bench.DEFAULT_WORKLOAD)
    assert e.value.code == 2
    with pytest.raises(SystemExit) as e:
        bench._workload(_args(page_size=32), bench.DEFAULT_WORKLOAD)
    assert e.value.code == 2
    w = bench._workload(_args(shape="2,4096,100,4096"), bench.DEFAULT_WORKLOAD)
    assert (w.batch, w.capacity, w.len_lo, w.len_hi) == (2, 4096, 100, 4096)
    paged = "gqa_decode_paged_b16_c131072_p64_int8kv_16q_t2"
    w = bench._workload(_args(page_size=16, q_tokens=3, scales_by_position=True), paged)
    assert (w.page_size, w.q_tokens) == (16, 3) and "scales by position" in w.name
