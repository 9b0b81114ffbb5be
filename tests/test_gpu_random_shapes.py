"""Seeded random sweep of decode shapes against the fp64 oracle: dtype pairs,
32 or 16 query heads, batch, capacity, length range, automatic or explicit
splits and the one-launch merge over a contiguous cache, and page size,
query tokens and both INT8 scale layouts over a page pool. Every case is a
pure function of its index, printed before it runs; every output row of
every request is compared, at the bound the hand-written cases use."""

import numpy as np
import pytest
import torch

from gpu_util import (Workload, all_pairs, binding, compare, compare_paged, make_inputs,
                      oracle_pairs, require_gpu, run_decode, run_paged)

pytestmark = pytest.mark.gpu

CAPACITIES = [17, 64, 65, 100, 640, 1000, 2049, 4096, 8191]
KV_FOR = {"f16": ["f16", "fp8_e4m3", "int8"], "bf16": ["bf16", "fp8_e4m3", "int8"]}


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()


def _scales(rng, kd):
    if kd == "fp8_e4m3":
        return float(rng.choice([1 / 64, 1 / 16, 0.5])), float(rng.choice([1 / 64, 1 / 8, 1.0]))
    if kd == "int8":
        return float(rng.choice([0.5, 1.0, 2.0])), float(rng.choice([0.25, 1.0, 3.0]))
    return 1.0, 1.0


def _honoured(plan_fn, desc, num_splits):
    """num_splits if the plan honours it, else None (the automatic plan)."""
    try:
        plan_fn(desc, num_splits)
        return num_splits
    except ValueError:
        return None


def contiguous_case(i):
    rng = np.random.default_rng(9000 + i)
    qd = str(rng.choice(["f16", "bf16"]))
    kd = str(rng.choice(KV_FOR[qd]))
    hq = int(rng.choice([32, 16]))
    B = int(rng.integers(1, 7))
    C = int(rng.choice(CAPACITIES))
    lo = int(rng.integers(1, C + 1))
    hi = int(rng.integers(lo, C + 1))
    ks, vs = _scales(rng, kd)
    w = Workload(f"rand{i}", B, C, lo, hi, qd, kd, q_scale=float(rng.uniform(0.3, 2.0)),
                 k_scale=ks, v_scale=vs, seed=9100 + i, num_q_heads=hq)
    mode = str(rng.choice(["auto", "splits", "fused"]))
    splits = int(rng.choice([2, 3, 5, 8, 13])) if mode != "auto" else None
    return w, mode, splits


def paged_case(i):
    rng = np.random.default_rng(9500 + i)
    qd = str(rng.choice(["f16", "bf16"]))
    kd = str(rng.choice(KV_FOR[qd]))
    hq = int(rng.choice([32, 16]))
    G = hq // 8
    T = int(rng.integers(1, 16 // G + 1))
    P = int(rng.choice([16, 32, 64, 128, 256]))
    B = int(rng.integers(1, 6))
    max_pages = int(rng.integers(1, 4097 // P + 2))
    C = max_pages * P
    lo = int(rng.integers(T, C + 1))
    hi = int(rng.integers(lo, C + 1))
    ks, vs = _scales(rng, kd)
    w = Workload(f"rand_paged{i}", B, C, lo, hi, qd, kd, q_scale=float(rng.uniform(0.3, 2.0)),
                 k_scale=ks, v_scale=vs, seed=9600 + i, num_q_heads=hq, page_size=P, q_tokens=T)
    by_position = kd == "int8" and bool(rng.integers(0, 2))
    splits = int(rng.choice([2, 4, 7])) if rng.integers(0, 3) == 0 else None
    return w, by_position, splits


@pytest.mark.parametrize("i", range(96))
def test_random_contiguous_shape_matches_the_oracle(i):
    w, mode, splits = contiguous_case(i)
    print(f"[case] contiguous {i}: {w} mode={mode} splits={splits}", flush=True)
    b = binding()
    inp = make_inputs(w, device="cuda")
    desc = b.make_desc(inp["q"], inp["kv"], inp["k_scale"], inp["v_scale"],
                       fused_combine=mode == "fused")
    splits = _honoured(b.gqa_plan, desc, splits) if splits else None
    out = torch.full_like(inp["q"], float("nan"))
    out, prep = run_decode(inp, "prepared", num_splits=splits, out=out,
                           fused_combine=mode == "fused")
    print(f"[plan] {prep.plan}", flush=True)
    if splits is not None:
        assert prep.plan["num_splits"] == splits
    compare(out, oracle_pairs(inp, all_pairs(w.batch)), inp, f"random contiguous {i}")
    prep.destroy()


@pytest.mark.parametrize("i", range(48))
def test_random_paged_shape_matches_the_oracle(i):
    from gqa_kv_cache_attn_amd.inputs import make_paged_inputs
    w, by_position, splits = paged_case(i)
    print(f"[case] paged {i}: {w} by_position={by_position} splits={splits}", flush=True)
    b = binding()
    inp = make_paged_inputs(w, device="cuda", scales_by_position=by_position)
    desc = b.make_paged_desc(inp["q"], inp["kv_pages"], inp["block_table"], inp["k_scale"],
                             inp["v_scale"], by_position)
    splits = _honoured(b.gqa_plan_paged, desc, splits) if splits else None
    out = torch.full_like(inp["q"], float("nan"))
    out, prep = run_paged(inp, "prepared", num_splits=splits, out=out)
    print(f"[plan] {prep.plan}", flush=True)
    if splits is not None:
        assert prep.plan["num_splits"] == splits
    compare_paged(out, inp, range(w.batch), f"random paged {i}")
    prep.destroy()
