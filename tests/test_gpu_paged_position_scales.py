"""GPU parity of INT8 page pools whose row scales are indexed by position
([batch, 2, 8, max_pages * page_size], GQA_PAGED_SCALES_BY_POSITION) against
the paged oracle, on every route and page size; bit equality with the pool
layout on the same data; the append into that layout, byte for byte."""

import numpy as np
import pytest
import torch

from gpu_util import Workload, binding, compare_paged, run_paged, require_gpu
from gqa_kv_cache_attn_amd.inputs import make_paged_inputs, position_scales, storage_bits
from oracle.paged import kv_append_paged_int8_reference

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()


def _w(qd="bf16", hq=16, T=2, C=1000, B=5, P=16, seed=401, q_scale=0.75):
    return Workload(f"paged_pos_{qd}_{hq}q_T{T}_P{P}_C{C}", B, C, T, C, qd, "int8",
                    q_scale=q_scale, k_scale=0.5, v_scale=2.0, seed=seed, num_q_heads=hq,
                    page_size=P, q_tokens=T)


def _both_layouts(w, lens):
    """The same draw twice: row scales in the pool layout and by position."""
    lens = torch.tensor(lens, dtype=torch.int32)
    page = make_paged_inputs(w, device="cuda", seq_lens=lens)
    pos = dict(page)
    pos["kv_scales"] = position_scales(page["kv_scales"], page["block_table"], w.page_size)
    pos["scales_by_position"] = True
    return page, pos


@pytest.mark.parametrize("qd,hq,T", [("bf16", 16, 2), ("f16", 16, 8), ("bf16", 32, 3),
                                      ("f16", 32, 1)])
@pytest.mark.parametrize("P", [16, 32, 64, 128])
@pytest.mark.parametrize("num_splits", [None, 1, 3])
def test_position_scales_parity_and_bit_equality_with_the_pool_layout(qd, hq, T, P, num_splits):
    w = _w(qd, hq, T, P=P, seed=400 + P + T)
    page, pos = _both_layouts(w, [T, 17 + T, 64, 999, 1000])
    out_pos, prep = run_paged(pos, "prepared", num_splits=num_splits)
    if num_splits is not None:
        assert prep.plan["num_splits"] == num_splits
    compare_paged(out_pos, pos, range(w.batch), f"{w.name}/S={num_splits}")
    out_page, _ = run_paged(page, "prepared", num_splits=num_splits)
    assert torch.equal(out_pos.view(torch.int16), out_page.view(torch.int16)), \
        "the two scale layouts must give the same bits"


@pytest.mark.parametrize("case", ["fewer_slabs_than_workgroups", "one_long_head", "mixed_with_empty"])
@pytest.mark.parametrize("P", [16, 32, 256])
def test_position_scales_balanced_partitions(case, P):
    T = 2
    if case == "fewer_slabs_than_workgroups":
        B, C, lens = 6, 4096, [T, 65, 200, 17 + T, 128, 129]
    elif case == "one_long_head":
        B, C, lens = 1, 70000, [69999]
    else:
        B, C, lens = 7, 5000, [0, 4999, T, 0, 5000, 2500, 64]
    w = _w("bf16", 16, T, C=C, B=B, P=P, seed=430 + len(case) + P)
    page, pos = _both_layouts(w, lens)
    out = torch.full_like(pos["q"], float("nan"))
    out, prep = run_paged(pos, "prepared", out=out)
    assert prep.plan["route"] == 2
    compare_paged(out, pos, [i for i, L in enumerate(lens) if L > 0], f"position scales/{case}")
    got = out.float().cpu().numpy()
    for i, L in enumerate(lens):
        if L == 0:
            assert np.all(got[i] == 0), i
    out_page, _ = run_paged(page, "prepared")
    assert torch.equal(out.view(torch.int16), out_page.view(torch.int16))


@pytest.mark.parametrize("num_splits", [None, 1, 4])
@pytest.mark.parametrize("P", [16, 64])
def test_position_scales_past_each_length_are_never_read(num_splits, P):
    """NaN row scales at every position at or past a request's length, and
    NaN-making codes in every page no request uses."""
    w = _w("bf16", 16, 2, C=8192, B=4, P=P, seed=465)
    lens = [2, 3000, 5001, 8191]
    _, pos = _both_layouts(w, lens)
    pool, table, sc = pos["kv_pages"], pos["block_table"], pos["kv_scales"]
    used = torch.zeros(pool.shape[0], dtype=torch.bool, device="cuda")
    for b, L in enumerate(lens):
        used[table[b, :-(-L // P)].long()] = True
        sc[b, :, :, L:] = float("nan")
    pool[~used] = 127
    out, _ = run_paged(pos, "prepared", num_splits=num_splits)
    compare_paged(out, pos, range(4), f"position scales nan past L, P={P}, S={num_splits}")


def test_position_scales_convenience_call_and_workload_shape():
    """The convenience entry point, and the 128k INT8 workload's geometry with
    16-slot pages (every (request, KV head) pair of the first request)."""
    w = _w("bf16", 16, 2, C=131072, B=2, P=16, seed=470)
    _, pos = _both_layouts(w, [131072, 70001])
    out, _ = run_paged(pos, "convenience")
    compare_paged(out, pos, [1], "position scales, 128k capacity, 16-slot pages")


@pytest.mark.parametrize("P,T", [(16, 1), (16, 3), (64, 4)])
def test_position_scale_append_matches_the_oracle_byte_for_byte(P, T):
    """gqa_kv_append_paged_int8 with scales by position: codes in the pages and
    scales at [b, plane, g, slot], including a token that crosses a page, one
    whose slot lies past the table and one whose entry lies outside the pool
    (neither writes anything)."""
    b = binding()
    rng = np.random.default_rng(480 + P + T)
    B, max_pages, num_pages = 4, 3, 14
    codes = torch.tensor(rng.integers(-127, 128, size=(num_pages, 2, 8, P, 128)), dtype=torch.int8,
                         device="cuda")
    sc = torch.tensor(rng.integers(0, 1 << 15, size=(B, 2, 8, max_pages * P)).astype(np.int16),
                      device="cuda").view(torch.bfloat16)
    table_np = np.array([[3, 7, 1], [0, -1, 2], [4, num_pages, 6], [8, 9, 11]], dtype=np.int32)
    table = torch.tensor(table_np, device="cuda")
    pos_np = np.array([P - 1, P - 2, 2 * P - 1, 3 * P - 2], dtype=np.int32)
    positions = torch.tensor(pos_np, device="cuda")
    k = torch.randn(B, T, 8, 128, device="cuda").to(torch.bfloat16)
    v = torch.randn(B, T, 8, 128, device="cuda").to(torch.bfloat16)
    want_c, want_s = kv_append_paged_int8_reference(
        storage_bits(codes), storage_bits(sc), table_np, pos_np, k.float().cpu().numpy(),
        v.float().cpu().numpy(), 0.25, 4.0, scales_by_position=True)
    b.gqa_kv_append_paged_int8(codes, sc, table, k, v, positions, 0.25, 4.0, num_q_heads=16,
                               scales_by_position=True)
    torch.cuda.synchronize()
    assert np.array_equal(storage_bits(codes), want_c)
    assert np.array_equal(storage_bits(sc), want_s)


def test_position_scale_append_then_decode_matches_the_oracle():
    """Append T new tokens to a position-scale pool, then decode them: the
    verify pass reads the rows and scales just written."""
    T, P = 3, 16
    w = _w("bf16", 16, T, C=1024, B=3, P=P, seed=490)
    start = [40, 500, 1021 - T + 1]
    _, pos = _both_layouts(w, [s + T for s in start])
    k = torch.randn(3, T, 8, 128, device="cuda").to(torch.bfloat16)
    v = torch.randn(3, T, 8, 128, device="cuda").to(torch.bfloat16)
    binding().gqa_kv_append_paged_int8(
        pos["kv_pages"], pos["kv_scales"], pos["block_table"], k, v,
        torch.tensor(start, dtype=torch.int32, device="cuda"), 1.0, 1.0, num_q_heads=16,
        scales_by_position=True)
    out, _ = run_paged(pos, "prepared")
    compare_paged(out, pos, range(3), "position scales: append then verify")


def test_position_scales_graph_replay_with_rewritten_lengths():
    """A captured prepared step over a position-scale pool, replayed after
    the lengths change; every replay equals the eager call on the same state."""
    b = binding()
    w = _w("bf16", 16, 2, C=4096, B=3, P=16, seed=495)
    _, pos = _both_layouts(w, [4096, 3000, 2])
    out = torch.empty_like(pos["q"])
    prep = b.prepare_gqa_decode_paged(pos["q"], pos["kv_pages"], pos["block_table"],
                                      pos["seq_lens"], out, pos["q_scale"],
                                      k_scale=pos["k_scale"], v_scale=pos["v_scale"],
                                      kv_scales=pos["kv_scales"], scales_by_position=True)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        b.launch_gqa_decode_prepared(prep)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        b.launch_gqa_decode_prepared(prep)
    for lens in ([4096, 3000, 2], [17, 4000, 64], [2, 2, 4095]):
        pos["seq_lens"].copy_(torch.tensor(lens, dtype=torch.int32))
        g.replay()
        torch.cuda.synchronize()
        replayed = out.clone()
        b.launch_gqa_decode_prepared(prep)
        torch.cuda.synchronize()
        assert torch.equal(replayed.view(torch.int16), out.view(torch.int16)), lens
        compare_paged(out, pos, range(3), f"position scales graph replay {lens}")
    del g
    prep.destroy()
