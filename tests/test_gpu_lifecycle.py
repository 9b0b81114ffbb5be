"""GPU lifecycle of the prepared API: hipGraph capture and replay with lengths
rewritten in place, the convenience call's refusal to allocate inside a
capture, two handles on concurrent streams, guard bands, error paths that
must leave the output untouched, and the timed launch."""

import pytest
import torch

from gpu_util import Workload, all_pairs, binding, compare, make_inputs, oracle_pairs, prepare
from gpu_util import require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()


def _inputs(B=4, C=4096, qd="bf16", kd="bf16", seed=31, hq=32):
    fp8 = kd == "fp8_e4m3"
    w = Workload(f"life_{qd}_{kd}", B, C, 1, C, qd, kd, q_scale=0.9,
                 k_scale=1 / 64 if fp8 else 1.0, v_scale=1 / 64 if fp8 else 1.0, seed=seed,
                 num_q_heads=hq)
    return make_inputs(w, device="cuda")


def _prepare(inp, out, num_splits=None, fused_combine=False):
    return prepare(inp, out, num_splits, fused_combine)


@pytest.mark.parametrize("kd,hq", [("bf16", 32), ("fp8_e4m3", 32), ("int8", 16)])
@pytest.mark.parametrize("plan", ["balanced", "chunked", "fused"])
def test_graph_replay_with_rewritten_lengths_matches_direct_launch(kd, hq, plan):
    b = binding()
    inp = _inputs(kd=kd, hq=hq)
    out = torch.empty_like(inp["q"])
    prep = _prepare(inp, out, num_splits=None if plan == "balanced" else 8,
                    fused_combine=plan == "fused")
    assert prep.plan["route"] == (2 if plan == "balanced" else 1) and prep.workspace_bytes > 0
    lens = inp["seq_lens"]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        b.launch_gqa_decode_prepared(prep)          # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        b.launch_gqa_decode_prepared(prep)

    # Long, then shrinking, then growing lengths: stale partials must never leak.
    schedule = [[4096, 4096, 4096, 4096], [4000, 1, 2049, 63], [17, 16, 15, 1],
                [1, 2, 3, 4], [4096, 777, 64, 65], [2048, 2048, 2048, 2048]]
    for new in schedule:
        lens.copy_(torch.tensor(new, dtype=torch.int32))
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        replayed = out.clone()
        # eager work between replays, then a direct launch with the same lengths
        out.fill_(float("nan"))
        b.launch_gqa_decode_prepared(prep)
        torch.cuda.synchronize()
        assert torch.equal(replayed.view(torch.int16), out.view(torch.int16)), new
    compare(replayed, oracle_pairs(inp, all_pairs(4)), inp, f"graph replay {kd}")
    del graph
    prep.destroy()


def test_convenience_call_refuses_to_allocate_inside_capture():
    b = binding()
    inp = _inputs(B=2, C=4096)
    out = torch.empty_like(inp["q"])
    plan = b.gqa_plan(b.make_desc(inp["q"], inp["kv"]))
    assert plan["workspace_bytes"] > 0
    x = torch.zeros(4, device="cuda")
    stream = torch.cuda.Stream()   # no convenience call has used this pooled stream yet
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        with pytest.raises(b.GqaError) as ei:
            b.gqa_decode(inp["q"], inp["kv"], inp["seq_lens"], inp["q_scale"], out)
        x.add_(1.0)
    assert ei.value.status == b.GQA_ERR_CAPTURE
    graph.replay()
    torch.cuda.synchronize()
    assert torch.all(x == 1.0)


def test_convenience_call_under_capture_takes_two_launches_when_counters_are_dirty():
    """A small problem's automatic plan merges in one launch, which needs its
    per-head counters at zero. When an earlier, larger plan left partials in
    the stream's cached workspace, clearing them inside a capture would record
    a memset, so the captured call takes the two-launch merge instead of
    failing; its replays equal the eager one-launch result bit for bit."""
    b = binding()
    big = _inputs(B=8, C=8192, seed=61)
    small = _inputs(B=1, C=1024, seed=62)
    assert b.gqa_plan(b.make_desc(small["q"], small["kv"]))["fused_merge"] == 1
    out_big, eager, replayed = (torch.empty_like(x["q"]) for x in (big, small, small))
    stream = torch.cuda.Stream()
    # torch's pooled streams do not wait for the default stream, where the
    # inputs were just drawn
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        b.gqa_decode(big["q"], big["kv"], big["seq_lens"], big["q_scale"], out_big)
        b.gqa_decode(small["q"], small["kv"], small["seq_lens"], small["q_scale"], eager)
        # the small call cleared its counters; the big one dirties them again
        b.gqa_decode(big["q"], big["kv"], big["seq_lens"], big["q_scale"], out_big)
    stream.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        b.gqa_decode(small["q"], small["kv"], small["seq_lens"], small["q_scale"], replayed)
    for _ in range(3):
        replayed.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(replayed.view(torch.int16), eager.view(torch.int16))
    compare(replayed, oracle_pairs(small, all_pairs(1)), small, "captured convenience, small")
    del graph


def test_two_handles_on_two_concurrent_streams():
    b = binding()
    inp1 = _inputs(seed=41)
    inp2 = _inputs(seed=42, kd="fp8_e4m3")
    o1, o2 = torch.empty_like(inp1["q"]), torch.empty_like(inp2["q"])
    p1, p2 = _prepare(inp1, o1), _prepare(inp2, o2)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    for _ in range(5):
        with torch.cuda.stream(s1):
            b.launch_gqa_decode_prepared(p1)
        with torch.cuda.stream(s2):
            b.launch_gqa_decode_prepared(p2)
    torch.cuda.synchronize()
    compare(o1, oracle_pairs(inp1, all_pairs(4)), inp1, "stream 1")
    compare(o2, oracle_pairs(inp2, all_pairs(4)), inp2, "stream 2")


@pytest.mark.parametrize("num_splits", [None, 1])
def test_output_guard_bands_are_untouched(num_splits):
    inp = _inputs(B=3, C=1000, qd="f16", kd="f16")
    n = inp["q"].numel()
    pad = 4096
    buf = torch.full((n + 2 * pad,), 12345.0, dtype=torch.float16, device="cuda")
    out = buf[pad:pad + n].view_as(inp["q"])
    prep = _prepare(inp, out, num_splits)
    binding().launch_gqa_decode_prepared(prep)
    torch.cuda.synchronize()
    assert torch.all(buf[:pad] == 12345.0) and torch.all(buf[pad + n:] == 12345.0)
    compare(out, oracle_pairs(inp, all_pairs(3)), inp, "guard bands")


def test_invalid_calls_enqueue_nothing_and_leave_out_untouched():
    b = binding()
    inp = _inputs(B=2, C=512)
    out = torch.full_like(inp["q"], 7.0)
    with pytest.raises(ValueError):
        b.gqa_decode(inp["q"], inp["kv"], inp["seq_lens"], 0.0, out)
    with pytest.raises(ValueError):
        b.gqa_decode(inp["q"], inp["kv"], inp["seq_lens"], float("nan"), out)
    with pytest.raises(ValueError):
        b.prepare_gqa_decode(inp["q"], inp["kv"], inp["seq_lens"], out, num_splits=31)
    with pytest.raises(ValueError):   # out aliases q
        b.prepare_gqa_decode(inp["q"], inp["kv"], inp["seq_lens"], inp["q"])
    with pytest.raises(ValueError):   # a scale on a 16-bit cache is rejected, not ignored
        b.gqa_decode(inp["q"], inp["kv"], inp["seq_lens"], 1.0, out, k_scale=0.5)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)


def test_int8_entry_points_reject_mismatches_and_aliases():
    b = binding()
    inp = _inputs(B=2, C=512, kd="int8", hq=16)
    out = torch.full_like(inp["q"], 7.0)
    with pytest.raises(ValueError):   # an INT8 cache needs its row scales
        b.gqa_decode(inp["q"], inp["kv"], inp["seq_lens"], 1.0, out)
    with pytest.raises(ValueError):
        b.prepare_gqa_decode(inp["q"], inp["kv"], inp["seq_lens"], out)
    alias = inp["kv_scales"].view(-1)[:out.numel()].view_as(out)
    before = alias.clone()
    with pytest.raises(ValueError):   # out overlapping kv_scales
        b.gqa_decode_int8(inp["q"], inp["kv"], inp["kv_scales"], inp["seq_lens"], 1.0, alias)
    with pytest.raises(ValueError):   # scales of the wrong shape
        b.gqa_decode_int8(inp["q"], inp["kv"], inp["kv_scales"][:, :, :, :100].contiguous(),
                          inp["seq_lens"], 1.0, out)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
    assert torch.equal(alias.view(torch.int16), before.view(torch.int16))


def test_convenience_calls_with_different_plans_share_the_workspace_safely():
    """Back-to-back convenience calls on one stream whose plans lay the cached
    workspace out differently (batch, capacity, route): each result matches the
    oracle, so no plan starts from control words another plan left dirty."""
    from gpu_util import run_decode
    cases = [(32, 4096, "bf16"), (4, 8192, "bf16"), (32, 4096, "bf16"), (3, 1000, "f16"),
             (8, 2048, "fp8_e4m3")]
    for i, (B, C, kd) in enumerate(cases):
        qd = "f16" if kd == "f16" else "bf16"
        fp8 = kd == "fp8_e4m3"
        w = Workload(f"reuse{i}", B, C, 1, C, qd, kd, q_scale=0.8,
                     k_scale=1 / 64 if fp8 else 1.0, v_scale=1 / 64 if fp8 else 1.0, seed=60 + i)
        inp = make_inputs(w, device="cuda")
        out, _ = run_decode(inp, "convenience")
        pairs = all_pairs(B) if B <= 8 else [(b, (3 * b) % 8) for b in range(B)]
        compare(out, oracle_pairs(inp, pairs), inp, f"workspace reuse {i} (B={B}, C={C}, {kd})")


@pytest.mark.parametrize("kd,hq,B,C,one_per_cu", [
    ("bf16", 32, 1, 65536, True),        # a single request
    ("int8", 16, 1, 16384, True),
    ("bf16", 32, 16, 4096, True),        # 256 MiB of K+V at capacity
    ("fp8_e4m3", 32, 1, 65536, False),   # fp8 keeps the resident grid
    ("bf16", 32, 8, 32768, False),       # 512 MiB at capacity
])
def test_balanced_grid_follows_the_problem_size(kd, hq, B, C, one_per_cu):
    """prepare sizes the balanced grid for the device: one workgroup per CU for
    small 16-bit / INT8 problems, every resident slot otherwise; both give the
    oracle's result."""
    inp = _inputs(B=B, C=C, kd=kd, hq=hq, seed=40 + B)
    out = torch.full_like(inp["q"], float("nan"))
    prep = _prepare(inp, out)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    W = prep.plan["num_workgroups"]
    assert prep.plan["route"] == 2
    if one_per_cu:
        assert W == cus, (W, cus)
    else:
        assert W > cus and W % cus == 0, (W, cus)
    binding().launch_gqa_decode_prepared(prep)
    torch.cuda.synchronize()
    pairs = [(b, g) for b in range(B) for g in range(8)][:16]
    compare(out, oracle_pairs(inp, pairs), inp, f"grid {W} {kd} B={B} C={C}")
    prep.destroy()


@pytest.mark.parametrize("plan", ["balanced", "chunked", "one_launch", "paged"])
def test_timed_launch_gives_the_same_bits_with_its_events_in_order(plan):
    """launch_gqa_decode_prepared_timed, which bench times the attention kernel
    with: the same output as the plain launch, bit for bit; its three events
    recorded in stream order (start, after the attention kernel, end); and any
    of them may be left out."""
    from gqa_kv_cache_attn_amd.inputs import make_paged_inputs
    b = binding()
    if plan == "paged":
        w = Workload("life_timed_paged", 3, 4096, 1, 4096, "bf16", "bf16", q_scale=0.8, seed=77,
                     page_size=16, q_tokens=2)
        inp = make_paged_inputs(w, device="cuda")
        out = torch.full_like(inp["q"], float("nan"))
        prep = b.prepare_gqa_decode_paged(inp["q"], inp["kv_pages"], inp["block_table"],
                                          inp["seq_lens"], out, inp["q_scale"])
    else:
        inp = _inputs(B=1, C=1024, seed=78) if plan == "one_launch" else _inputs(seed=79)
        out = torch.full_like(inp["q"], float("nan"))
        prep = _prepare(inp, out, num_splits=8 if plan == "chunked" else None)
    want_route = {"balanced": 2, "chunked": 1, "one_launch": 1, "paged": 2}[plan]
    assert prep.plan["route"] == want_route
    assert prep.plan["fused_merge"] == (1 if plan == "one_launch" else 0)
    b.launch_gqa_decode_prepared(prep)
    torch.cuda.synchronize()
    plain = out.clone()
    out.fill_(float("nan"))
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    for e in evs:
        e.record()                                 # creates the underlying HIP event
    b.launch_gqa_decode_prepared_timed(prep, *evs)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), plain.view(torch.int16))
    t_att, t_rest = evs[0].elapsed_time(evs[1]), evs[1].elapsed_time(evs[2])
    assert t_att > 0 and t_rest >= 0, (t_att, t_rest)
    for left_out in range(3):
        out.fill_(float("nan"))
        b.launch_gqa_decode_prepared_timed(prep, *[None if i == left_out else e
                                                   for i, e in enumerate(evs)])
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), plain.view(torch.int16)), left_out
    prep.destroy()
