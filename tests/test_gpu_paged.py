"""GPU parity of the paged entry points (page pool + block table, T query tokens
per request, causal among themselves) against the paged oracle, on every
route, dtype pair and geometry, plus the special cases of the layout."""

import dataclasses

import numpy as np
import pytest
import torch

from gpu_util import (
    Workload,
    binding,
    compare_paged,
    decoded_out,
    out_ulp,
    paged_oracle_request,
    require_gpu,
    run_decode,
    run_paged,
)
from gqa_kv_cache_attn_amd.inputs import PAGED_WORKLOADS, make_inputs, make_paged_inputs, storage_bits
from oracle import decode_int8_rows, decode_storage, gqa_decode_head

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()


# (q dtype, kv dtype, query heads, query tokens)
PCASES = [("bf16", "bf16", 32, 3), ("f16", "f16", 32, 4), ("bf16", "fp8_e4m3", 32, 2),
          ("f16", "fp8_e4m3", 32, 1), ("bf16", "int8", 16, 8), ("f16", "int8", 16, 3),
          ("bf16", "bf16", 16, 1), ("bf16", "int8", 32, 4)]
PIDS = [f"{q}-{k}-{h}q-T{t}" for q, k, h, t in PCASES]


def _pw(qd, kd, hq, T, C=1000, B=5, P=16, seed=201, q_scale=0.75):
    fp8 = kd == "fp8_e4m3"
    ks, vs = (1 / 64, 1 / 32) if fp8 else ((0.5, 2.0) if kd == "int8" else (1.0, 1.0))
    return Workload(f"paged_{qd}_{kd}_{hq}q_T{T}_P{P}_C{C}", B, C, T, C, qd, kd, q_scale=q_scale,
                    k_scale=ks, v_scale=vs, seed=seed, num_q_heads=hq, page_size=P, q_tokens=T)


@pytest.mark.parametrize("qd,kd,hq,T", PCASES, ids=PIDS)
@pytest.mark.parametrize("P", [16, 64])
@pytest.mark.parametrize("num_splits", [None, 1, 3])
def test_paged_parity_on_every_route(qd, kd, hq, T, P, num_splits):
    w = _pw(qd, kd, hq, T, P=P, seed=200 + P + T)
    lens = torch.tensor([T, 17 + T, 64, 999, 1000], dtype=torch.int32)
    inp = make_paged_inputs(w, device="cuda", seq_lens=lens)
    out, prep = run_paged(inp, "prepared", num_splits=num_splits)
    if num_splits is not None:
        assert prep.plan["num_splits"] == num_splits
    compare_paged(out, inp, range(w.batch), f"{w.name}/S={num_splits}")


@pytest.mark.parametrize("qd,kd,hq,T", PCASES, ids=PIDS)
@pytest.mark.parametrize("case", ["fewer_slabs_than_workgroups", "one_long_head", "mixed_with_empty"])
@pytest.mark.parametrize("P", [32, 64])
def test_paged_balanced_split_partitions(qd, kd, hq, T, case, P):
    _balanced_partition_case(qd, kd, hq, T, case, P)


@pytest.mark.parametrize("qd,T", [("bf16", 2), ("f16", 5)])
@pytest.mark.parametrize("case", ["fewer_slabs_than_workgroups", "one_long_head", "mixed_with_empty"])
@pytest.mark.parametrize("P", [16, 32, 128, 256])
def test_paged_int8_block_order(qd, T, case, P):
    """int8 pools walk 64-slot blocks on the balanced route: within one page
    (128, 256) or across the 4 or 2 pages a block spans (16, 32)."""
    _balanced_partition_case(qd, "int8", 16, T, case, P)


def _balanced_partition_case(qd, kd, hq, T, case, P):
    if case == "fewer_slabs_than_workgroups":
        B, C, lens = 6, 4096, [T, 65, 200, 17 + T, 128, 129]
    elif case == "one_long_head":
        B, C, lens = 1, 70000, [69999]
    else:
        B, C, lens = 7, 5000, [0, 4999, T, 0, 5000, 2500, 64]
    w = _pw(qd, kd, hq, T, C=C, B=B, P=P, seed=230 + len(case) + P)
    inp = make_paged_inputs(w, device="cuda", seq_lens=torch.tensor(lens, dtype=torch.int32))
    out = torch.full_like(inp["q"], float("nan"))
    out, prep = run_paged(inp, "prepared", out=out)
    assert prep.plan["route"] == 2
    got = decoded_out(out, qd)
    for i, L in enumerate(lens):
        if L == 0:
            assert np.all(got[i] == 0), i
    compare_paged(out, inp, [i for i, L in enumerate(lens) if L > 0], f"paged balanced/{case}")


@pytest.mark.parametrize("qd,kd,hq,T", PCASES, ids=PIDS)
def test_paged_short_route(qd, kd, hq, T):
    w = _pw(qd, kd, hq, T, C=64, B=4, P=16, seed=250)
    inp = make_paged_inputs(w, device="cuda", seq_lens=torch.tensor([T, 33, 63, 64], dtype=torch.int32))
    out, prep = run_paged(inp, "prepared")
    assert prep.plan["route"] == 0 and prep.workspace_bytes == 0
    compare_paged(out, inp, range(4), w.name)


@pytest.mark.parametrize("kd", ["bf16", "fp8_e4m3", "int8"])
@pytest.mark.parametrize("num_splits", [None, 1, 4])
@pytest.mark.parametrize("P", [32, 128])
def test_paged_garbage_outside_the_prefix_is_never_read(kd, num_splits, P):
    """NaN in every page no request uses, and in every slot past a length."""
    hq = 16 if kd == "int8" else 32
    w = _pw("bf16", kd, hq, 2, C=700, B=4, P=P, seed=260)
    lens = torch.tensor([2, 250, 333, 699], dtype=torch.int32)
    inp = make_paged_inputs(w, device="cuda", seq_lens=lens)
    pool, table = inp["kv_pages"], inp["block_table"]
    used = torch.zeros(pool.shape[0], dtype=torch.bool, device="cuda")
    nan = {"fp8_e4m3": 0x7F, "int8": 127}.get(kd, float("nan"))
    for b, L in enumerate(lens.tolist()):
        n = -(-L // P)
        used[table[b, :n].long()] = True
        last = int(table[b, n - 1])
        if L % P:
            pool[last, :, :, L % P:] = nan
            if kd == "int8":
                inp["kv_scales"][last, :, :, L % P:] = float("nan")
    pool[~used] = nan
    if kd == "int8":
        inp["kv_scales"][~used] = float("nan")
    out, _ = run_paged(inp, "prepared", num_splits=num_splits)
    compare_paged(out, inp, range(4), f"paged nan-garbage {kd}")


@pytest.mark.parametrize("P", [16, 32, 64])
def test_paged_int8_balanced_route_never_reads_past_the_prefix(P):
    """The balanced route over an int8 pool: NaN codes and NaN row scales in
    every unused page and every slot past a length (the block order's scale
    loads must read 0 there, not the pool's other rows)."""
    w = _pw("bf16", "int8", 16, 2, C=8192, B=4, P=P, seed=265)
    lens = torch.tensor([2, 3000, 5001, 8191], dtype=torch.int32)
    inp = make_paged_inputs(w, device="cuda", seq_lens=lens)
    pool, table, sc = inp["kv_pages"], inp["block_table"], inp["kv_scales"]
    used = torch.zeros(pool.shape[0], dtype=torch.bool, device="cuda")
    for b, L in enumerate(lens.tolist()):
        n = -(-L // P)
        used[table[b, :n].long()] = True
        last = int(table[b, n - 1])
        if L % P:
            pool[last, :, :, L % P:] = 127
            sc[last, :, :, L % P:] = float("nan")
    pool[~used] = 127
    sc[~used] = float("nan")
    out, prep = run_paged(inp, "prepared")
    assert prep.plan["route"] == 2
    compare_paged(out, inp, range(4), f"paged int8 balanced nan-garbage P={P}")


@pytest.mark.parametrize("num_splits", [None, 1, 2])
def test_tokens_that_see_no_slot_get_zeros(num_splits):
    """L < T: token t sees L - T + 1 + t slots; tokens with none give zeros."""
    T = 4
    w = _pw("f16", "f16", 32, T, C=300, B=3, P=16, seed=270)
    lens = torch.tensor([1, 3, 300], dtype=torch.int32)
    inp = make_paged_inputs(w, device="cuda", seq_lens=lens)
    out = torch.full_like(inp["q"], float("nan"))
    out, _ = run_paged(inp, "prepared", num_splits=num_splits, out=out)
    got = decoded_out(out, "f16")
    full = paged_oracle_request(inp, 2)
    assert np.all(np.abs(got[2] - full) - 0.5 * out_ulp(full, "f16") <= 2e-3)
    for b, L in enumerate([1, 3]):
        pages = inp["kv_pages"].index_select(0, inp["block_table"][b, :1].long())
        kv = pages[0].double().cpu().numpy()           # the request's first page, [2, 8, 16, 128]
        q = inp["q"][b].double().cpu().numpy()
        for t in range(T):
            visible = L - T + 1 + t
            if visible <= 0:
                assert np.all(got[b, t] == 0), (b, t)
                continue
            for g in range(8):
                ref = gqa_decode_head(q[t, 4 * g:4 * g + 4], kv[0, g, :visible], kv[1, g, :visible],
                                      inp["q_scale"])
                err = np.abs(got[b, t, 4 * g:4 * g + 4] - ref) - 0.5 * out_ulp(ref, "f16")
                assert err.max() <= 2e-3, (b, t, g)


def test_paged_equals_the_contiguous_entry_point_on_an_identity_table():
    """A contiguous cache is the pool with page_size = capacity and table [b]."""
    C, B = 256, 3
    w = Workload("contig", B, C, 1, C, "bf16", "bf16", q_scale=0.6, seed=280)
    inp = make_inputs(w, device="cuda")
    ref, _ = run_decode(inp, "prepared", num_splits=4)
    b = binding()
    out = torch.empty_like(inp["q"]).unsqueeze(1)
    table = torch.arange(B, dtype=torch.int32, device="cuda").view(B, 1)
    prep = b.prepare_gqa_decode_paged(inp["q"].unsqueeze(1), inp["kv"], table, inp["seq_lens"], out,
                                      0.6, num_splits=4)
    b.launch_gqa_decode_prepared(prep)
    torch.cuda.synchronize()
    # same chunks, same merge order: the two paths agree bit for bit
    assert torch.equal(out[:, 0].view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("P", [16, 64])
def test_pages_in_pool_order_give_the_same_result_as_shuffled_pages(P):
    """The same logical cache under the drawn (shuffled) table and with every
    request's pages moved into pool order: the kernel sees the same rows in the
    same slots, so the two outputs agree bit for bit (and with the oracle)."""
    b = binding()
    w = _pw("bf16", "bf16", 32, 3, C=8192, B=4, P=P, seed=285)
    inp = make_paged_inputs(w, device="cuda")
    table = inp["block_table"]
    B, max_pages = table.shape
    ordered = torch.arange(B * max_pages, dtype=torch.int32, device="cuda").view(B, max_pages)
    pool_ordered = torch.empty_like(inp["kv_pages"])
    pool_ordered[ordered.view(-1).long()] = inp["kv_pages"][table.view(-1).long()]
    outs = []
    for pool, tab in ((inp["kv_pages"], table), (pool_ordered, ordered)):
        out = torch.empty_like(inp["q"])
        prep = b.prepare_gqa_decode_paged(inp["q"], pool, tab, inp["seq_lens"], out,
                                          inp["q_scale"])
        assert prep.plan["route"] == 2   # the balanced split, as the bench workload takes
        b.launch_gqa_decode_prepared(prep)
        torch.cuda.synchronize()
        outs.append(out)
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    compare_paged(outs[1], inp, [0, B - 1], f"{w.name}/pool order")


@pytest.mark.parametrize("plan", ["balanced", "chunked"])
def test_paged_graph_replay_with_rewritten_lengths_and_pages(plan):
    b = binding()
    w = _pw("bf16", "fp8_e4m3", 32, 3, C=4096, B=4, P=16, seed=290)
    inp = make_paged_inputs(w, device="cuda")
    out = torch.empty_like(inp["q"])
    prep = b.prepare_gqa_decode_paged(inp["q"], inp["kv_pages"], inp["block_table"],
                                      inp["seq_lens"], out, inp["q_scale"],
                                      num_splits=None if plan == "balanced" else 8,
                                      k_scale=inp["k_scale"], v_scale=inp["v_scale"])
    assert prep.plan["route"] == (2 if plan == "balanced" else 1)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        b.launch_gqa_decode_prepared(prep)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        b.launch_gqa_decode_prepared(prep)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(291)
    for new in ([4096, 4096, 4096, 4096], [4000, 3, 2049, 63], [17, 16, 15, 3], [4096, 777, 64, 65]):
        inp["seq_lens"].copy_(torch.tensor(new, dtype=torch.int32))
        # move every page to a new id and rewrite the table to match
        perm = torch.randperm(inp["kv_pages"].shape[0], generator=gen, device="cuda")
        moved = torch.empty_like(inp["kv_pages"])
        moved[perm] = inp["kv_pages"]
        inp["kv_pages"].copy_(moved)
        inp["block_table"].copy_(perm[inp["block_table"].long()].to(torch.int32))
        del moved
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        replayed = out.clone()
        out.fill_(float("nan"))
        b.launch_gqa_decode_prepared(prep)
        torch.cuda.synchronize()
        assert torch.equal(replayed.view(torch.int16), out.view(torch.int16)), new
    compare_paged(replayed, inp, range(4), f"paged graph replay {plan}")
    del graph
    prep.destroy()


@pytest.mark.parametrize("w", PAGED_WORKLOADS, ids=[w.name for w in PAGED_WORKLOADS])
def test_paged_workload_parity(w):
    print(f"[case] {w.name}", flush=True)
    inp = make_paged_inputs(w, device="cuda")
    out_c, _ = run_paged(inp, "convenience")
    out_p, prep = run_paged(inp, "prepared")
    print(f"[plan] {prep.plan}", flush=True)
    assert torch.equal(out_c.view(torch.int16), out_p.view(torch.int16))
    compare_paged(out_c, inp, [0, w.batch - 1], w.name)


def test_paged_argument_errors_enqueue_nothing():
    b = binding()
    w = _pw("bf16", "int8", 16, 2, C=256, B=2, P=16, seed=300)
    inp = make_paged_inputs(w, device="cuda")
    out = torch.full_like(inp["q"], 7.0)
    args = (inp["q"], inp["kv_pages"], inp["block_table"], inp["seq_lens"])
    with pytest.raises(ValueError):   # an int8 pool needs its row scales
        b.gqa_decode_paged(*args, 1.0, out)
    with pytest.raises(ValueError):   # page size not a power of two
        b.gqa_decode_paged(inp["q"], inp["kv_pages"][:, :, :, :12].contiguous(), inp["block_table"],
                           inp["seq_lens"], 1.0, out, kv_scales=inp["kv_scales"][..., :12].contiguous())
    q9 = torch.zeros(2, 9, 16, 128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):   # 9 tokens x 2 heads per KV head > 16 MFMA rows
        b.gqa_decode_paged(q9, *args[1:], 1.0, torch.empty_like(q9), kv_scales=inp["kv_scales"])
    alias = inp["kv_scales"].view(-1)[:out.numel()].view_as(out)
    with pytest.raises(ValueError):   # out overlapping the row scales
        b.gqa_decode_paged(*args, 1.0, alias, kv_scales=inp["kv_scales"])
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)


def _head_rows(inp, b, plane, g, L):
    """Decoded fp64 rows [L, 128] of KV head g of request b, gathered page by page
    through the block table."""
    P = inp["page_size"]
    n = -(-L // P)
    ids = inp["block_table"][b, :n].long()
    rows = inp["kv_pages"][:, plane, g].index_select(0, ids).reshape(n * P, -1)[:L]
    if inp["kv_dtype"] == "int8":
        sc = inp["kv_scales"][:, plane, g].index_select(0, ids).reshape(n * P)[:L]
        return decode_int8_rows(storage_bits(rows), storage_bits(sc))
    return decode_storage(storage_bits(rows), inp["kv_dtype"])


@pytest.mark.parametrize("kd,hq,T,P", [("bf16", 32, 1, 16), ("int8", 16, 2, 64)])
def test_paged_maximum_capacity_every_slot_valid(kd, hq, T, P):
    """A request as long as the largest accepted capacity (2^22 slots) in a
    shuffled pool: 262144 pages of 16 slots (bf16, a 16 GiB pool) or 65536 of 64
    (INT8, the block order), so page offsets pass 2^31 bytes. A large q_scale
    (4; 8 for INT8, whose k_scale here is 0.5) concentrates the weights on a
    few dozen slots spread over the range.
    Oracle: the contiguous definition on the head's rows gathered through the
    table, each token with its causal prefix."""
    C = 1 << 22
    w = _pw("bf16", kd, hq, T, C=C, B=1, P=P, seed=2424, q_scale=8.0 if kd == "int8" else 4.0)
    inp = make_paged_inputs(w, device="cuda", seq_lens=torch.tensor([C], dtype=torch.int32))
    G = hq // 8
    q = decode_storage(storage_bits(inp["q"][0]), "bf16")          # [T, Hq, 128]
    refs = {}
    for g in (0, 7):
        k, v = _head_rows(inp, 0, 0, g, C), _head_rows(inp, 0, 1, g, C)
        refs[g] = np.stack([gqa_decode_head(q[t, G * g:G * g + G], k[:C - T + 1 + t],
                                            v[:C - T + 1 + t], inp["q_scale"], inp["k_scale"],
                                            inp["v_scale"]) for t in range(T)])
        del k, v
    for ns in (None, 64):
        out = torch.full_like(inp["q"], float("nan"))
        out, prep = run_paged(inp, "prepared", num_splits=ns, out=out)
        assert prep.plan["route"] == (2 if ns is None else 1)
        got = decoded_out(out, "bf16")[0]
        for g, ref in refs.items():
            err = np.abs(got[:, G * g:G * g + G] - ref)
            assert np.all(np.isfinite(err)), (g, ns)
            assert (err - 0.5 * out_ulp(ref, "bf16")).max() <= 2e-3, (g, ns, err.max())
        print(f"[parity] paged max capacity {kd} P={P} T={T} S={ns}: "
              f"max_abs_ref={max(np.abs(r).max() for r in refs.values()):.3e}", flush=True)
        prep.destroy()
    del inp
    torch.cuda.empty_cache()


def test_paged_batch_of_4096_requests():
    """The most requests the paged balanced split takes (one LDS prefix entry per
    request), with ragged lengths and two query tokens."""
    B = 4096
    w = _pw("bf16", "bf16", 32, 2, C=256, B=B, P=16, seed=4096)
    lens = torch.randint(2, 257, (B,), generator=torch.Generator().manual_seed(7), dtype=torch.int32)
    inp = make_paged_inputs(w, device="cuda", seq_lens=lens)
    out = torch.full_like(inp["q"], float("nan"))
    out, prep = run_paged(inp, "prepared", out=out)
    assert prep.plan["route"] == 2
    compare_paged(out, inp, list(range(0, B, 211)) + [B - 1], "paged batch 4096")
    assert torch.isfinite(out.float()).all()
    prep.destroy()
