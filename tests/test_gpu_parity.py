"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs, element by element, to the contract tolerance (max-abs
2e-3 for a 16-bit or row-scaled INT8 cache, 2e-2 for fp8_e4m3), plus the exact
special cases. Every case runs at 32 query heads (4 per KV head) and, where
listed, at 16 (2 per KV head)."""

import dataclasses

import numpy as np
import pytest
import torch

from gpu_util import (
    Workload,
    all_pairs,
    compare,
    decoded_out,
    make_inputs,
    oracle_pairs,
    require_gpu,
    run_decode,
)
from gqa_kv_cache_attn_amd.inputs import WORKLOADS
from oracle import decode_e4m3fn_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()


# ------------------------------------------------------------- the five workloads
@pytest.mark.parametrize("w", WORKLOADS, ids=[w.name for w in WORKLOADS])
def test_workload_parity(w):
    print(f"[case] {w.name}", flush=True)
    inp = make_inputs(w, device="cuda")
    out_c, _ = run_decode(inp, "convenience")
    out_p, prep = run_decode(inp, "prepared")
    print(f"[plan] {prep.plan}", flush=True)
    # Every (request, KV head) pair, the full-size long-context workloads
    # included (the oracle decodes fp8 bytes through its 256-entry table).
    refs = oracle_pairs(inp, all_pairs(w.batch))
    compare(out_c, refs, inp, w.name, contract_only=True)
    # Same plan, same kernels: the two entry points agree bit for bit.
    assert torch.equal(out_c.view(torch.int16), out_p.view(torch.int16))


# ------------------------------------------------------------- split / tail coverage
# (q dtype, kv dtype, query heads)
CASES = [("f16", "f16", 32), ("bf16", "bf16", 32), ("bf16", "fp8_e4m3", 32),
         ("f16", "fp8_e4m3", 32), ("bf16", "int8", 16), ("f16", "int8", 16),
         ("bf16", "int8", 32), ("f16", "f16", 16), ("bf16", "fp8_e4m3", 16)]
CASE_IDS = [f"{q}-{k}-{h}q" for q, k, h in CASES]


def _small(qd, kd, C=1000, B=5, seed=77, q_scale=0.75, hq=32):
    fp8 = kd == "fp8_e4m3"
    # an INT8 cache also takes per-tensor scales on top of its row scales
    ks, vs = (1 / 64, 1 / 32) if fp8 else ((0.5, 2.0) if kd == "int8" else (1.0, 1.0))
    return Workload(f"ragged_{qd}_{kd}_{hq}q_C{C}", B, C, 1, C, qd, kd, q_scale=q_scale,
                    k_scale=ks, v_scale=vs, seed=seed, num_q_heads=hq)


@pytest.mark.parametrize("qd,kd,hq", CASES, ids=CASE_IDS)
@pytest.mark.parametrize("num_splits", [None, 1, 2, 3, 7, 9, 63])
def test_split_counts_and_ragged_tails(qd, kd, hq, num_splits):
    w = _small(qd, kd, hq=hq)
    lens = torch.tensor([1, 17, 64, 999, 1000], dtype=torch.int32)
    inp = make_inputs(w, device="cuda", seq_lens=lens)
    out, prep = run_decode(inp, "prepared", num_splits=num_splits)
    if num_splits is not None:
        assert prep.plan["num_splits"] == num_splits
    compare(out, oracle_pairs(inp, all_pairs(w.batch)), inp, f"{w.name}/S={num_splits}")


@pytest.mark.parametrize("qd,kd,hq", CASES, ids=CASE_IDS)
@pytest.mark.parametrize("num_splits", [None, 7, 63])
def test_fused_combine_variant(qd, kd, hq, num_splits):
    """The one-launch variant (last workgroup of a head merges) agrees too."""
    w = _small(qd, kd, seed=78, hq=hq)
    lens = torch.tensor([1000, 999, 1, 64, 65], dtype=torch.int32)
    inp = make_inputs(w, device="cuda", seq_lens=lens)
    out, prep = run_decode(inp, "prepared", num_splits=num_splits, fused_combine=True)
    assert prep.plan["route"] == 1
    compare(out, oracle_pairs(inp, all_pairs(w.batch)), inp, f"{w.name}/fused/S={num_splits}")
    if num_splits is not None:
        sep, _ = run_decode(inp, "prepared", num_splits=num_splits)
        # Same chunk partials, same merge order: identical bits.
        assert torch.equal(out.view(torch.int16), sep.view(torch.int16))


@pytest.mark.parametrize("qd,kd,hq", CASES, ids=CASE_IDS)
@pytest.mark.parametrize("case", ["fewer_slabs_than_workgroups", "one_long_head",
                                  "mixed_with_empty", "many_requests"])
def test_balanced_split_partitions(qd, kd, hq, case):
    """The balanced split covers every head exactly once whatever the mix of
    lengths: heads shorter than a workgroup's share, one head spread over the
    whole grid, empty requests in between, and many short requests."""
    if case == "fewer_slabs_than_workgroups":   # 104 slabs for hundreds of workgroups
        B, C, lens = 6, 4096, [1, 65, 200, 17, 128, 129]
    elif case == "one_long_head":
        B, C, lens = 1, 70000, [69999]
    elif case == "mixed_with_empty":
        B, C, lens = 7, 5000, [0, 4999, 1, 0, 5000, 2500, 64]
    else:
        B, C = 300, 320
        lens = [(37 * i) % 321 for i in range(B)]
    w = _small(qd, kd, C=C, B=B, seed=90 + len(case), hq=hq)
    inp = make_inputs(w, device="cuda", seq_lens=torch.tensor(lens, dtype=torch.int32))
    out = torch.full_like(inp["q"], float("nan"))
    out, prep = run_decode(inp, "prepared", out=out)
    assert prep.plan["route"] == 2
    got = decoded_out(out, qd)
    empty = [i for i, L in enumerate(lens) if L == 0]
    for i in empty:
        assert np.all(got[i] == 0), i
    pairs = [(i, g) for i in range(B) if lens[i] > 0 for g in range(8)]
    if len(pairs) > 240:
        pairs = pairs[::7]
    compare(out, oracle_pairs(inp, pairs), inp, f"balanced/{case}/{qd}/{kd}")


@pytest.mark.parametrize("qd,kd,hq", CASES, ids=CASE_IDS)
@pytest.mark.parametrize("C", [1, 7, 16, 33, 63, 64])
def test_short_route(qd, kd, hq, C):
    w = _small(qd, kd, C=C, B=6, seed=100 + C, hq=hq)
    inp = make_inputs(w, device="cuda")
    out, prep = run_decode(inp, "prepared")
    assert prep.plan["route"] == 0 and prep.workspace_bytes == 0
    compare(out, oracle_pairs(inp, all_pairs(w.batch)), inp, w.name)


# ------------------------------------------------------------- exact special cases
@pytest.mark.parametrize("qd,kd,hq", CASES, ids=CASE_IDS)
@pytest.mark.parametrize("num_splits", [None, 1, 4])
def test_single_token_returns_v_row0_bit_exact(qd, kd, hq, num_splits):
    w = _small(qd, kd, C=256, B=3, seed=5, hq=hq)
    if kd == "int8":   # v_scale 1: v8 * row scale is exact in any output format
        w = dataclasses.replace(w, v_scale=1.0)
    inp = make_inputs(w, device="cuda", seq_lens=torch.ones(3, dtype=torch.int32))
    if kd == "int8":   # row scales of a few bits, so v8 * scale fits an f16 output exactly
        inp["kv_scales"].copy_(torch.ldexp(torch.ones_like(inp["kv_scales"]),
                                           (torch.arange(256, device="cuda") % 5 - 8)
                                           .to(torch.int32).view(1, 1, 1, 256).expand(3, 2, 8, 256))
                               .to(torch.bfloat16))
    out, _ = run_decode(inp, "prepared", num_splits=num_splits)
    got = decoded_out(out, qd)
    refs = oracle_pairs(inp, all_pairs(3))
    G = hq // 8
    for (b, g), ref in refs.items():
        assert np.array_equal(got[b, G * g:G * g + G], ref), (b, g)


@pytest.mark.parametrize("num_splits,fused", [(None, False), (1, False), (None, True)])
def test_zero_and_overlong_lengths(num_splits, fused):
    """Length <= 0 gives zeros; length > capacity behaves as capacity."""
    w = _small("bf16", "bf16", C=512, B=4, seed=9)
    inp = make_inputs(w, device="cuda", seq_lens=torch.tensor([0, -5, 600, 512], dtype=torch.int32))
    out = torch.full_like(inp["q"], float("nan"))
    out, _ = run_decode(inp, "prepared", num_splits=num_splits, out=out, fused_combine=fused)
    got = decoded_out(out, "bf16")
    assert np.all(got[0] == 0) and np.all(got[1] == 0)
    inp_cap = dict(inp, seq_lens=torch.tensor([1, 1, 512, 512], dtype=torch.int32, device="cuda"))
    refs = oracle_pairs(inp_cap, [(b, g) for b in (2, 3) for g in range(8)])
    compare(out, refs, inp, "overlong")


@pytest.mark.parametrize("qd,kd,hq", CASES, ids=CASE_IDS)
@pytest.mark.parametrize("num_splits", [None, 1, 5])
def test_nan_garbage_past_length_is_never_read(qd, kd, hq, num_splits):
    w = _small(qd, kd, C=700, B=4, seed=11, hq=hq)
    lens = torch.tensor([1, 250, 333, 699], dtype=torch.int32)
    inp = make_inputs(w, device="cuda", seq_lens=lens)
    kv = inp["kv"]
    for b, L in enumerate(lens.tolist()):
        if kd == "fp8_e4m3":
            kv[b, :, :, L:] = 0x7F        # e4m3fn NaN
        elif kd == "int8":
            kv[b, :, :, L:] = 127
            inp["kv_scales"][b, :, :, L:] = float("nan")
        else:
            kv[b, :, :, L:] = float("nan")
    out, _ = run_decode(inp, "prepared", num_splits=num_splits)
    compare(out, oracle_pairs(inp, all_pairs(4)), inp, f"nan-garbage {qd}/{kd}")


@pytest.mark.parametrize("kd", ["bf16", "fp8_e4m3", "int8"])
def test_capacity_padding_is_invisible(kd):
    qd = "bf16"
    L = 301
    w = _small(qd, kd, C=L, B=2, seed=13, hq=16 if kd == "int8" else 32)
    tight = make_inputs(w, device="cuda", seq_lens=torch.full((2,), L, dtype=torch.int32))
    wide_kv = torch.empty(2, 2, 8, 4 * L, 128, dtype=tight["kv"].dtype, device="cuda")
    wide_sc = None
    if kd == "fp8_e4m3":
        wide_kv.fill_(0x7F)
    elif kd == "int8":
        wide_kv.fill_(-128)
        wide_sc = torch.full((2, 2, 8, 4 * L), float("nan"), dtype=torch.bfloat16, device="cuda")
        wide_sc[:, :, :, :L] = tight["kv_scales"]
    else:
        wide_kv.fill_(float("nan"))
    wide_kv[:, :, :, :L] = tight["kv"]
    wide = dict(tight, kv=wide_kv, kv_scales=wide_sc)
    out_t, _ = run_decode(tight, "prepared")
    out_w, _ = run_decode(wide, "prepared")
    refs = oracle_pairs(tight, all_pairs(2))
    compare(out_t, refs, tight, "tight")
    compare(out_w, refs, wide, "padded x4 with NaN")


@pytest.mark.parametrize("kd,hq", [("f16", 32), ("fp8_e4m3", 32), ("int8", 16), ("f16", 16)])
def test_head_h_reads_kv_head_h_div_group(kd, hq):
    qd = "f16"
    G = hq // 8
    w = _small(qd, kd, C=200, B=3, seed=15, hq=hq)
    inp = make_inputs(w, device="cuda", seq_lens=torch.tensor([200, 1, 77], dtype=torch.int32))
    for g in range(8):
        if kd == "fp8_e4m3":   # e4m3fn code for g * 32 (value g / v_scale-scaled below)
            code = int(torch.tensor(float(g)).to(torch.float8_e4m3fn).view(torch.uint8))
            inp["kv"][:, 1, g] = code
        elif kd == "int8":     # V = g * 1.0 through the row scale
            inp["kv"][:, 1, g] = g
            inp["kv_scales"][:, 1, g] = 1.0
        else:
            inp["kv"][:, 1, g] = float(g)
    out, _ = run_decode(inp, "prepared", num_splits=3)
    got = decoded_out(out, qd)
    for h in range(hq):
        assert np.all(got[:, h] == (h // G) * inp["v_scale"]), h


def test_identical_keys_average_the_values():
    w = _small("bf16", "bf16", C=4096, B=2, seed=17)
    inp = make_inputs(w, device="cuda", seq_lens=torch.tensor([4096, 1234], dtype=torch.int32))
    inp["kv"][:, 0] = inp["kv"][:, 0, :, :1]
    out, _ = run_decode(inp, "prepared")
    refs = oracle_pairs(inp, all_pairs(2))
    for (b, g), ref in refs.items():
        L = int(inp["seq_lens"][b])
        mean = inp["kv"][b, 1, g, :L].double().mean(0).cpu().numpy()
        np.testing.assert_allclose(ref, np.tile(mean, (4, 1)), rtol=0, atol=1e-12)
    compare(out, refs, inp, "identical keys")


# ------------------------------------------------------------- fp8 decode on the device
@pytest.mark.parametrize("qd", ["bf16", "f16"])
def test_fp8_every_code_decodes_exactly(qd):
    """V row 0 holds all 256 e4m3fn codes; with L = 1 the output is
    v_scale * decode(code) exactly (NaN codes give NaN)."""
    B = 2
    w = Workload("fp8codes", B, 16, 1, 1, qd, "fp8_e4m3", k_scale=1.0, v_scale=1 / 64, seed=19)
    inp = make_inputs(w, device="cuda", seq_lens=torch.ones(B, dtype=torch.int32))
    codes = (torch.arange(B * 8 * 128, device="cuda") % 256).to(torch.uint8).view(B, 8, 128)
    inp["kv"][:, 1, :, 0] = codes
    out, _ = run_decode(inp, "prepared")
    got = decoded_out(out, qd)
    want = decode_e4m3fn_bits(codes.cpu().numpy()) / 64.0
    for h in range(32):
        g_ = got[:, h]
        w_ = want[:, h // 4]
        assert np.array_equal(np.isnan(g_), np.isnan(w_)), h
        assert np.array_equal(g_[~np.isnan(g_)], w_[~np.isnan(w_)]), h


@pytest.mark.parametrize("qd", ["bf16", "f16"])
def test_fp8_full_code_range_parity(qd):
    """K and V bytes uniform over every finite e4m3fn code (subnormals to 448)."""
    B, C = 3, 640
    w = Workload("fp8range", B, C, 1, C, qd, "fp8_e4m3", q_scale=1.0, k_scale=1 / 4096,
                 v_scale=1 / 64, seed=21)
    inp = make_inputs(w, device="cuda", seq_lens=torch.tensor([640, 321, 16], dtype=torch.int32))
    gen = torch.Generator(device="cuda")
    gen.manual_seed(23)
    raw = torch.randint(0, 256, inp["kv"].shape, generator=gen, device="cuda", dtype=torch.int32)
    raw = torch.where((raw & 0x7F) == 0x7F, raw - 1, raw)   # drop the two NaN codes
    inp["kv"].copy_(raw.to(torch.uint8))
    out, _ = run_decode(inp, "prepared", num_splits=4)
    compare(out, oracle_pairs(inp, all_pairs(B)), inp, f"fp8 full range q={qd}")


# ------------------------------------------------------------- INT8 row-scaled cache
@pytest.mark.parametrize("qd", ["bf16", "f16"])
def test_int8_every_value_decodes_exactly(qd):
    """V row 0 holds every int8 value -128..127 with power-of-two row scales;
    with L = 1 the output is value * scale exactly."""
    B = 2
    w = Workload("int8values", B, 16, 1, 1, qd, "int8", seed=25, num_q_heads=16)
    inp = make_inputs(w, device="cuda", seq_lens=torch.ones(B, dtype=torch.int32))
    vals = (torch.arange(B * 8 * 128, device="cuda") % 256 - 128).to(torch.int8).view(B, 8, 128)
    inp["kv"][:, 1, :, 0] = vals
    exps = torch.arange(B * 8, device="cuda").view(B, 8) % 7 - 10        # 2^-10 .. 2^-4
    inp["kv_scales"][:, 1, :, 0] = torch.ldexp(torch.ones(B, 8, device="cuda"), exps.float())
    out, _ = run_decode(inp, "prepared")
    got = decoded_out(out, qd)
    want = vals.double().cpu().numpy() * np.ldexp(1.0, exps.cpu().numpy())[..., None]
    for h in range(16):
        assert np.array_equal(got[:, h], want[:, h // 2]), h


@pytest.mark.parametrize("qd", ["bf16", "f16"])
@pytest.mark.parametrize("num_splits", [None, 1, 6])
def test_int8_wide_row_scales_and_odd_capacity(qd, num_splits):
    """Row scales spread over 2^-14 .. 2^4 (per token and plane), extreme int8
    values, and a capacity that is not a multiple of 4 (the scale planes lose
    their 8-byte alignment), on every route."""
    B, C = 4, 1003
    w = Workload("int8wide", B, C, 1, C, qd, "int8", q_scale=0.25, seed=27, num_q_heads=16)
    inp = make_inputs(w, device="cuda",
                      seq_lens=torch.tensor([1003, 1, 514, 999], dtype=torch.int32))
    gen = torch.Generator(device="cuda")
    gen.manual_seed(29)
    e = torch.randint(-14, 5, inp["kv_scales"].shape, generator=gen, device="cuda")
    inp["kv_scales"].copy_(torch.ldexp(torch.ones_like(e, dtype=torch.float32), e.float())
                           .to(torch.bfloat16))
    raw = torch.randint(-128, 128, inp["kv"].shape, generator=gen, device="cuda")
    inp["kv"].copy_(raw.to(torch.int8))
    out, _ = run_decode(inp, "prepared", num_splits=num_splits)
    compare(out, oracle_pairs(inp, all_pairs(B)), inp, f"int8 wide scales q={qd} S={num_splits}")


def test_batch_zero_is_a_no_op():
    b = pytest.importorskip("gqa_kv_cache_attn_amd.binding")
    q = torch.empty(0, 32, 128, dtype=torch.bfloat16, device="cuda")
    kv = torch.empty(0, 2, 8, 64, 128, dtype=torch.bfloat16, device="cuda")
    lens = torch.empty(0, dtype=torch.int32, device="cuda")
    out = b.gqa_decode(q, kv, lens)
    assert out.shape == (0, 32, 128)



@pytest.mark.parametrize("kd,hq", [("bf16", 32), ("int8", 16)])
def test_maximum_capacity_every_slot_valid(kd, hq):
    """The largest accepted capacity (2^22 slots) with every slot valid: the last
    KV head's planes start 15 GiB (bf16) / 7.5 GiB (INT8) into the cache.
    q_scale = 4 concentrates each row's weights on a few dozen slots spread
    over the whole range (dropping its upper half would move outputs by ~0.3),
    so a wrong offset anywhere in it shows. Automatic (balanced, one request:
    one workgroup per CU) and a 64-way chunked split."""
    C = 1 << 22
    w = Workload(f"max_capacity_{kd}", 1, C, C, C, "bf16", kd, q_scale=4.0, seed=2222,
                 num_q_heads=hq)
    inp = make_inputs(w, device="cuda")
    assert int(inp["seq_lens"][0]) == C
    ref = oracle_pairs(inp, [(0, 7), (0, 0)])
    for ns in (None, 64):
        out = torch.full_like(inp["q"], float("nan"))
        out, prep = run_decode(inp, "prepared", num_splits=ns, out=out)
        assert prep.plan["route"] == (2 if ns is None else 1)
        compare(out, ref, inp, f"max capacity {kd} S={ns}")
        prep.destroy()
    del inp
    torch.cuda.empty_cache()


@pytest.mark.parametrize("B,route", [(4096, 2), (4097, 1)])
def test_batch_limits(B, route):
    """4096 requests, the most the balanced split takes (its slab prefix has
    one LDS entry per request), and 4097, which the automatic plan hands to
    the chunked split. Ragged lengths U[1, 256]; oracle on a sample of heads
    that includes the first and last request."""
    w = Workload(f"batch_{B}", B, 256, 1, 256, "bf16", "bf16", q_scale=0.8, seed=B)
    inp = make_inputs(w, device="cuda")
    out = torch.full_like(inp["q"], float("nan"))
    out, prep = run_decode(inp, "prepared", out=out)
    assert prep.plan["route"] == route
    pairs = [(b, (3 * b) % 8) for b in list(range(0, B, 97)) + [B - 2, B - 1]]
    compare(out, oracle_pairs(inp, pairs), inp, f"batch {B}")
    assert torch.isfinite(out.float()).all()
    prep.destroy()
