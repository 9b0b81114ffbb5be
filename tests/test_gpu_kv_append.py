"""GPU parity of the KV append (cache write before each decode step): the cache
after gqa_kv_append (or the page pool after gqa_kv_append_paged) equals the
oracle's, byte for byte."""

import numpy as np
import pytest
import torch

from gpu_util import (Workload, all_pairs, binding, compare, compare_paged, make_inputs,
                      oracle_pairs, require_gpu)
from gqa_kv_cache_attn_amd.inputs import make_paged_inputs, storage_bits
from oracle import decode_storage
from oracle.kv_append import kv_append_int8_reference, kv_append_reference
from oracle.paged import kv_append_paged_int8_reference, kv_append_paged_reference

pytestmark = pytest.mark.gpu

TORCH = {"f16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()


def _expected(kv, k_new, v_new, positions, src, kd, ks, vs):
    kv_bits = storage_bits(kv)
    k_bits, v_bits = storage_bits(k_new), storage_bits(v_new)
    with np.errstate(invalid="ignore"):      # NaN patterns stay NaN
        k32 = decode_storage(k_bits, src).astype(np.float32)
        v32 = decode_storage(v_bits, src).astype(np.float32)
    return kv_append_reference(kv_bits, k32, v32, positions.cpu().numpy(), kd, ks, vs,
                               new_bits=(k_bits, v_bits))


@pytest.mark.parametrize("src,kd,ks,vs", [("f16", "f16", 1.0, 1.0), ("bf16", "bf16", 1.0, 1.0),
                                          ("bf16", "fp8_e4m3", 1 / 64, 1 / 64),
                                          ("f16", "fp8_e4m3", 0.0137, 0.75)])
def test_append_is_byte_exact(src, kd, ks, vs):
    B, C = 5, 300
    w = Workload("append", B, C, 1, C, src, kd, k_scale=ks, v_scale=vs, seed=51)
    inp = make_inputs(w, device="cuda")
    kv = inp["kv"]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(52)
    k_new = (torch.randn(B, 8, 128, generator=gen, device="cuda") * 40).to(TORCH[src])
    v_new = (torch.randn(B, 8, 128, generator=gen, device="cuda") * 3).to(TORCH[src])
    k_new[0, 0, :6] = torch.tensor([float("nan"), float("inf"), -float("inf"), 0.0, -0.0, 1e-7])
    positions = torch.tensor([0, 299, 17, -1, 300], dtype=torch.int32, device="cuda")
    want = _expected(kv, k_new, v_new, positions, src, kd, ks, vs)
    binding().gqa_kv_append(kv, k_new, v_new, positions, ks, vs)
    torch.cuda.synchronize()
    got = storage_bits(kv)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("src", ["f16", "bf16"])
@pytest.mark.parametrize("scale", [1.0, 1 / 64, 0.0137])
def test_fp8_quantise_every_16bit_value(src, scale):
    """Every one of the 65536 f16 (or bf16) bit patterns, through the device encoder."""
    B = 64                                   # 64 * 8 * 128 = 65536 values per plane
    bits = torch.arange(1 << 16, dtype=torch.int32).to(torch.int16).view(torch.int16)
    vals = bits.view(TORCH[src]).reshape(B, 8, 128).to("cuda")
    kv = torch.zeros(B, 2, 8, 1, 128, dtype=torch.uint8, device="cuda")
    positions = torch.zeros(B, dtype=torch.int32, device="cuda")
    want = _expected(kv, vals, vals, positions, src, "fp8_e4m3", scale, scale)
    binding().gqa_kv_append(kv, vals, vals.clone(), positions, scale, scale)
    torch.cuda.synchronize()
    got = storage_bits(kv)
    bad = np.flatnonzero(got.ravel() != want.ravel())
    assert bad.size == 0, f"{bad.size} mismatches, first at {bad[:5]}"


@pytest.mark.parametrize("src,kd", [("bf16", "bf16"), ("bf16", "fp8_e4m3")])
def test_append_then_decode(src, kd):
    """A decode step after appending token L at slot L attends over L + 1 tokens."""
    B, C = 4, 2048
    fp8 = kd == "fp8_e4m3"
    w = Workload("append_decode", B, C, 1, C - 1, src, kd, q_scale=0.8,
                 k_scale=1 / 64 if fp8 else 1.0, v_scale=1 / 64 if fp8 else 1.0, seed=53)
    inp = make_inputs(w, device="cuda")
    lens = inp["seq_lens"]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(54)
    k_new = torch.randn(B, 8, 128, generator=gen, device="cuda").to(TORCH[src])
    v_new = torch.randn(B, 8, 128, generator=gen, device="cuda").to(TORCH[src])
    b = binding()
    b.gqa_kv_append(inp["kv"], k_new, v_new, lens, inp["k_scale"], inp["v_scale"])
    lens += 1
    out = b.gqa_decode(inp["q"], inp["kv"], lens, inp["q_scale"], k_scale=inp["k_scale"],
                       v_scale=inp["v_scale"])
    torch.cuda.synchronize()
    compare(out, oracle_pairs(inp, all_pairs(B)), inp, f"append+decode {src}/{kd}")


def test_append_argument_errors():
    b = binding()
    kv = torch.zeros(2, 2, 8, 16, 128, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(2, 8, 128, dtype=torch.bfloat16, device="cuda")
    pos = torch.zeros(2, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):           # a scale on a 16-bit cache
        b.gqa_kv_append(kv, k, k, pos, 0.5, 1.0)
    with pytest.raises(ValueError):           # f16 rows into a bf16 cache
        b.gqa_kv_append(kv, k.half(), k.half(), pos)
    flat = kv.view(-1)
    with pytest.raises(ValueError):           # k_new inside the cache
        b.gqa_kv_append(kv, flat[:2 * 8 * 128].view(2, 8, 128), k, pos)


# ---------------------------------------------------------------- page pool
def _expected_paged(pool, table, k_new, v_new, positions, src, kd, ks, vs):
    k_bits, v_bits = storage_bits(k_new), storage_bits(v_new)
    with np.errstate(invalid="ignore"):
        k32 = decode_storage(k_bits, src).astype(np.float32)
        v32 = decode_storage(v_bits, src).astype(np.float32)
    return kv_append_paged_reference(storage_bits(pool), table.cpu().numpy(),
                                     positions.cpu().numpy(), k32, v32, kd, ks, vs,
                                     new_bits=(k_bits, v_bits))


def _new_rows(B, T, src, seed):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    k_new = (torch.randn(B, T, 8, 128, generator=gen, device="cuda") * 40).to(TORCH[src])
    v_new = (torch.randn(B, T, 8, 128, generator=gen, device="cuda") * 3).to(TORCH[src])
    return k_new, v_new


@pytest.mark.parametrize("src,kd,ks,vs", [("f16", "f16", 1.0, 1.0), ("bf16", "bf16", 1.0, 1.0),
                                          ("bf16", "fp8_e4m3", 1 / 64, 1 / 64),
                                          ("f16", "fp8_e4m3", 0.0137, 0.75)])
@pytest.mark.parametrize("P", [16, 64])
@pytest.mark.parametrize("T", [1, 3])
def test_paged_append_is_byte_exact(src, kd, ks, vs, P, T):
    """Slots across page boundaries, before slot 0, past the last page, and in
    table entries outside the pool (those write nothing)."""
    B, C = 6, 256
    w = Workload("append_paged", B, C, 1, C, src, kd, k_scale=ks, v_scale=vs, seed=61,
                 page_size=P, q_tokens=T)
    inp = make_paged_inputs(w, device="cuda")
    pool, table = inp["kv_pages"], inp["block_table"]
    max_pages, num_pages = table.shape[1], pool.shape[0]
    table[4, 0] = -1                      # request 4 writes into entry 0 only: skipped
    table[5, 1] = num_pages + 7           # request 5 crosses into entry 1: skipped there
    k_new, v_new = _new_rows(B, T, src, 62)
    k_new[0, 0, 0, :6] = torch.tensor([float("nan"), float("inf"), -float("inf"), 0.0, -0.0, 1e-7])
    # request 1 (T > 1) crosses a page boundary; request 2's later tokens fall
    # past the last page; request 3 starts before slot 0; request 5 starts in
    # its first page and crosses into the bad entry
    positions = torch.tensor([0, P - 1, max_pages * P - 1, -1, 0, P - 1], dtype=torch.int32,
                             device="cuda")
    print(f"[case] paged append {src}->{kd} P={P} T={T}", flush=True)
    want = _expected_paged(pool, table, k_new, v_new, positions, src, kd, ks, vs)
    binding().gqa_kv_append_paged(pool, table, k_new, v_new, positions, ks, vs)
    torch.cuda.synchronize()
    got = storage_bits(pool)
    bad = np.flatnonzero(got.ravel() != want.ravel())
    assert bad.size == 0, f"{bad.size} mismatching bytes, first at {bad[:5]}"


@pytest.mark.parametrize("src,kd", [("bf16", "bf16"), ("bf16", "fp8_e4m3"), ("f16", "f16")])
@pytest.mark.parametrize("hq,T", [(32, 4), (16, 3)])
def test_paged_append_then_verify_pass(src, kd, hq, T):
    """The verify step of speculative decoding: T draft tokens appended at
    slots L .. L + T - 1, then decoded with lengths L + T; the pool must equal
    the oracle's and the output the oracle's decode of that pool."""
    B, C, P = 4, 1024, 16
    fp8 = kd == "fp8_e4m3"
    w = Workload("append_verify", B, C, 1, C - T, src, kd, q_scale=0.8,
                 k_scale=1 / 64 if fp8 else 1.0, v_scale=1 / 64 if fp8 else 1.0, seed=63,
                 num_q_heads=hq, page_size=P, q_tokens=T)
    inp = make_paged_inputs(w, device="cuda")
    lens = inp["seq_lens"]
    k_new, v_new = _new_rows(B, T, src, 64)
    want = _expected_paged(inp["kv_pages"], inp["block_table"], k_new, v_new, lens, src, kd,
                           inp["k_scale"], inp["v_scale"])
    b = binding()
    b.gqa_kv_append_paged(inp["kv_pages"], inp["block_table"], k_new, v_new, lens,
                          inp["k_scale"], inp["v_scale"], num_q_heads=hq)
    lens += T
    out = torch.empty_like(inp["q"])
    b.gqa_decode_paged(inp["q"], inp["kv_pages"], inp["block_table"], lens, inp["q_scale"], out,
                       k_scale=inp["k_scale"], v_scale=inp["v_scale"])
    torch.cuda.synchronize()
    assert np.array_equal(storage_bits(inp["kv_pages"]), want)
    compare_paged(out, inp, range(B), f"paged append+verify {src}/{kd}/{hq}q/T={T}")


def test_paged_append_argument_errors():
    b = binding()
    pool = torch.zeros(4, 2, 8, 16, 128, dtype=torch.bfloat16, device="cuda")
    table = torch.zeros(2, 2, dtype=torch.int32, device="cuda")
    k = torch.zeros(2, 2, 8, 128, dtype=torch.bfloat16, device="cuda")
    pos = torch.zeros(2, dtype=torch.int32, device="cuda")
    before = pool.clone()
    with pytest.raises(ValueError):           # a scale on a 16-bit pool
        b.gqa_kv_append_paged(pool, table, k, k, pos, 0.5, 1.0)
    with pytest.raises(ValueError):           # f16 rows into a bf16 pool
        b.gqa_kv_append_paged(pool, table, k.half(), k.half(), pos)
    with pytest.raises(ValueError):           # 5 tokens x 4 query heads per KV head > 16 rows
        k5 = torch.zeros(2, 5, 8, 128, dtype=torch.bfloat16, device="cuda")
        b.gqa_kv_append_paged(pool, table, k5, k5, pos)
    flat = pool.view(-1)
    with pytest.raises(ValueError):           # k_new inside the pool
        b.gqa_kv_append_paged(pool, table, flat[:2 * 2 * 8 * 128].view(2, 2, 8, 128), k, pos)
    torch.cuda.synchronize()
    assert torch.equal(pool, before)


# ---------------------------------------------------------------- captured decode loop
@pytest.mark.parametrize("paged", [False, True], ids=["contiguous", "paged"])
@pytest.mark.parametrize("kd", ["bf16", "fp8_e4m3", "int8"])
def test_captured_decode_loop_matches_eager_steps(paged, kd):
    """One decode step captured once and replayed: append the step's new rows at
    the current lengths, advance the lengths on the device, attend. Nothing in
    it allocates or waits on the host, so it replays; every replay must equal
    the same calls made eagerly on a copy of the state, and the last one the
    oracle."""
    b = binding()
    fp8, int8 = kd == "fp8_e4m3", kd == "int8"
    B, C, T = 4, 2048, (2 if paged else 1)
    ks = vs = 1 / 64 if fp8 else 1.0
    w = Workload("loop", B, C, 100, C - 8, "bf16", kd, q_scale=0.9, k_scale=ks, v_scale=vs,
                 seed=71, page_size=16 if paged else 0, q_tokens=T, num_q_heads=16 if int8 else 32)

    def state():
        inp = make_paged_inputs(w, device="cuda") if paged else make_inputs(w, device="cuda")
        out = torch.empty_like(inp["q"])
        if paged:
            prep = b.prepare_gqa_decode_paged(inp["q"], inp["kv_pages"], inp["block_table"],
                                              inp["seq_lens"], out, inp["q_scale"],
                                              k_scale=ks, v_scale=vs, kv_scales=inp["kv_scales"])
        elif int8:
            prep = b.prepare_gqa_decode_int8(inp["q"], inp["kv"], inp["kv_scales"], inp["seq_lens"],
                                             out, inp["q_scale"], k_scale=ks, v_scale=vs)
        else:
            prep = b.prepare_gqa_decode(inp["q"], inp["kv"], inp["seq_lens"], out, inp["q_scale"],
                                        k_scale=ks, v_scale=vs)
        return inp, out, prep

    shape = (B, T, 8, 128) if paged else (B, 8, 128)
    k_new = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
    v_new = torch.zeros_like(k_new)

    def step(inp, prep):
        if paged and int8:
            b.gqa_kv_append_paged_int8(inp["kv_pages"], inp["kv_scales"], inp["block_table"],
                                       k_new, v_new, inp["seq_lens"], ks, vs)
        elif paged:
            b.gqa_kv_append_paged(inp["kv_pages"], inp["block_table"], k_new, v_new,
                                  inp["seq_lens"], ks, vs)
        elif int8:
            b.gqa_kv_append_int8(inp["kv"], inp["kv_scales"], k_new, v_new, inp["seq_lens"], ks, vs)
        else:
            b.gqa_kv_append(inp["kv"], k_new, v_new, inp["seq_lens"], ks, vs)
        inp["seq_lens"].add_(T)
        b.launch_gqa_decode_prepared(prep)

    g_inp, g_out, g_prep = state()       # the captured copy
    e_inp, e_out, e_prep = state()       # the eager copy (same seed, same contents)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        b.launch_gqa_decode_prepared(g_prep)   # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(g_inp, g_prep)

    gen = torch.Generator(device="cuda")
    gen.manual_seed(72)
    for i in range(4):
        k_new.copy_(torch.randn(shape, generator=gen, device="cuda").to(torch.bfloat16))
        v_new.copy_(torch.randn(shape, generator=gen, device="cuda").to(torch.bfloat16))
        graph.replay()
        torch.cuda.synchronize()
        step(e_inp, e_prep)                  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(g_inp["seq_lens"], e_inp["seq_lens"]), i
        assert torch.equal(g_out.view(torch.int16), e_out.view(torch.int16)), i
    cache = "kv_pages" if paged else "kv"
    assert torch.equal(g_inp[cache].view(torch.uint8), e_inp[cache].view(torch.uint8))
    if int8:
        assert torch.equal(g_inp["kv_scales"].view(torch.int16), e_inp["kv_scales"].view(torch.int16))
    if paged:
        compare_paged(g_out, g_inp, range(B), f"captured loop paged {kd}")
    else:
        compare(g_out, oracle_pairs(g_inp, all_pairs(B)), g_inp, f"captured loop {kd}")
    del graph
    g_prep.destroy()
    e_prep.destroy()



# ---------------------------------------------------------------- INT8 cache (row scales)
def _scale_bits(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _rows_f32(t, src):
    with np.errstate(invalid="ignore"):
        return decode_storage(storage_bits(t), src).astype(np.float32)


def _int8_rows(B, shape, src, seed):
    """New rows of assorted magnitudes: N(0,1) times 40 / 3 / 1e-3 / 1e-30 per
    request, one all-zero row and one row of exact ties (max 127: scale 1)."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    x = torch.randn(*shape, generator=gen, device="cuda")
    mags = torch.tensor([40.0, 3.0, 1e-3, 1e-30, 1.0], device="cuda")
    x *= mags[torch.arange(B, device="cuda") % 5].view(B, *([1] * (x.dim() - 1)))
    x[0].view(-1, 128)[0] = 0.0
    ties = torch.zeros(128, device="cuda")
    ties[:8] = torch.tensor([127.0, 2.5, 3.5, -4.5, 0.5, -0.5, 126.5, -1.5])
    x[1].view(-1, 128)[1] = ties
    return x.to(TORCH[src])


@pytest.mark.parametrize("src,ks,vs", [("bf16", 1.0, 1.0), ("f16", 1.0, 1.0), ("bf16", 0.5, 4.0),
                                       ("f16", 0.0137, 0.75)])
def test_int8_append_is_byte_exact(src, ks, vs):
    """Codes and bf16 row scales equal the oracle's quantise-on-write, byte for byte."""
    B, C = 5, 300
    w = Workload("append_int8", B, C, 1, C, src, "int8", k_scale=ks, v_scale=vs, seed=81,
                 num_q_heads=16)
    inp = make_inputs(w, device="cuda")
    kv, sc = inp["kv"], inp["kv_scales"]
    k_new = _int8_rows(B, (B, 8, 128), src, 82)
    v_new = _int8_rows(B, (B, 8, 128), src, 83)
    positions = torch.tensor([0, 299, 17, -1, 300], dtype=torch.int32, device="cuda")
    want_c, want_s = kv_append_int8_reference(kv.cpu().numpy(), _scale_bits(sc),
                                              _rows_f32(k_new, src), _rows_f32(v_new, src),
                                              positions.cpu().numpy(), ks, vs)
    binding().gqa_kv_append_int8(kv, sc, k_new, v_new, positions, ks, vs)
    torch.cuda.synchronize()
    assert np.array_equal(kv.cpu().numpy(), want_c)
    assert np.array_equal(_scale_bits(sc), want_s)


@pytest.mark.parametrize("src", ["f16", "bf16"])
def test_int8_append_of_every_16bit_value(src):
    """All 65536 f16 (bf16) bit patterns in order, as 512 rows of 128 per
    plane: rows mix magnitudes within a binade range; rows holding a NaN or an
    infinity are unspecified and not compared."""
    B = 64
    bits = torch.arange(1 << 16, dtype=torch.int32).to(torch.int16)
    vals = bits.view(TORCH[src]).reshape(B, 8, 128).to("cuda")
    kv = torch.zeros(B, 2, 8, 1, 128, dtype=torch.int8, device="cuda")
    sc = torch.zeros(B, 2, 8, 1, dtype=torch.bfloat16, device="cuda")
    positions = torch.zeros(B, dtype=torch.int32, device="cuda")
    x32 = _rows_f32(vals, src)
    want_c, want_s = kv_append_int8_reference(kv.cpu().numpy(), _scale_bits(sc), x32, x32,
                                              positions.cpu().numpy(), 1.0, 1.0)
    binding().gqa_kv_append_int8(kv, sc, vals, vals.clone(), positions)
    torch.cuda.synchronize()
    finite = np.isfinite(x32).all(axis=-1)                 # [B, 8]
    got_c, got_s = kv.cpu().numpy()[:, :, :, 0], _scale_bits(sc)[:, :, :, 0]
    for plane in range(2):
        assert np.array_equal(got_s[:, plane][finite], want_s[:, plane, :, 0][finite])
        bad = np.flatnonzero((got_c[:, plane] != want_c[:, plane, :, 0])[finite].any(axis=-1))
        assert bad.size == 0, f"plane {plane}: {bad.size} rows differ, first {bad[:5]}"


@pytest.mark.parametrize("src", ["bf16", "f16"])
def test_int8_append_then_decode(src):
    """A decode step over an INT8 cache after appending token L at slot L."""
    B, C = 4, 2048
    w = Workload("append_decode_int8", B, C, 1, C - 1, src, "int8", q_scale=0.8, seed=84,
                 num_q_heads=16)
    inp = make_inputs(w, device="cuda")
    lens = inp["seq_lens"]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(85)
    k_new = torch.randn(B, 8, 128, generator=gen, device="cuda").to(TORCH[src])
    v_new = torch.randn(B, 8, 128, generator=gen, device="cuda").to(TORCH[src])
    b = binding()
    b.gqa_kv_append_int8(inp["kv"], inp["kv_scales"], k_new, v_new, lens)
    lens += 1
    out = b.gqa_decode_int8(inp["q"], inp["kv"], inp["kv_scales"], lens, inp["q_scale"])
    torch.cuda.synchronize()
    compare(out, oracle_pairs(inp, all_pairs(B)), inp, f"int8 append+decode {src}")


@pytest.mark.parametrize("src", ["bf16", "f16"])
@pytest.mark.parametrize("P,T", [(16, 1), (16, 3), (64, 2), (128, 8)])
def test_paged_int8_append_is_byte_exact(src, P, T):
    B, C = 5, 1000
    w = Workload("paged_append_int8", B, C, 1, C, src, "int8", k_scale=0.5, v_scale=2.0,
                 seed=86, num_q_heads=16, page_size=P, q_tokens=T)
    inp = make_paged_inputs(w, device="cuda")
    pool, sc, table = inp["kv_pages"], inp["kv_scales"], inp["block_table"]
    k_new = _int8_rows(B, (B, T, 8, 128), src, 87)
    v_new = _int8_rows(B, (B, T, 8, 128), src, 88)
    cap = table.shape[1] * P
    positions = torch.tensor([0, P - 1, cap - T, -1, cap], dtype=torch.int32, device="cuda")
    want_c, want_s = kv_append_paged_int8_reference(
        pool.cpu().numpy(), _scale_bits(sc), table.cpu().numpy(), positions.cpu().numpy(),
        _rows_f32(k_new, src), _rows_f32(v_new, src), 0.5, 2.0)
    binding().gqa_kv_append_paged_int8(pool, sc, table, k_new, v_new, positions, 0.5, 2.0)
    torch.cuda.synchronize()
    assert np.array_equal(pool.cpu().numpy(), want_c)
    assert np.array_equal(_scale_bits(sc), want_s)


def test_int8_append_argument_errors():
    b = binding()
    kv = torch.zeros(2, 2, 8, 16, 128, dtype=torch.int8, device="cuda")
    sc = torch.zeros(2, 2, 8, 16, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(2, 8, 128, dtype=torch.bfloat16, device="cuda")
    pos = torch.zeros(2, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):           # scales of the wrong shape
        b.gqa_kv_append_int8(kv, sc[:, :, :, :8], k, k, pos)
    with pytest.raises(ValueError):           # the plain form refuses an INT8 cache
        b.gqa_kv_append(kv, k, k, pos)
    with pytest.raises(ValueError):           # scales inside the cache
        b.gqa_kv_append_int8(kv, kv.view(-1)[:2 * 2 * 8 * 16 * 2].view(torch.bfloat16)
                             .view(2, 2, 8, 16), k, k, pos)
