"""Pins for the paged / multi-token oracle (oracle/paged.py): facts fixed by
mathematics or by a library routine, each chosen so that a plausible mistake
(slot j read from the wrong page or row, an off-by-one causal limit, token
order reversed, grouping lost) fails at least one of them."""

import math

import numpy as np
import pytest
import torch

from oracle import HEAD_DIM, NUM_KV_HEADS, decode_int8_rows, gqa_decode_reference
from oracle.brute import brute_decode
from oracle.kv_append import (kv_append_int8_reference, kv_append_reference, quantise_fp8,
                               quantise_int8_rows)
from oracle.paged import (gather_pages, gqa_decode_multi, gqa_decode_paged_reference,
                          int8_rows_by_position, kv_append_paged_int8_reference,
                          kv_append_paged_reference)


def _scatter_case(rng, B, P, max_pages, lens, spare=3, dtype=np.float64):
    """Contiguous rows X [B, 2, 8, max_pages*P, 128] written into a shuffled pool
    by explicit loops (the inverse of the gather under test); unused pages NaN."""
    C = P * max_pages
    X = rng.standard_normal((B, 2, NUM_KV_HEADS, C, HEAD_DIM)).astype(dtype)
    num_pages = B * max_pages + spare
    ids = rng.permutation(num_pages)[:B * max_pages].reshape(B, max_pages)
    pool = np.full((num_pages, 2, NUM_KV_HEADS, P, HEAD_DIM), np.nan, dtype=dtype)
    for b in range(B):
        for p in range(max_pages):
            for s in range(P):
                pool[ids[b, p], :, :, s] = X[b, :, :, p * P + s]
    return X, pool, ids.astype(np.int32), np.asarray(lens)


@pytest.mark.parametrize("P", [16, 32, 48])
def test_gather_inverts_an_explicit_scatter(P):
    rng = np.random.default_rng(3)
    X, pool, table, lens = _scatter_case(rng, 3, P, 4, [4 * P, 1, 2 * P + 5])
    for b in range(3):
        L = int(lens[b])
        assert np.array_equal(gather_pages(pool, table[b], L, P), X[b, :, :, :L])


def test_single_token_paged_equals_the_contiguous_definition():
    rng = np.random.default_rng(5)
    P = 16
    X, pool, table, lens = _scatter_case(rng, 2, P, 3, [48, 17])
    q = rng.standard_normal((2, 1, 32, HEAD_DIM))
    got = gqa_decode_paged_reference(q, pool, table, lens, P, 0.8, 0.5, 2.0)
    want = gqa_decode_reference(q[:, 0], X, lens, 0.8, 0.5, 2.0)
    np.testing.assert_allclose(got[:, 0], want, rtol=0, atol=1e-14)


@pytest.mark.parametrize("Hq,T", [(32, 1), (32, 2), (32, 4), (16, 3), (16, 8)])
def test_causal_rows_match_sdpa_with_a_boolean_mask(Hq, T):
    """fp64 scaled_dot_product_attention with an explicit mask j <= L - T + t."""
    rng = np.random.default_rng(7 + T)
    P = 16
    lens = [40, T + 3]
    X, pool, table, lens = _scatter_case(rng, 2, P, 3, lens)
    q = rng.standard_normal((2, T, Hq, HEAD_DIM))
    qs, ks, vs = 0.9, 0.25, 3.0
    got = gqa_decode_paged_reference(q, pool, table, lens, P, qs, ks, vs)
    for b, L in enumerate(lens):
        mask = torch.tensor([[j <= L - T + t for j in range(L)] for t in range(T)])
        sd = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[b]).permute(1, 0, 2).unsqueeze(0),          # [1, Hq, T, D]
            torch.from_numpy(X[b, 0, :, :L]).unsqueeze(0),                 # [1, 8, L, D]
            torch.from_numpy(X[b, 1, :, :L]).unsqueeze(0),
            attn_mask=mask, scale=qs * ks / math.sqrt(HEAD_DIM), enable_gqa=True)
        want = vs * sd[0].permute(1, 0, 2).numpy()                          # [T, Hq, D]
        np.testing.assert_allclose(got[b], want, rtol=0, atol=1e-12)


def test_causal_rows_match_brute_force():
    rng = np.random.default_rng(11)
    B, T, C = 2, 3, 6
    q = rng.standard_normal((B, T, 32, HEAD_DIM))
    kv = rng.standard_normal((B, 2, NUM_KV_HEADS, C, HEAD_DIM))
    lens = [6, 3]
    got = gqa_decode_multi(q, [kv[b] for b in range(B)], lens, 0.7)
    for t in range(T):
        lt = [L - T + 1 + t for L in lens]
        want = np.array(brute_decode(q[:, t].tolist(), kv.tolist(), lt, 0.7))
        np.testing.assert_allclose(got[:, t], want, rtol=0, atol=1e-12)


def test_identical_keys_give_the_mean_of_each_causal_prefix():
    rng = np.random.default_rng(13)
    T, L = 4, 20
    kv = rng.standard_normal((1, 2, NUM_KV_HEADS, L, HEAD_DIM))
    kv[0, 0] = kv[0, 0, :, :1]
    q = rng.standard_normal((1, T, 32, HEAD_DIM))
    got = gqa_decode_multi(q, [kv[0]], [L])
    for t in range(T):
        visible = L - T + 1 + t
        for h in range(32):
            np.testing.assert_allclose(got[0, t, h], kv[0, 1, h // 4, :visible].mean(0),
                                       rtol=0, atol=1e-13)


def test_last_token_sees_the_whole_length_and_first_token_one_less_per_step():
    rng = np.random.default_rng(17)
    T, L = 3, 30
    kv = rng.standard_normal((1, 2, NUM_KV_HEADS, L, HEAD_DIM))
    q = rng.standard_normal((1, T, 32, HEAD_DIM))
    got = gqa_decode_multi(q, [kv[0]], [L], 1.3)
    for t in range(T):
        single = gqa_decode_reference(q[:, t], kv, [L - T + 1 + t], 1.3)
        np.testing.assert_allclose(got[:, t], single, rtol=0, atol=1e-14)
    # a token that saw one slot fewer differs (the causal limit matters)
    assert not np.allclose(got[0, 0], gqa_decode_reference(q[:, 0], kv, [L], 1.3)[0])


def test_page_relabelling_and_garbage_outside_the_prefix_do_not_matter():
    rng = np.random.default_rng(19)
    P = 32
    X, pool, table, lens = _scatter_case(rng, 3, P, 3, [70, 33, 96], spare=5)
    q = rng.standard_normal((3, 2, 16, HEAD_DIM))
    base = gqa_decode_paged_reference(q, pool, table, lens, P)
    assert np.all(np.isfinite(base))
    perm = rng.permutation(pool.shape[0])           # new id of old page i is perm[i]
    pool2 = np.empty_like(pool)
    pool2[perm] = pool
    np.testing.assert_array_equal(gqa_decode_paged_reference(q, pool2, perm[table], lens, P), base)
    pool3 = pool.copy()                             # NaN past each length inside used pages
    for b, L in enumerate(lens):
        for j in range(L, 3 * P):
            pool3[table[b, j // P], :, :, j % P] = np.nan
    np.testing.assert_array_equal(gqa_decode_paged_reference(q, pool3, table, lens, P), base)


def test_int8_pages_decode_each_row_with_its_own_scale():
    """Two pages, one token each visible: the output is the V row times its own
    row scale (int8 * bf16 exact), whichever page the slot sits in."""
    P = 16
    vals = np.zeros((2, 2, NUM_KV_HEADS, P, HEAD_DIM), dtype=np.int8)
    vals[:, 1, :, :, 5] = [[[7] * P] * NUM_KV_HEADS, [[-3] * P] * NUM_KV_HEADS]
    sbits = np.zeros((2, 2, NUM_KV_HEADS, P), dtype=np.uint16)
    sbits[0] = np.uint16(0x3F00)   # 0.5
    sbits[1] = np.uint16(0x4100)   # 8.0
    pages = decode_int8_rows(vals, sbits)
    q = np.zeros((2, 1, 32, HEAD_DIM))
    out = gqa_decode_paged_reference(q, pages, np.array([[1], [0]]), [1, 1], P)
    assert np.all(out[0, 0, :, 5] == -24.0) and np.all(out[1, 0, :, 5] == 3.5)


def test_rejects_impossible_inputs():
    rng = np.random.default_rng(23)
    X, pool, table, lens = _scatter_case(rng, 1, 16, 2, [20])
    q = rng.standard_normal((1, 4, 32, HEAD_DIM))
    with pytest.raises(ValueError):          # L < T: the first token would see nothing
        gqa_decode_paged_reference(q, pool, table, [3], 16)
    with pytest.raises(ValueError):          # table entry outside the pool
        gqa_decode_paged_reference(q, pool, np.array([[0, pool.shape[0]]]), [20], 16)
    with pytest.raises(ValueError):          # length beyond max_pages * page_size
        gqa_decode_paged_reference(q, pool, table, [33], 16)


# ---------------------------------------------------------------- appending to a pool
def _bits_case(rng, num_pages, P, B, T):
    pool = rng.integers(0, 256, size=(num_pages, 2, NUM_KV_HEADS, P, HEAD_DIM), dtype=np.uint8)
    k = rng.standard_normal((B, T, NUM_KV_HEADS, HEAD_DIM)).astype(np.float32)
    v = rng.standard_normal((B, T, NUM_KV_HEADS, HEAD_DIM)).astype(np.float32)
    return pool, k, v


def test_append_on_an_identity_table_is_the_contiguous_append():
    """page_size = capacity and block_table[b] = [b]: the pool is the contiguous
    cache, so one token per request must land exactly where the contiguous
    append puts it (fp8 codes and 16-bit copies alike)."""
    rng = np.random.default_rng(51)
    B, C = 3, 16
    pool, k, v = _bits_case(rng, B, C, B, 1)
    pos = [0, 15, 9]
    table = np.arange(B).reshape(B, 1)
    got = kv_append_paged_reference(pool, table, pos, k, v, "fp8_e4m3", 0.5, 0.125)
    want = kv_append_reference(pool, k[:, 0], v[:, 0], pos, "fp8_e4m3", 0.5, 0.125)
    assert np.array_equal(got, want)
    kb = rng.integers(0, 1 << 16, size=k.shape, dtype=np.uint16)
    vb = rng.integers(0, 1 << 16, size=k.shape, dtype=np.uint16)
    pool16 = rng.integers(0, 1 << 16, size=(B, 2, NUM_KV_HEADS, C, HEAD_DIM), dtype=np.uint16)
    got = kv_append_paged_reference(pool16, table, pos, k, v, "bf16", new_bits=(kb, vb))
    want = kv_append_reference(pool16, k[:, 0], v[:, 0], pos, "bf16", new_bits=(kb[:, 0], vb[:, 0]))
    assert np.array_equal(got, want)


@pytest.mark.parametrize("P", [16, 32])
def test_appended_tokens_are_read_back_at_their_slots_and_nothing_else_changes(P):
    """Through the separately pinned gather: slot positions[b] + t of request b
    holds token t's encoded rows (also across a page boundary); every other
    row of the pool keeps its bytes."""
    rng = np.random.default_rng(52)
    B, T, max_pages, num_pages = 3, 3, 4, 15
    pool, k, v = _bits_case(rng, num_pages, P, B, T)
    table = rng.permutation(num_pages)[:B * max_pages].reshape(B, max_pages)
    pos = [P - 1, 0, 2 * P + 5]          # request 0 crosses into its second page
    got = kv_append_paged_reference(pool, table, pos, k, v, "fp8_e4m3", 0.25, 2.0)
    touched = np.zeros((num_pages, P), dtype=bool)
    for b in range(B):
        rows = gather_pages(got, table[b], pos[b] + T, P)        # [2, 8, L, 128]
        for t in range(T):
            s = pos[b] + t
            assert np.array_equal(rows[0, :, s], quantise_fp8(k[b, t], 0.25))
            assert np.array_equal(rows[1, :, s], quantise_fp8(v[b, t], 2.0))
            touched[table[b, s // P], s % P] = True
    assert touched.sum() == B * T
    assert np.array_equal(got.transpose(0, 3, 1, 2, 4)[~touched], pool.transpose(0, 3, 1, 2, 4)[~touched])


def test_append_skips_slots_and_pages_out_of_range():
    rng = np.random.default_rng(53)
    P, B, T, max_pages, num_pages = 16, 4, 2, 2, 6
    pool, k, v = _bits_case(rng, num_pages, P, B, T)
    table = np.array([[0, 1], [2, -1], [3, num_pages], [4, 5]])
    # request 0: slots -2, -1 (before the start); request 1: slots 15, 16 (16 is in
    # page entry -1); request 2: slots 16, 17 in entry num_pages; request 3:
    # slots 31, 32 (32 beyond max_pages * P)
    pos = [-2, 15, 16, 31]
    got = kv_append_paged_reference(pool, table, pos, k, v, "fp8_e4m3", 1.0, 1.0)
    want = pool.copy()
    want[2, 0, :, 15] = quantise_fp8(k[1, 0], 1.0)
    want[2, 1, :, 15] = quantise_fp8(v[1, 0], 1.0)
    want[5, 0, :, 15] = quantise_fp8(k[3, 0], 1.0)
    want[5, 1, :, 15] = quantise_fp8(v[3, 0], 1.0)
    assert np.array_equal(got, want)



def test_int8_append_on_an_identity_table_is_the_contiguous_int8_append():
    rng = np.random.default_rng(54)
    B, C = 3, 16
    codes = rng.integers(-127, 128, size=(B, 2, NUM_KV_HEADS, C, HEAD_DIM)).astype(np.int8)
    sbits = rng.integers(0, 1 << 15, size=(B, 2, NUM_KV_HEADS, C)).astype(np.uint16)
    k = rng.standard_normal((B, 1, NUM_KV_HEADS, HEAD_DIM)).astype(np.float32)
    v = rng.standard_normal((B, 1, NUM_KV_HEADS, HEAD_DIM)).astype(np.float32)
    pos = [0, 15, 9]
    table = np.arange(B).reshape(B, 1)
    got = kv_append_paged_int8_reference(codes, sbits, table, pos, k, v, 0.5, 2.0)
    want = kv_append_int8_reference(codes, sbits, k[:, 0], v[:, 0], pos, 0.5, 2.0)
    assert all(np.array_equal(g, w) for g, w in zip(got, want))


def test_int8_append_lands_at_its_slots_and_skips_what_is_out_of_range():
    """Through the separately pinned gather: slot positions[b] + t holds token
    t's rows and row scales (across a page boundary too); slots past the
    table and entries outside the pool write nothing; all else is unchanged."""
    rng = np.random.default_rng(55)
    P, B, T, max_pages, num_pages = 16, 4, 3, 3, 12
    codes = rng.integers(-127, 128, size=(num_pages, 2, NUM_KV_HEADS, P, HEAD_DIM)).astype(np.int8)
    sbits = rng.integers(0, 1 << 15, size=(num_pages, 2, NUM_KV_HEADS, P)).astype(np.uint16)
    k = rng.standard_normal((B, T, NUM_KV_HEADS, HEAD_DIM)).astype(np.float32)
    v = rng.standard_normal((B, T, NUM_KV_HEADS, HEAD_DIM)).astype(np.float32)
    table = np.array([[3, 7, 1], [0, -1, 2], [4, num_pages, 6], [8, 9, 11]])
    # 0: crosses pages; 1: t = 2 hits entry -1; 2: t = 0 hits entry num_pages;
    # 3: t >= 1 lies past the table
    pos = [P - 1, P - 2, 2 * P - 1, 3 * P - 1]
    got, gsc = kv_append_paged_int8_reference(codes, sbits, table, pos, k, v, 0.25, 4.0)
    touched = np.zeros((num_pages, P), dtype=bool)
    for b in range(B):
        for t in range(T):
            s_ = pos[b] + t
            if s_ >= max_pages * P or not 0 <= table[b, s_ // P] < num_pages:
                continue
            page, row = table[b, s_ // P], s_ % P
            kc, ks = quantise_int8_rows(k[b, t], 0.25)
            vc, vs = quantise_int8_rows(v[b, t], 4.0)
            assert np.array_equal(got[page, 0, :, row], kc) and np.array_equal(gsc[page, 0, :, row], ks)
            assert np.array_equal(got[page, 1, :, row], vc) and np.array_equal(gsc[page, 1, :, row], vs)
            touched[page, row] = True
    assert touched.sum() == 3 + 2 + 2 + 1
    keep = ~touched
    assert np.array_equal(got.transpose(0, 3, 1, 2, 4)[keep], codes.transpose(0, 3, 1, 2, 4)[keep])
    assert np.array_equal(gsc.transpose(0, 3, 1, 2)[keep], sbits.transpose(0, 3, 1, 2)[keep])


# ---------------------------------------------------------------------------
# INT8 pools whose row scales are indexed by position ([B, 2, 8, max_pages * P]).

def _int8_pool_case(rng, B, P, max_pages, spare=3):
    num_pages = B * max_pages + spare
    codes = rng.integers(-127, 128, size=(num_pages, 2, NUM_KV_HEADS, P, HEAD_DIM)).astype(np.int8)
    # finite positive bf16 scales spread over 2^-14 .. 2^4 (exponent field 113..131)
    sbits = (rng.integers(113, 132, size=(num_pages, 2, NUM_KV_HEADS, P)) << 7 |
             rng.integers(0, 128, size=(num_pages, 2, NUM_KV_HEADS, P))).astype(np.uint16)
    table = rng.permutation(num_pages)[:B * max_pages].reshape(B, max_pages).astype(np.int32)
    return codes, sbits, table


@pytest.mark.parametrize("P", [16, 32, 64])
def test_position_scales_decode_as_the_page_scales_they_were_gathered_from(P):
    """Relabelling invariance: the same pool with its page scales moved to the
    positions that read them decodes to the same rows, element for element
    (a plane/head transposition or an off-by-one slot in the position
    indexing fails this)."""
    rng = np.random.default_rng(60 + P)
    B, max_pages = 3, 4
    codes, sbits, table = _int8_pool_case(rng, B, P, max_pages)
    lens = [max_pages * P, 1, 2 * P + 5]
    C = max_pages * P
    pos_scales = np.full((B, 2, NUM_KV_HEADS, C), 0x7FC0, dtype=np.uint16)   # NaN past L
    for b in range(B):
        L = lens[b]
        pos_scales[b, :, :, :L] = gather_pages(sbits[..., None], table[b], L, P)[..., 0]
    got = int8_rows_by_position(codes, pos_scales, table, lens, P)
    for b in range(B):
        L = lens[b]
        want = decode_int8_rows(gather_pages(codes, table[b], L, P),
                                gather_pages(sbits[..., None], table[b], L, P)[..., 0])
        assert got[b].shape == (2, NUM_KV_HEADS, L, HEAD_DIM)
        assert np.array_equal(got[b], want)


def test_position_scales_on_an_identity_table_are_the_contiguous_int8_cache():
    """With page b holding request b's slots in order, the pool and its
    position scales are the contiguous INT8 cache and its scale array, and
    decode with the contiguous definition."""
    rng = np.random.default_rng(61)
    B, C = 2, 16
    codes = rng.integers(-127, 128, size=(B, 2, NUM_KV_HEADS, C, HEAD_DIM)).astype(np.int8)
    sbits = (rng.integers(118, 128, size=(B, 2, NUM_KV_HEADS, C)) << 7).astype(np.uint16)
    lens = [16, 9]
    table = np.arange(B).reshape(B, 1)
    rows = int8_rows_by_position(codes, sbits, table, lens, C)
    q = rng.standard_normal((B, 1, 32, HEAD_DIM))
    got = gqa_decode_multi(q, rows, lens, 0.7, 0.5, 2.0)[:, 0]
    X = decode_int8_rows(codes, sbits)
    want = gqa_decode_reference(q[:, 0], X, lens, 0.7, 0.5, 2.0)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-14)


def test_position_scale_append_on_an_identity_table_is_the_contiguous_int8_append():
    rng = np.random.default_rng(62)
    B, C = 3, 16
    codes = rng.integers(-127, 128, size=(B, 2, NUM_KV_HEADS, C, HEAD_DIM)).astype(np.int8)
    sbits = rng.integers(0, 1 << 15, size=(B, 2, NUM_KV_HEADS, C)).astype(np.uint16)
    k = rng.standard_normal((B, 1, NUM_KV_HEADS, HEAD_DIM)).astype(np.float32)
    v = rng.standard_normal((B, 1, NUM_KV_HEADS, HEAD_DIM)).astype(np.float32)
    pos = [0, 15, 9]
    table = np.arange(B).reshape(B, 1)
    got = kv_append_paged_int8_reference(codes, sbits, table, pos, k, v, 0.5, 2.0,
                                         scales_by_position=True)
    want = kv_append_int8_reference(codes, sbits, k[:, 0], v[:, 0], pos, 0.5, 2.0)
    assert all(np.array_equal(g, w) for g, w in zip(got, want))


def test_position_scale_append_writes_the_scale_at_the_position_and_skips_with_the_row():
    """Across a page boundary, with shuffled pages: the codes land as in the
    page-scale append (separately pinned) and each scale at [b, plane, g,
    slot]; a token whose slot lies past the table or whose entry lies outside
    the pool writes neither; every other scale is unchanged."""
    rng = np.random.default_rng(63)
    P, B, T, max_pages, num_pages = 16, 4, 3, 3, 12
    codes = rng.integers(-127, 128, size=(num_pages, 2, NUM_KV_HEADS, P, HEAD_DIM)).astype(np.int8)
    page_sb = rng.integers(0, 1 << 15, size=(num_pages, 2, NUM_KV_HEADS, P)).astype(np.uint16)
    pos_sb = rng.integers(0, 1 << 15, size=(B, 2, NUM_KV_HEADS, max_pages * P)).astype(np.uint16)
    k = rng.standard_normal((B, T, NUM_KV_HEADS, HEAD_DIM)).astype(np.float32)
    v = rng.standard_normal((B, T, NUM_KV_HEADS, HEAD_DIM)).astype(np.float32)
    table = np.array([[3, 7, 1], [0, -1, 2], [4, num_pages, 6], [8, 9, 11]])
    pos = [P - 1, P - 2, 2 * P - 1, 3 * P - 1]
    got_c, got_s = kv_append_paged_int8_reference(codes, pos_sb, table, pos, k, v, 0.25, 4.0,
                                                  scales_by_position=True)
    want_c, _ = kv_append_paged_int8_reference(codes, page_sb, table, pos, k, v, 0.25, 4.0)
    assert np.array_equal(got_c, want_c)
    touched = np.zeros((B, max_pages * P), dtype=bool)
    for b in range(B):
        for t in range(T):
            s_ = pos[b] + t
            if s_ >= max_pages * P or not 0 <= table[b, s_ // P] < num_pages:
                continue
            _, ks = quantise_int8_rows(k[b, t], 0.25)
            _, vs = quantise_int8_rows(v[b, t], 4.0)
            assert np.array_equal(got_s[b, 0, :, s_], ks) and np.array_equal(got_s[b, 1, :, s_], vs)
            touched[b, s_] = True
    assert touched.sum() == 3 + 2 + 2 + 1
    keep = ~touched
    assert np.array_equal(got_s.transpose(0, 3, 1, 2)[keep], pos_sb.transpose(0, 3, 1, 2)[keep])


def test_position_scales_reject_a_wrong_shape():
    rng = np.random.default_rng(64)
    codes, sbits, table = _int8_pool_case(rng, 2, 16, 2)
    with pytest.raises(ValueError):
        int8_rows_by_position(codes, np.zeros((2, 2, NUM_KV_HEADS, 16), np.uint16), table, [5, 5], 16)
