"""Pins for the CPU oracle: facts fixed by the pages or by mathematics.

Each test would fail for a plausible mistake in the oracle (dropped scale,
misplaced k/v scale, wrong head mapping, transposed K/V, off-by-one length,
missing max shift, wrong fp8 exponent bias or subnormal rule). None of them
re-types the oracle's own vectorised formula.
"""

import math
import os

import numpy as np
import pytest
import torch

from oracle import (
    GROUP,
    HEAD_DIM,
    NUM_KV_HEADS,
    NUM_Q_HEADS,
    decode_bf16_bits,
    decode_e4m3fn_bits,
    decode_e4m3fn_lookup,
    decode_f16_bits,
    decode_storage,
    e4m3fn_table,
    gqa_decode_head,
    gqa_decode_reference,
    gqa_decode_weights,
)
from oracle.brute import brute_decode

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_case(rng, B, C, lens=None):
    q = rng.standard_normal((B, NUM_Q_HEADS, HEAD_DIM))
    kv = rng.standard_normal((B, 2, NUM_KV_HEADS, C, HEAD_DIM))
    if lens is None:
        lens = rng.integers(1, C + 1, size=B)
    return q, kv, np.asarray(lens)


# ---------------------------------------------------------------- pin 9: formats
def test_e4m3fn_matches_torch_for_all_codes():
    """Library special case: torch.float8_e4m3fn is the format the pages name."""
    codes = np.arange(256, dtype=np.uint8)
    ours = decode_e4m3fn_bits(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    both_nan = np.isnan(ours) & np.isnan(ref)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert np.array_equal(ours[~both_nan], ref[~both_nan])
    # sign of zero is preserved too
    assert math.copysign(1.0, ours[0x80]) == -1.0


def test_e4m3fn_anchor_values_from_spec():
    path = os.path.join(GOLDEN, "e4m3fn_anchor_values.txt")
    n = 0
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            code_s, val_s = line.split()
            got = decode_e4m3fn_bits(np.array([int(code_s, 16)], dtype=np.uint8))[0]
            want = float(val_s)
            if math.isnan(want):
                assert math.isnan(got), code_s
            else:
                assert got == want and math.copysign(1, got) == math.copysign(1, want), code_s
            n += 1
    assert n >= 10


def test_e4m3fn_lookup_equals_the_definition_on_every_code():
    """The table decoder is the definition decoder evaluated once per code:
    equal on all 256 codes (NaN where it is NaN, signed zeros kept) and on a
    multi-dimensional array of random bytes, the shape a cache slice has."""
    codes = np.arange(256, dtype=np.uint8)
    ref = decode_e4m3fn_bits(codes)
    for got in (e4m3fn_table(), decode_e4m3fn_lookup(codes)):
        assert got.dtype == np.float64 and got.shape == (256,)
        assert np.array_equal(np.isnan(got), np.isnan(ref))
        fin = ~np.isnan(ref)
        assert np.array_equal(got[fin], ref[fin])
        assert np.array_equal(np.signbit(got[fin]), np.signbit(ref[fin]))
    rng = np.random.default_rng(11)
    arr = rng.integers(0, 256, size=(3, 2, 5, 128), dtype=np.uint8)
    got, ref = decode_storage(arr, "fp8_e4m3"), decode_e4m3fn_bits(arr)
    assert got.shape == arr.shape
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[~np.isnan(ref)], ref[~np.isnan(ref)])
    # The cached table cannot be altered through the copy e4m3fn_table returns.
    t = e4m3fn_table()
    t[:] = 0.0
    assert decode_e4m3fn_lookup(np.array([0x38], dtype=np.uint8))[0] == 1.0


def test_e4m3fn_all_finite_codes_exact_in_bf16_and_f16():
    # Why converting fp8 to bf16/f16 on the GPU loses nothing: every finite
    # e4m3fn value has <= 4 significant bits and exponent in [-9, 8].
    vals = decode_e4m3fn_bits(np.arange(256, dtype=np.uint8))
    vals = vals[np.isfinite(vals)]
    assert np.array_equal(torch.tensor(vals).to(torch.bfloat16).double().numpy(), vals)
    assert np.array_equal(torch.tensor(vals).to(torch.float16).double().numpy(), vals)


def test_16bit_decoders_match_torch():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 1 << 16, size=4096).astype(np.uint16)
    bf = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    hf = torch.from_numpy(bits.view(np.int16)).view(torch.float16).double().numpy()
    ob, oh = decode_bf16_bits(bits), decode_f16_bits(bits)
    assert np.array_equal(np.isnan(ob), np.isnan(bf)) and np.array_equal(ob[~np.isnan(ob)], bf[~np.isnan(bf)])
    assert np.array_equal(np.isnan(oh), np.isnan(hf)) and np.array_equal(oh[~np.isnan(oh)], hf[~np.isnan(hf)])


# ---------------------------------------------------------------- pin 1: weights
def test_softmax_weights_sum_to_one():
    rng = np.random.default_rng(1)
    q, kv, lens = _rand_case(rng, 3, 50)
    for w in gqa_decode_weights(q, kv, lens, q_scale=0.7):
        assert w.min() >= 0.0
        assert np.max(np.abs(w.sum(axis=1) - 1.0)) <= 1e-12


# ---------------------------------------------------------------- pin 2: L = 1
@pytest.mark.parametrize("v_scale", [1.0, 1.0 / 64])
def test_single_token_returns_scaled_v_row0(v_scale):
    rng = np.random.default_rng(2)
    q, kv, _ = _rand_case(rng, 2, 9)
    lens = np.array([1, 1])
    out = gqa_decode_reference(q, kv, lens, q_scale=3.0, k_scale=0.25, v_scale=v_scale)
    for b in range(2):
        for h in range(NUM_Q_HEADS):
            assert np.array_equal(out[b, h], v_scale * kv[b, 1, h // GROUP, 0])


# ---------------------------------------------------------------- pin 3: identical keys
def test_identical_keys_give_mean_of_values():
    rng = np.random.default_rng(3)
    q, kv, _ = _rand_case(rng, 2, 40)
    lens = np.array([17, 40])
    kv[:, 0] = kv[:, 0, :, :1, :]          # every key equals key 0
    out = gqa_decode_reference(q, kv, lens, v_scale=0.5)
    for b, L in enumerate(lens):
        for h in range(NUM_Q_HEADS):
            want = 0.5 * kv[b, 1, h // GROUP, :L].mean(axis=0)
            np.testing.assert_allclose(out[b, h], want, rtol=0, atol=1e-14)


# ---------------------------------------------------------------- pin 4: padding
@pytest.mark.parametrize("pad", ["random", "nan"])
def test_capacity_padding_is_invisible(pad):
    rng = np.random.default_rng(4)
    L = np.array([5, 13])
    q, kv_tight, _ = _rand_case(rng, 2, 13, L)
    kv_tight[0, :, :, 5:] = rng.standard_normal(kv_tight[0, :, :, 5:].shape)
    kv_wide = (rng.standard_normal((2, 2, NUM_KV_HEADS, 52, HEAD_DIM)) if pad == "random"
               else np.full((2, 2, NUM_KV_HEADS, 52, HEAD_DIM), np.nan))
    kv_wide[:, :, :, :13] = kv_tight
    kv_wide[0, :, :, 5:13] = np.nan if pad == "nan" else 1e3
    a = gqa_decode_reference(q, kv_tight, L)
    b = gqa_decode_reference(q, kv_wide, L)
    assert np.array_equal(a, b)
    assert np.all(np.isfinite(b))


# ---------------------------------------------------------------- pin 5: brute force
def test_brute_force_agrees_on_tiny_inputs():
    rng = np.random.default_rng(5)
    q, kv, _ = _rand_case(rng, 2, 6)
    lens = np.array([6, 3])
    qs, ks, vs = 0.8, 1.7, 0.3
    ref = gqa_decode_reference(q, kv, lens, qs, ks, vs)
    brute = np.array(brute_decode(q.tolist(), kv.tolist(), lens.tolist(), qs, ks, vs))
    np.testing.assert_allclose(ref, brute, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- pin 6: SDPA
def test_matches_torch_sdpa_fp64_with_gqa():
    rng = np.random.default_rng(6)
    q, kv, _ = _rand_case(rng, 3, 70)
    lens = np.array([70, 1, 33])
    qs, ks, vs = 0.5, 2.0, 0.125
    ref = gqa_decode_reference(q, kv, lens, qs, ks, vs)
    for b, L in enumerate(lens):
        qt = torch.from_numpy(q[b]).view(1, NUM_Q_HEADS, 1, HEAD_DIM)
        kt = torch.from_numpy(kv[b, 0, :, :L]).view(1, NUM_KV_HEADS, L, HEAD_DIM)
        vt = torch.from_numpy(kv[b, 1, :, :L]).view(1, NUM_KV_HEADS, L, HEAD_DIM)
        sd = torch.nn.functional.scaled_dot_product_attention(
            qt, kt, vt, scale=qs * ks / math.sqrt(HEAD_DIM), enable_gqa=True)
        np.testing.assert_allclose(ref[b], vs * sd[0, :, 0].numpy(), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- pin 7: grouping
def test_head_h_reads_kv_head_h_div_4():
    rng = np.random.default_rng(8)
    q, kv, _ = _rand_case(rng, 2, 11)
    lens = np.array([11, 4])
    for g in range(NUM_KV_HEADS):
        kv[:, 1, g] = float(g)
    out = gqa_decode_reference(q, kv, lens)
    for h in range(NUM_Q_HEADS):
        np.testing.assert_allclose(out[:, h], float(h // 4), rtol=0, atol=1e-13, err_msg=str(h))


# ---------------------------------------------------------------- closed form
@pytest.mark.parametrize("qs,ks,vs", [(1.0, 1.0, 1.0), (0.5, 1.0 / 64, 1.0 / 64), (3.0, 0.25, 2.0)])
def test_two_token_closed_form(qs, ks, vs):
    """Two keys, k0 = 0, k1 = c*e0: weight of key 1 is the logistic function
    of the score gap qs*ks*q0*c/sqrt(128); out = vs*((1-w)v0 + w v1)."""
    rng = np.random.default_rng(9)
    B, C = 1, 4
    q = np.zeros((B, NUM_Q_HEADS, HEAD_DIM))
    kv = rng.standard_normal((B, 2, NUM_KV_HEADS, C, HEAD_DIM))
    a = np.linspace(-3.0, 3.0, NUM_Q_HEADS)
    q[0, :, 0] = a
    q[0, :, 1:] = rng.standard_normal((NUM_Q_HEADS, HEAD_DIM - 1))
    cvals = np.linspace(0.5, 4.0, NUM_KV_HEADS)
    kv[0, 0, :, 0] = 0.0
    kv[0, 0, :, 1] = 0.0
    kv[0, 0, :, 1, 0] = cvals
    out = gqa_decode_reference(q, kv, [2], qs, ks, vs)
    for h in range(NUM_Q_HEADS):
        g = h // 4
        gap = qs * ks * a[h] * cvals[g] / math.sqrt(128.0)
        w1 = 1.0 / (1.0 + math.exp(-gap))
        want = vs * ((1.0 - w1) * kv[0, 1, g, 0] + w1 * kv[0, 1, g, 1])
        np.testing.assert_allclose(out[0, h], want, rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------- pin 8: limits
def test_one_hot_limit_and_huge_scores():
    """One key whose scaled score beats every other by > 60 nats takes all
    the weight (the rest sum to < 9 * e^-60)."""
    rng = np.random.default_rng(10)
    qrows = rng.standard_normal((GROUP, HEAD_DIM)) * 1e-3
    qrows[:, 0] = 1.0 + np.abs(rng.standard_normal(GROUP))
    k = rng.standard_normal((9, HEAD_DIM)) * 1e-3
    v = rng.standard_normal((9, HEAD_DIM))
    k[4] = 0.0
    k[4, 0] = 61.0 * math.sqrt(HEAD_DIM)
    out = gqa_decode_head(qrows, k, v)
    np.testing.assert_allclose(out, np.tile(v[4], (GROUP, 1)), rtol=0, atol=1e-20)
    # scores of order 1e4 would overflow exp without the max shift
    out2 = gqa_decode_head(qrows, k * 20.0, v)
    assert np.all(np.isfinite(out2))
    np.testing.assert_allclose(out2, np.tile(v[4], (GROUP, 1)), rtol=0, atol=1e-20)


def test_joint_token_permutation_invariance():
    rng = np.random.default_rng(11)
    qrows = rng.standard_normal((GROUP, HEAD_DIM))
    k = rng.standard_normal((37, HEAD_DIM))
    v = rng.standard_normal((37, HEAD_DIM))
    perm = rng.permutation(37)
    a = gqa_decode_head(qrows, k, v, 0.9, 1.1, 0.7)
    b = gqa_decode_head(qrows, k[perm], v[perm], 0.9, 1.1, 0.7)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-14)


# ---------------------------------------------------------------- contract errors
@pytest.mark.parametrize("bad", [0.0, -1.0, float("nan"), float("inf")])
def test_rejects_bad_scales(bad):
    rng = np.random.default_rng(12)
    q, kv, lens = _rand_case(rng, 1, 4)
    with pytest.raises(ValueError):
        gqa_decode_reference(q, kv, lens, q_scale=bad)
    with pytest.raises(ValueError):
        gqa_decode_reference(q, kv, lens, v_scale=bad)


@pytest.mark.parametrize("L", [0, 5])
def test_rejects_lengths_outside_capacity(L):
    rng = np.random.default_rng(13)
    q, kv, _ = _rand_case(rng, 1, 4)
    with pytest.raises(ValueError):
        gqa_decode_reference(q, kv, [L])


# ---------------------------------------------------------------- KV append (fp8 encode)
from oracle.kv_append import encode_e4m3fn, kv_append_reference, quantise_fp8  # noqa: E402


def test_e4m3fn_encode_round_trips_every_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert np.array_equal(encode_e4m3fn(decode_e4m3fn_bits(codes)), codes)


def test_e4m3fn_encode_matches_torch_inside_the_range():
    """Library special case: torch's cast rounds to nearest-even; it agrees
    with ours wherever it does not overflow (|x| <= 464)."""
    bits = np.arange(1 << 16, dtype=np.uint16)
    for vals in (decode_f16_bits(bits), decode_bf16_bits(bits)):
        vals = vals[np.isfinite(vals) & (np.abs(vals) <= 464.0)]
        ref = torch.from_numpy(vals.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(encode_e4m3fn(vals), ref)


def test_e4m3fn_encode_is_nearest_with_ties_to_even_brute_force():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = decode_e4m3fn_bits(codes)
    rng = np.random.default_rng(31)
    pos = np.unique(vals[vals > 0])
    midpoints = (pos[:-1] + pos[1:]) / 2          # exact ties between neighbouring codes
    xs = np.concatenate([rng.uniform(-447.9, 447.9, 3000), rng.uniform(-0.02, 0.02, 3000),
                         midpoints, -midpoints, [pos[0] / 2]])
    got = encode_e4m3fn(xs)
    for x, g in zip(xs, got):
        d = np.abs(vals - x)
        best = np.flatnonzero(d == d.min())
        cand = codes[best]
        if len(cand) > 1:   # a tie: the even mantissa wins (+0 and -0 are one value)
            even = [c for c in cand if (c & 1) == 0 and (math.copysign(1, x) < 0) == bool(c & 0x80)]
            cand = even or [c for c in cand if (c & 1) == 0]
        assert g in cand, (x, hex(g), [hex(c) for c in cand])


def test_e4m3fn_encode_saturates_and_keeps_nan():
    x = np.array([448.0, 449.0, 464.0, 465.0, 1e30, np.inf, -448.5, -np.inf, np.nan, 0.0, -0.0])
    assert [hex(c) for c in encode_e4m3fn(x)] == ["0x7e", "0x7e", "0x7e", "0x7e", "0x7e", "0x7e",
                                                "0xfe", "0xfe", "0x7f", "0x0", "0x80"]


def test_quantise_divides_in_fp32():
    rng = np.random.default_rng(32)
    x = rng.standard_normal(20000).astype(np.float32)
    scale = 0.0137
    ref = (torch.from_numpy(x) / torch.tensor(scale, dtype=torch.float32)).clamp(-448, 448)
    ref = ref.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(quantise_fp8(x, scale), ref)


def test_kv_append_writes_only_the_target_slots():
    rng = np.random.default_rng(33)
    B, C = 3, 7
    kv = rng.integers(0, 256, size=(B, 2, NUM_KV_HEADS, C, HEAD_DIM), dtype=np.uint8)
    k_new = rng.standard_normal((B, NUM_KV_HEADS, HEAD_DIM)).astype(np.float32)
    v_new = rng.standard_normal((B, NUM_KV_HEADS, HEAD_DIM)).astype(np.float32)
    pos = [6, -1, 7]          # request 1 and 2 fall outside [0, C): nothing written
    out = kv_append_reference(kv, k_new, v_new, pos, "fp8_e4m3", 0.25, 0.5)
    assert np.array_equal(out[1:], kv[1:])
    mask = np.ones(C, dtype=bool)
    mask[6] = False
    assert np.array_equal(out[0][:, :, mask], kv[0][:, :, mask])
    assert np.array_equal(out[0, 0, :, 6], quantise_fp8(k_new[0], 0.25))
    assert np.array_equal(decode_e4m3fn_bits(out[0, 1, :, 6]), decode_e4m3fn_bits(quantise_fp8(v_new[0], 0.5)))


# ---------------------------------------------------------------- INT8 KV, 16Q/8KV
from oracle import decode_int8_rows  # noqa: E402


def test_int8_row_decode_matches_torch():
    rng = np.random.default_rng(41)
    vals = rng.integers(-128, 128, size=(5, 7, HEAD_DIM)).astype(np.int8)
    sbits = torch.randn(5, 7).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ref = (torch.from_numpy(vals).double() *
           torch.from_numpy(sbits.view(np.int16)).view(torch.bfloat16).double()[..., None]).numpy()
    assert np.array_equal(decode_int8_rows(vals, sbits), ref)


def test_sixteen_query_heads_read_kv_head_h_div_2():
    rng = np.random.default_rng(42)
    q = rng.standard_normal((2, 16, HEAD_DIM))
    kv = rng.standard_normal((2, 2, NUM_KV_HEADS, 9, HEAD_DIM))
    for g in range(NUM_KV_HEADS):
        kv[:, 1, g] = float(g)
    out = gqa_decode_reference(q, kv, [9, 3])
    for h in range(16):
        np.testing.assert_allclose(out[:, h], float(h // 2), rtol=0, atol=1e-13)


def test_sixteen_query_heads_match_sdpa_and_brute_force():
    rng = np.random.default_rng(43)
    q = rng.standard_normal((2, 16, HEAD_DIM))
    kv = rng.standard_normal((2, 2, NUM_KV_HEADS, 6, HEAD_DIM))
    lens = np.array([6, 2])
    ref = gqa_decode_reference(q, kv, lens, 0.7)
    brute = np.array(brute_decode(q.tolist(), kv.tolist(), lens.tolist(), 0.7))
    np.testing.assert_allclose(ref, brute, rtol=0, atol=1e-12)
    for b, L in enumerate(lens):
        sd = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[b]).view(1, 16, 1, HEAD_DIM),
            torch.from_numpy(kv[b, 0, :, :L]).view(1, 8, L, HEAD_DIM),
            torch.from_numpy(kv[b, 1, :, :L]).view(1, 8, L, HEAD_DIM),
            scale=0.7 / math.sqrt(HEAD_DIM), enable_gqa=True)
        np.testing.assert_allclose(ref[b], sd[0, :, 0].numpy(), rtol=0, atol=1e-12)


def test_int8_row_scales_act_per_token():
    """Closed form: two tokens with equal int8 keys but key scales s0 != s1 give
    weights in ratio exp((s1 - s0) * q.k8 / sqrt(128)); V scales scale each row."""
    k8 = np.zeros((2, HEAD_DIM), dtype=np.int8)
    k8[:, 0] = 10
    v8 = np.zeros((2, HEAD_DIM), dtype=np.int8)
    v8[0, 1], v8[1, 1] = 20, -30
    ks = torch.tensor([0.5, 0.25]).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    vs = torch.tensor([2.0, 0.125]).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    qrows = np.zeros((2, HEAD_DIM))
    qrows[:, 0] = [1.0, -2.0]
    out = gqa_decode_head(qrows, decode_int8_rows(k8, ks), decode_int8_rows(v8, vs))
    for r in range(2):
        gap = qrows[r, 0] * 10 * (0.25 - 0.5) / math.sqrt(HEAD_DIM)
        w1 = 1 / (1 + math.exp(-gap))
        assert out[r, 1] == pytest.approx((1 - w1) * 40.0 + w1 * (-3.75), rel=1e-14)


# ---------------------------------------------------------------- KV append (INT8 rows)
from fractions import Fraction  # noqa: E402

from oracle.kv_append import (  # noqa: E402
    f32_to_bf16_bits,
    kv_append_int8_reference,
    quantise_int8_rows,
)


def _bf16_bits_torch(x32):
    return torch.from_numpy(np.asarray(x32, np.float32)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


def test_bf16_rounding_matches_torch():
    """Library special case: torch's fp32 -> bf16 cast rounds to nearest-even."""
    rng = np.random.default_rng(51)
    x = (rng.standard_normal(50000) * np.exp2(rng.integers(-60, 60, 50000))).astype(np.float32)
    # exact ties (dropped half = 0x8000) with odd and even kept parts, and carries
    # out of the fraction into the exponent
    kept = rng.integers(0x0080, 0x7F70, 4000, dtype=np.uint32)   # finite normals, no carry to Inf
    ties = ((kept << 16) | np.uint32(0x8000)).view(np.float32)
    carry = np.array([0x3FFFFFFF, 0x3FFF8000, 0x3FFF7FFF, 0x407FFFFF], np.uint32).view(np.float32)
    for v in (x, ties, -ties, carry):
        assert np.array_equal(f32_to_bf16_bits(v), _bf16_bits_torch(v))


def test_bf16_rounding_anchor_values():
    vals = np.array([1.0, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 2 - 2.0 ** -9, -0.0, 127 / 127.0],
                    np.float32)
    assert [hex(v) for v in f32_to_bf16_bits(vals)] == \
        ["0x3f80", "0x3f80", "0x3f82", "0x4000", "0x8000", "0x3f80"]


def _row_cases():
    rng = np.random.default_rng(52)
    rows = [rng.standard_normal((6, HEAD_DIM)) * np.exp2(rng.integers(-20, 20, (6, 1))),
            rng.uniform(-1, 1, (4, HEAD_DIM)) * 1e-30,
            rng.integers(-300, 300, (4, HEAD_DIM)).astype(np.float64),   # many exact quotients
            np.eye(4, HEAD_DIM) * 3.5 - 1.25]
    return [r.astype(np.float32) for r in rows]


@pytest.mark.parametrize("scale", [1.0, 0.37, 4.0])
def test_int8_rows_round_trip_within_half_a_step(scale):
    """Decoded through the decode oracle, every stored value is within half a
    quantisation step of y = x / scale; the scale is max|y| / 127 to bf16
    precision; the largest element maps to +-126 or +-127 with its sign."""
    for x in _row_cases():
        codes, sbits = quantise_int8_rows(x, scale)
        y = (x / np.float32(scale)).astype(np.float64)
        s = decode_bf16_bits(sbits)
        amax = np.abs(y).max(axis=1)
        assert np.all(np.abs(s - amax / 127) <= amax / 127 * 2.0 ** -8)
        err = np.abs(decode_int8_rows(codes, sbits) - y)
        assert np.all(err <= 0.5 * s[:, None] * (1 + 1e-6)), err.max()
        top = np.argmax(np.abs(y), axis=1)
        ctop = codes[np.arange(len(x)), top].astype(int)
        assert np.all(np.isin(np.abs(ctop), [126, 127]))
        assert np.all(np.sign(ctop) == np.sign(y[np.arange(len(x)), top]))
        assert np.abs(codes.astype(int)).max() <= 127


def test_int8_rows_codes_are_nearest_integers_brute_force():
    """Each code is the integer nearest to y / s (ties to even) in exact
    arithmetic, clamped to +-127, except where the exact quotient lies within
    2^-16 of a tie and the fp32 quotient's rounding may pick either side."""
    for x in _row_cases():
        codes, sbits = quantise_int8_rows(x[:2], 1.0)
        s = decode_bf16_bits(sbits)
        for r in range(2):
            S = Fraction(float(s[r]))
            for d in range(HEAD_DIM):
                q = Fraction(float(x[r, d])) / S
                lo = math.floor(q)
                frac = q - lo
                if abs(frac - Fraction(1, 2)) < Fraction(1, 1 << 16):
                    assert codes[r, d] in (max(-127, min(127, lo)), max(-127, min(127, lo + 1)))
                    continue
                want = lo + 1 if frac > Fraction(1, 2) else lo
                assert codes[r, d] == max(-127, min(127, want)), (r, d, float(q))


def test_int8_rows_exact_ties_go_to_the_even_code():
    """max|y| = 127 makes the scale exactly 1, so y / s = y: halves are exact
    ties and take the even neighbour (126.5 -> 126, -4.5 -> -4, 3.5 -> 4)."""
    row = np.zeros(HEAD_DIM, np.float32)
    vals = [127.0, 2.5, 3.5, -4.5, 0.5, -0.5, 126.5, -1.5, 5.25, -6.75]
    row[:len(vals)] = vals
    codes, sbits = quantise_int8_rows(row[None], 1.0)
    assert sbits[0] == 0x3F80   # 1.0
    assert codes[0, :len(vals)].tolist() == [127, 2, 4, -4, 0, 0, 126, -2, 5, -7]
    assert not codes[0, len(vals):].any()


def test_int8_rows_zero_rows_sign_symmetry_and_scale_division():
    z = np.zeros((3, HEAD_DIM), np.float32)
    codes, sbits = quantise_int8_rows(z, 1.0)
    assert not codes.any() and not sbits.any()
    for x in _row_cases():
        c, sb = quantise_int8_rows(x, 1.0)
        cn, sbn = quantise_int8_rows(-x, 1.0)
        assert np.array_equal(cn, -c) and np.array_equal(sbn, sb)
        k = np.float32(0.3)
        assert all(np.array_equal(u, v) for u, v in
                   zip(quantise_int8_rows(x, 0.3), quantise_int8_rows((x / k).astype(np.float32), 1.0)))


def test_kv_append_int8_writes_only_the_target_slots():
    rng = np.random.default_rng(53)
    B, C = 3, 7
    codes = rng.integers(-127, 128, size=(B, 2, NUM_KV_HEADS, C, HEAD_DIM)).astype(np.int8)
    sbits = rng.integers(0, 1 << 15, size=(B, 2, NUM_KV_HEADS, C)).astype(np.uint16)
    k_new = rng.standard_normal((B, NUM_KV_HEADS, HEAD_DIM)).astype(np.float32)
    v_new = rng.standard_normal((B, NUM_KV_HEADS, HEAD_DIM)).astype(np.float32)
    out, osc = kv_append_int8_reference(codes, sbits, k_new, v_new, [6, -1, 7], 0.5, 2.0)
    assert np.array_equal(out[1:], codes[1:]) and np.array_equal(osc[1:], sbits[1:])
    mask = np.ones(C, dtype=bool)
    mask[6] = False
    assert np.array_equal(out[0][:, :, mask], codes[0][:, :, mask])
    assert np.array_equal(osc[0][:, :, mask], sbits[0][:, :, mask])
    kc, ks = quantise_int8_rows(k_new[0], 0.5)
    vc, vs = quantise_int8_rows(v_new[0], 2.0)
    assert np.array_equal(out[0, 0, :, 6], kc) and np.array_equal(osc[0, 0, :, 6], ks)
    assert np.array_equal(out[0, 1, :, 6], vc) and np.array_equal(osc[0, 1, :, 6], vs)
