"""Reference for appending one token's K and V rows to the cache (with fp8
quantise-on-write).

TEST INFRASTRUCTURE ONLY: used by tests, never by the product path.

What is computed. Every decode step first writes the new token's K and V
into the cache before attention reads it (the Thor Qwen3-VL doc, "Runtime
architecture", RoPE-and-KV-writes paragraph: decode writes one row per token
into the cache). The write lands at slot `positions[b]` of every KV head of
request b in the `[batch, 2, 8, capacity, 128]` layout of the GQA-decode
article's input contract. A 16-bit cache stores the value as is. An fp8
cache stores `x / scale` as an OCP E4M3FN byte, the per-tensor scale of the
Thor FP8-KV notes (section 1: K with k_scale, V with v_scale; the cache is
uint8 bytes reinterpreted as float8_e4m3fn).

Readings taken: the division happens in fp32 (the kernel's precision, so both
sides take the rounding decision identically); the result is rounded to
nearest, ties to even; magnitudes at or above 448 (the largest finite E4M3FN
value) saturate to +-448 instead of becoming NaN; a NaN input stores the NaN
code 0x7F; positions outside [0, capacity) write nothing.

An INT8 cache (the Orin Qwen3-VL doc, "INT8 KV cache": INT8 mirrors with one
BF16 scale per (position, KV head) row) is written row by row. The doc does
not say how a row is quantised; the same doc quantises its INT8 weights
symmetrically with scale = amax / 127 ("Weight quantization" table), and that
reading is taken per row: y = x / k_scale (or v_scale), scale = max|y| / 127
rounded to bf16, code = y / scale rounded to the nearest integer (ties to
even) and clamped to +-127. Every division is an fp32 division and every
rounding decision is taken on fp32 values, the kernel's precision. A row
whose bf16 scale is 0 (all zeros) stores code 0.
"""

from __future__ import annotations

import numpy as np

from .gqa_oracle import HEAD_DIM, NUM_KV_HEADS, decode_bf16_bits

E4M3_MAX = 448.0


def encode_e4m3fn(x) -> np.ndarray:
    """Round each value to the nearest OCP E4M3FN code (ties to even), saturating.

    Written from the format definition: sign bit 7; exponent field 1..15 with
    bias 7 holds normals (1 + m/8) * 2^(e-7); field 0 holds subnormals
    (m/8) * 2^-6; 0x7F / 0xFF are NaN.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros(x.shape, dtype=np.uint8)
    sign = np.where(np.signbit(x), 0x80, 0).astype(np.uint8)
    a = np.abs(x)
    nan = np.isnan(x)
    sat = ~nan & (a >= E4M3_MAX)
    sub = ~nan & ~sat & (a < 2.0 ** -6)
    nor = ~nan & ~sat & ~sub
    # subnormals: a = m * 2^-9, m = 0..8 (m = 8 is the smallest normal, code 0x08)
    m_sub = np.rint(a[sub] * 2.0 ** 9).astype(np.int64)      # np.rint: ties to even
    out[sub] = m_sub.astype(np.uint8)
    # normals: a = (1 + f) * 2^e, e = -6..8
    an = a[nor]
    e = np.floor(np.log2(an)).astype(np.int64)
    # guard against log2 rounding at exact powers of two
    e = np.where(np.ldexp(1.0, e) > an, e - 1, e)
    e = np.where(np.ldexp(1.0, e + 1) <= an, e + 1, e)
    q = np.rint((an / np.ldexp(1.0, e) - 1.0) * 8.0).astype(np.int64)
    carry = q == 8
    q = np.where(carry, 0, q)
    e = np.where(carry, e + 1, e)
    out[nor] = (((e + 7) << 3) | q).astype(np.uint8)
    out[sat] = 0x7E
    out |= sign
    out[nan] = 0x7F
    return out


def quantise_fp8(values_f32, scale: float) -> np.ndarray:
    """fp32 x / fp32 scale (IEEE, round to nearest), then E4M3FN with saturation."""
    v = np.asarray(values_f32, dtype=np.float32)
    with np.errstate(all="ignore"):
        q = v / np.float32(scale)
    return encode_e4m3fn(q.astype(np.float64))


def kv_append_reference(kv_bits: np.ndarray, k_new_f32: np.ndarray, v_new_f32: np.ndarray,
                        positions, kv_dtype: str, k_scale: float = 1.0,
                        v_scale: float = 1.0, new_bits=None) -> np.ndarray:
    """Return a copy of the stored cache `kv_bits` [B,2,8,C,128] after the append.

    k_new_f32 / v_new_f32: [B, 8, 128] decoded new rows (fp32-exact values).
    For a 16-bit cache `new_bits` = (k_bits, v_bits) gives the stored patterns
    to copy verbatim (a 16-bit append is a copy).
    """
    out = np.array(kv_bits, copy=True)
    B, _, H, C, D = out.shape
    assert H == NUM_KV_HEADS and D == HEAD_DIM
    for b in range(B):
        p = int(positions[b])
        if p < 0 or p >= C:
            continue
        if kv_dtype == "fp8_e4m3":
            out[b, 0, :, p, :] = quantise_fp8(k_new_f32[b], k_scale)
            out[b, 1, :, p, :] = quantise_fp8(v_new_f32[b], v_scale)
        else:
            out[b, 0, :, p, :] = new_bits[0][b]
            out[b, 1, :, p, :] = new_bits[1][b]
    return out


INT8_MAX = 127


def f32_to_bf16_bits(values_f32) -> np.ndarray:
    """Round finite fp32 values to bfloat16 (nearest, ties to even); bit patterns.

    bf16 keeps the sign, the 8-bit exponent and the top 7 fraction bits of an
    fp32. Rounding the dropped 16 bits: add just under half of the kept
    unit (0x7FFF), plus one more when the kept part is odd, so an exact half
    goes to the even neighbour; a carry out of the fraction moves into the
    exponent, which is the next binade's correct value.
    """
    b = np.asarray(values_f32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


def quantise_int8_rows(values_f32, scale: float):
    """Rows [..., 128] of fp32 values -> (int8 codes [..., 128], bf16 scale bits [...]).

    y = x / scale; s = bf16(max|y| / 127); code = rint(y / s) clamped to
    +-127 (0 where s is 0). All arithmetic in fp32 (see the module notes).
    """
    x = np.asarray(values_f32, dtype=np.float32)
    with np.errstate(all="ignore"):
        y = (x / np.float32(scale)).astype(np.float32)
        amax = np.max(np.abs(y), axis=-1)
        s_bits = f32_to_bf16_bits((amax / np.float32(INT8_MAX)).astype(np.float32))
        s = decode_bf16_bits(s_bits).astype(np.float32)   # exact
        q = np.rint((y / s[..., None]).astype(np.float32))   # np.rint: ties to even
    q = np.where(s[..., None] > 0, q, 0.0)
    codes = np.clip(q, -INT8_MAX, INT8_MAX).astype(np.int8)
    return codes, s_bits


def kv_append_int8_reference(kv_codes, scale_bits, k_new_f32, v_new_f32, positions,
                             k_scale: float = 1.0, v_scale: float = 1.0):
    """Return copies of an INT8 cache (codes [B,2,8,C,128], bf16 scale bits
    [B,2,8,C]) after appending one token per request: the K row of KV head g
    of request b goes to slot positions[b] of plane 0 with its row scale, the
    V row to plane 1. Positions outside [0, C) write nothing."""
    codes = np.array(kv_codes, copy=True)
    scales = np.array(scale_bits, copy=True)
    B, _, H, C, D = codes.shape
    assert H == NUM_KV_HEADS and D == HEAD_DIM and scales.shape == (B, 2, H, C)
    for b in range(B):
        p = int(positions[b])
        if p < 0 or p >= C:
            continue
        codes[b, 0, :, p, :], scales[b, 0, :, p] = quantise_int8_rows(k_new_f32[b], k_scale)
        codes[b, 1, :, p, :], scales[b, 1, :, p] = quantise_int8_rows(v_new_f32[b], v_scale)
    return codes, scales
