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
"""

from __future__ import annotations

import numpy as np

from .gqa_oracle import HEAD_DIM, NUM_KV_HEADS

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
