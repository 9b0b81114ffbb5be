"""fp64 reference for single-token grouped-query decode attention over a KV cache.

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke entry and the
benchmark's CPU-baseline leg, never by the product path.

What is computed (sources are the pages this project follows):

* Geometry. One query token per request, 32 query heads sharing 8 KV heads
  (4:1 grouping) at head dimension 128. The query is ``[batch, 32, 128]``;
  the cache is ``[batch, 2, 8, capacity, 128]`` with plane 0 = K and
  plane 1 = V; ``capacity`` is the cache's token-slot count.
  [FlashInfer sm110_gqa_decode article (cf-1.com news 5454068),
  sections "why a separate SM110 GQA decode path" and "input contract".]
* Head mapping. The kernel is handed ``q.view(batch, 8, 4, 128)`` transposed
  to ``[batch, 4, 8, 128]``, so query head ``h`` belongs to KV head ``h // 4``.
  [same article, "convenience API" (the q.view/transpose call) and the
  launch-header description of EncodeQ.] The 16-query-head geometry of the
  INT8-KV decode (Orin Qwen3-VL doc, "INT8 KV cache": GQA 16Q/8KV) groups
  2 query heads per KV head the same way: head ``h`` reads KV head ``h // 2``.
* INT8 cache. One bf16 scale per (position, KV head) row: K = int8 * k_row_scale,
  V = int8 * v_row_scale [same doc, same section]; decoded by decode_int8_rows.
* Lengths. ``sequence_lengths[b]`` tokens of slot prefix ``[0, L)`` are the
  keys/values of request ``b``; slots ``>= L`` are not part of the attention.
  The pages make ``1 <= L <= capacity`` the caller's duty; the oracle raises
  on anything else. [same article, "input contract".]
* Scale. Scores are ``q_scale / sqrt(128) * dot(q, k)``. The GPU evaluates the
  same thing in the log2 domain with exp2 and ``q_scale/sqrt(128)/ln 2``
  folded in; exp2(x/ln2) == exp(x), so the oracle uses exp in fp64.
  [same article, "convenience API", the softmax_scale_log2 paragraph.]
* fp8 KV. With an fp8_e4m3 cache the scores are multiplied by ``k_scale`` and
  the normalised output by ``v_scale`` (both per-tensor). The fp8 bytes are a
  bit reinterpretation of ``torch.float8_e4m3fn`` (OCP E4M3FN), not a numeric
  conversion. [Qwen3.8-Flash-Next on Jetson AGX Thor: FP8 KV cache porting
  notes (kipfel.ltd), section 1, patch 1 items 4-6 and patch 2.]

The result is the plain definition written out, in fp64:

    s_j  = q_scale * k_scale / sqrt(128) * sum_d q[b,h,d] * K[b,h//4,j,d]
    p_j  = exp(s_j - max_i s_i) / sum_i exp(s_i - max_i s_i)      (j < L)
    out  = v_scale * sum_j p_j * V[b,h//4,j,:]

Readings taken where the pages are silent: the scales act on the exact fp32/
fp64 score (q is never pre-rounded with q_scale), k_scale = v_scale = 1 for
16-bit caches, and the output is returned in fp64 (callers round it).
"""

from __future__ import annotations

import math

import numpy as np

NUM_Q_HEADS = 32
NUM_KV_HEADS = 8
GROUP = NUM_Q_HEADS // NUM_KV_HEADS  # 4 query heads per KV head
HEAD_DIM = 128


# --------------------------------------------------------------------------
# Exact decoders of the stored formats.
# --------------------------------------------------------------------------

def decode_e4m3fn_bits(codes: np.ndarray) -> np.ndarray:
    """Decode OCP FP8 E4M3FN bytes to fp64, from the format's definition.

    E4M3FN is what ``torch.float8_e4m3fn`` stores (Thor FP8 KV notes, patch 1
    item 5: the uint8 cache is reinterpreted as float8_e4m3fn). Layout: sign
    bit 7, exponent bits 6..3 with bias 7, mantissa bits 2..0. Exponent field 0
    encodes subnormals ``2^-6 * m/8``; the all-ones pattern ``S.1111.111`` is
    NaN and there are no infinities, so exponent field 15 with mantissa 0..6
    is an ordinary normal number (largest 448).
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    exp_field = (c >> 3) & 0xF
    mant = (c & 0x7).astype(np.float64)
    normal = sign * np.ldexp(1.0 + mant / 8.0, (exp_field - 7).astype(np.int64))
    subnormal = sign * np.ldexp(mant / 8.0, -6)
    out = np.where(exp_field == 0, subnormal, normal)
    out = np.where((exp_field == 15) & ((c & 0x7) == 7), np.nan, out)
    return out


def e4m3fn_table() -> np.ndarray:
    """The 256 E4M3FN code values as fp64, index = code byte.

    Built once by running decode_e4m3fn_bits (the format definition above) on
    every code; a copy is returned so callers cannot alter the cached table.
    """
    global _E4M3FN_TABLE
    if _E4M3FN_TABLE is None:
        _E4M3FN_TABLE = decode_e4m3fn_bits(np.arange(256, dtype=np.uint8))
    return _E4M3FN_TABLE.copy()


_E4M3FN_TABLE = None


def decode_e4m3fn_lookup(codes: np.ndarray) -> np.ndarray:
    """decode_e4m3fn_bits by table lookup: the same values, one gather per byte.

    The uint8 cache bytes are the float8_e4m3fn bit patterns (Thor FP8 KV
    notes, patch 1 item 5), so decoding a byte is indexing the 256-entry
    table of decoded codes; this is what makes a full-size fp8 cache
    (gigabytes of codes) affordable on the CPU.
    """
    if _E4M3FN_TABLE is None:
        e4m3fn_table()
    return _E4M3FN_TABLE[np.asarray(codes, dtype=np.uint8)]


def decode_bf16_bits(bits: np.ndarray) -> np.ndarray:
    """Decode bfloat16 bit patterns to fp64 (bf16 is the top half of an fp32)."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):   # signalling-NaN patterns stay NaN
        return b.view(np.float32).astype(np.float64)


def decode_f16_bits(bits: np.ndarray) -> np.ndarray:
    """Decode IEEE binary16 bit patterns to fp64."""
    return np.asarray(bits).astype(np.uint16).view(np.float16).astype(np.float64)


def decode_int8_rows(values: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    """INT8 cache rows with one bf16 scale per row: value = int8 * scale.

    The Orin Qwen3-VL doc ("INT8 KV cache") keeps INT8 mirrors of the cache
    with one BF16 scale per (position, KV head) row. ``values`` [..., D] are
    the int8 entries, ``scale_bits`` [...] the bf16 bit patterns of the row
    scales; the product is exact in fp64.
    """
    v = np.asarray(values).astype(np.int8).astype(np.float64)
    return v * decode_bf16_bits(scale_bits)[..., None]


def decode_storage(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Decode a raw stored array (``uint16`` for f16/bf16, ``uint8`` for fp8)."""
    if dtype == "f16":
        return decode_f16_bits(bits)
    if dtype == "bf16":
        return decode_bf16_bits(bits)
    if dtype == "fp8_e4m3":
        return decode_e4m3fn_lookup(bits)
    raise ValueError(f"unknown storage dtype {dtype!r}")


# --------------------------------------------------------------------------
# The decode step.
# --------------------------------------------------------------------------

def _check_scales(q_scale: float, k_scale: float, v_scale: float) -> None:
    # The pages require q_scale finite and > 0 (prepared-API differences,
    # item 2); the per-tensor fp8 scales are taken to obey the same rule.
    for name, v in (("q_scale", q_scale), ("k_scale", k_scale), ("v_scale", v_scale)):
        if not (math.isfinite(v) and v > 0.0):
            raise ValueError(f"{name} must be finite and > 0, got {v!r}")


def gqa_decode_head(q_rows: np.ndarray, k: np.ndarray, v: np.ndarray,
                    q_scale: float = 1.0, k_scale: float = 1.0,
                    v_scale: float = 1.0, return_weights: bool = False):
    """One (request, KV head): ``q_rows`` [G, D] against K, V [L, D] (fp64).

    Returns the [G, D] output (and the [G, L] softmax weights if asked).
    ``k``/``v`` must already be cut to the valid prefix ``[0, L)``.
    """
    _check_scales(q_scale, k_scale, v_scale)
    q_rows = np.asarray(q_rows, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if k.shape[0] < 1 or k.shape != v.shape or q_rows.shape[1] != k.shape[1]:
        raise ValueError("need L >= 1 keys and matching K/V/q shapes")
    scale = q_scale * k_scale / math.sqrt(HEAD_DIM)
    scores = scale * (q_rows @ k.T)                       # [G, L]
    shifted = scores - scores.max(axis=1, keepdims=True)
    e = np.exp(shifted)
    w = e / e.sum(axis=1, keepdims=True)                  # [G, L]
    out = v_scale * (w @ v)                               # [G, D]
    return (out, w) if return_weights else out


def _check_geometry(q: np.ndarray, kv: np.ndarray, seq_lens: np.ndarray):
    # 32 query heads per request (4 per KV head), or 16 (2 per KV head, the
    # INT8-KV decode geometry of the Orin Qwen3-VL doc).
    if q.ndim != 3 or q.shape[1] not in (16, 32) or q.shape[2] != HEAD_DIM:
        raise ValueError(f"q must be [batch, 32 or 16, 128], got {q.shape}")
    if kv.ndim != 5 or kv.shape[1:3] != (2, NUM_KV_HEADS) or kv.shape[4] != HEAD_DIM:
        raise ValueError(f"kv must be [batch, 2, 8, capacity, 128], got {kv.shape}")
    if kv.shape[0] != q.shape[0] or np.shape(seq_lens) != (q.shape[0],):
        raise ValueError("batch mismatch between q, kv and sequence_lengths")
    cap = kv.shape[3]
    lens = np.asarray(seq_lens, dtype=np.int64)
    if np.any(lens < 1) or np.any(lens > cap):
        raise ValueError("sequence_lengths must lie in [1, capacity]")
    return lens


def gqa_decode_reference(q: np.ndarray, kv: np.ndarray, seq_lens,
                         q_scale: float = 1.0, k_scale: float = 1.0,
                         v_scale: float = 1.0) -> np.ndarray:
    """Full decode step: q [B,32,128], kv [B,2,8,C,128] (decoded fp64) -> [B,32,128] fp64."""
    q = np.asarray(q, dtype=np.float64)
    kv = np.asarray(kv, dtype=np.float64)
    lens = _check_geometry(q, kv, seq_lens)
    group = q.shape[1] // NUM_KV_HEADS
    out = np.empty_like(q)
    for b in range(q.shape[0]):
        L = int(lens[b])
        for g in range(NUM_KV_HEADS):
            rows = slice(group * g, group * (g + 1))   # heads h with h // group == g
            out[b, rows] = gqa_decode_head(q[b, rows], kv[b, 0, g, :L], kv[b, 1, g, :L],
                                           q_scale, k_scale, v_scale)
    return out


def gqa_decode_weights(q: np.ndarray, kv: np.ndarray, seq_lens,
                       q_scale: float = 1.0, k_scale: float = 1.0):
    """Softmax weights per (b, h): list over b of [32, L_b] fp64 arrays."""
    q = np.asarray(q, dtype=np.float64)
    kv = np.asarray(kv, dtype=np.float64)
    lens = _check_geometry(q, kv, seq_lens)
    group = q.shape[1] // NUM_KV_HEADS
    res = []
    for b in range(q.shape[0]):
        L = int(lens[b])
        w = np.empty((q.shape[1], L))
        for g in range(NUM_KV_HEADS):
            rows = slice(group * g, group * (g + 1))
            _, w[rows] = gqa_decode_head(q[b, rows], kv[b, 0, g, :L], kv[b, 1, g, :L],
                                         q_scale, k_scale, 1.0, return_weights=True)
        res.append(w)
    return res
