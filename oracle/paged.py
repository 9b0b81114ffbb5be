"""Reference for decode over a paged KV cache with several query tokens per
request (the verify pass of speculative decoding).

TEST INFRASTRUCTURE ONLY: used by tests, never by the product path. It shares
no code with the HIP library; the per-(request, KV head) arithmetic is the
pinned plain definition in ``gqa_oracle.gqa_decode_head``.

What is computed.

* Paged cache. The FreeToken Turing notes (change 2, the automatic attention
  backend) name a paged-KV decode backend that runs under CUDA-graph capture;
  the pages give no layout. Reading taken: a pool ``kv_pages`` of shape
  ``[num_pages, 2, 8, page_size, 128]`` (each page holds the same
  ``[2, 8, slots, 128]`` block as the contiguous cache of the GQA-decode
  article's input contract, for ``page_size`` slots), and an int32 block table
  ``[batch, max_pages]``: slot ``j`` of request ``b`` is row ``j % page_size``
  of page ``block_table[b, j // page_size]``. An INT8 pool carries its row
  scales as ``[num_pages, 2, 8, page_size]`` bf16 (Orin Qwen3-VL doc, "INT8 KV
  cache": one scale per (position, KV head) row), or, as a second layout,
  indexed by the request's position instead of the page:
  ``[batch, 2, 8, max_pages * page_size]``, the scale of slot ``j`` of
  request ``b`` at ``[b, plane, g, j]`` (the contiguous INT8 cache's scale
  layout, whatever page holds the row).
* Several query tokens. The Thor vLLM notes on MTP (K draft tokens per step,
  verified by the target model each step) imply a pass over K + 1 new tokens
  per request. Reading taken: ``T`` query tokens per request, ``q`` of shape
  ``[batch, T, Hq, 128]``; they are the last ``T`` of the ``L`` slots the
  length counts (already written to the cache), and token ``t`` (0-based)
  attends slots ``j < L - T + 1 + t``: causal among the new tokens, everything
  before them visible. ``T = 1`` is the single-token decode.

Everything else (head grouping h // (Hq / 8), the scales, the softmax) is the
single-token definition applied to each (request, token, KV head).

* Appending to a pool. The write before a step (the Thor Qwen3-VL doc,
  "Runtime architecture": decode writes each new token's K and V rows into
  the cache) lands, for new token t of request b, at slot
  ``positions[b] + t`` of the request, i.e. through the block table as above;
  the stored value is the one the contiguous append stores (16-bit: as is;
  fp8: ``kv_append.quantise_fp8``). Readings taken, as for the contiguous
  append: slots outside ``[0, max_pages * page_size)`` and table entries
  outside ``[0, num_pages)`` write nothing.
"""

from __future__ import annotations

import numpy as np

from .gqa_oracle import HEAD_DIM, NUM_KV_HEADS, decode_int8_rows, gqa_decode_head
from .kv_append import quantise_fp8, quantise_int8_rows


def gather_pages(kv_pages: np.ndarray, table_row, length: int, page_size: int) -> np.ndarray:
    """Logical rows [2, 8, length, ...] of one request, slot by slot."""
    kv_pages = np.asarray(kv_pages)
    if page_size < 1 or kv_pages.shape[3] != page_size:
        raise ValueError("page_size must be >= 1 and match kv_pages.shape[3]")
    num_pages = kv_pages.shape[0]
    out = np.empty((2, kv_pages.shape[2], length) + kv_pages.shape[4:], dtype=kv_pages.dtype)
    for j in range(length):
        logical = j // page_size
        if logical >= len(table_row):
            raise ValueError(f"slot {j} needs page {logical}, beyond the block table row")
        page = int(table_row[logical])
        if not 0 <= page < num_pages:
            raise ValueError(f"block table entry {page} outside [0, {num_pages})")
        out[:, :, j] = kv_pages[page, :, :, j % page_size]
    return out


def gqa_decode_multi(q: np.ndarray, kv_rows, seq_lens, q_scale: float = 1.0,
                     k_scale: float = 1.0, v_scale: float = 1.0) -> np.ndarray:
    """q [B, T, Hq, 128]; kv_rows[b] = decoded logical rows [2, 8, >= L_b, 128].

    Returns out [B, T, Hq, 128] (fp64): token t of request b attends slots
    j < L_b - T + 1 + t. Raises when a token would see no slot (L_b < T).
    """
    q = np.asarray(q, dtype=np.float64)
    if q.ndim != 4 or q.shape[2] not in (16, 32) or q.shape[3] != HEAD_DIM:
        raise ValueError(f"q must be [batch, T, 32 or 16, 128], got {q.shape}")
    B, T, Hq, _ = q.shape
    group = Hq // NUM_KV_HEADS
    lens = np.asarray(seq_lens, dtype=np.int64)
    if lens.shape != (B,) or len(kv_rows) != B:
        raise ValueError("batch mismatch between q, kv rows and sequence_lengths")
    out = np.empty_like(q)
    for b in range(B):
        L = int(lens[b])
        kvb = np.asarray(kv_rows[b], dtype=np.float64)
        if L < T or L > kvb.shape[2]:
            raise ValueError(f"request {b}: need T <= L <= its slots (T={T}, L={L})")
        for t in range(T):
            visible = L - T + 1 + t
            for g in range(NUM_KV_HEADS):
                rows = slice(group * g, group * (g + 1))
                out[b, t, rows] = gqa_decode_head(q[b, t, rows], kvb[0, g, :visible],
                                                  kvb[1, g, :visible], q_scale, k_scale, v_scale)
    return out


def gqa_decode_paged_reference(q: np.ndarray, kv_pages: np.ndarray, block_table, seq_lens,
                               page_size: int, q_scale: float = 1.0, k_scale: float = 1.0,
                               v_scale: float = 1.0) -> np.ndarray:
    """q [B, T, Hq, 128]; kv_pages decoded fp64 [num_pages, 2, 8, page_size, 128];
    block_table [B, max_pages] int; returns out [B, T, Hq, 128] (fp64)."""
    kv_pages = np.asarray(kv_pages, dtype=np.float64)
    if kv_pages.ndim != 5 or kv_pages.shape[1:3] != (2, NUM_KV_HEADS) or \
            kv_pages.shape[4] != HEAD_DIM:
        raise ValueError(f"kv_pages must be [num_pages, 2, 8, page_size, 128], got {kv_pages.shape}")
    table = np.asarray(block_table)
    lens = np.asarray(seq_lens, dtype=np.int64)
    if table.ndim != 2 or table.shape[0] != lens.shape[0]:
        raise ValueError("block_table must be [batch, max_pages]")
    if np.any(lens > table.shape[1] * page_size):
        raise ValueError("a length exceeds max_pages * page_size")
    rows = [gather_pages(kv_pages, table[b], int(lens[b]), page_size) for b in range(len(lens))]
    return gqa_decode_multi(q, rows, lens, q_scale, k_scale, v_scale)


def int8_rows_by_position(pool_codes, scale_bits_by_position, block_table, seq_lens,
                          page_size: int):
    """Decoded fp64 logical rows [2, 8, L_b, 128] of every request of an INT8
    pool whose row scales are indexed by position: the codes gathered through
    the block table, times the scales ``scale_bits_by_position[b, :, :, :L_b]``."""
    table = np.asarray(block_table)
    scales = np.asarray(scale_bits_by_position)
    lens = np.asarray(seq_lens, dtype=np.int64)
    if table.ndim != 2 or scales.shape[:3] != (table.shape[0], 2, NUM_KV_HEADS) or \
            scales.shape[3] != table.shape[1] * page_size:
        raise ValueError("scales must be [batch, 2, 8, max_pages * page_size]")
    rows = []
    for b in range(table.shape[0]):
        L = int(lens[b])
        codes = gather_pages(pool_codes, table[b], L, page_size)
        rows.append(decode_int8_rows(codes, scales[b, :, :, :L]))
    return rows


def kv_append_paged_reference(pool_bits: np.ndarray, block_table, positions, k_new_f32,
                              v_new_f32, kv_dtype: str, k_scale: float = 1.0,
                              v_scale: float = 1.0, new_bits=None) -> np.ndarray:
    """Return a copy of the stored pool ``pool_bits`` [num_pages, 2, 8, P, 128]
    after appending T tokens per request.

    k_new_f32 / v_new_f32: [B, T, 8, 128] decoded new rows (fp32-exact values);
    for a 16-bit pool ``new_bits`` = (k_bits, v_bits) [B, T, 8, 128] are the
    stored patterns to copy verbatim. Tokens are written in (b, t) order.
    """
    out = np.array(pool_bits, copy=True)
    num_pages, _, H, P, D = out.shape
    assert H == NUM_KV_HEADS and D == HEAD_DIM
    table = np.asarray(block_table)
    B, max_pages = table.shape
    T = np.asarray(k_new_f32).shape[1]
    for b in range(B):
        for t in range(T):
            s = int(positions[b]) + t
            if s < 0 or s >= max_pages * P:
                continue
            page = int(table[b, s // P])
            if not 0 <= page < num_pages:
                continue
            row = s % P
            if kv_dtype == "fp8_e4m3":
                out[page, 0, :, row, :] = quantise_fp8(k_new_f32[b][t], k_scale)
                out[page, 1, :, row, :] = quantise_fp8(v_new_f32[b][t], v_scale)
            else:
                out[page, 0, :, row, :] = new_bits[0][b][t]
                out[page, 1, :, row, :] = new_bits[1][b][t]
    return out


def kv_append_paged_int8_reference(pool_codes, pool_scale_bits, block_table, positions, k_new_f32,
                                   v_new_f32, k_scale: float = 1.0, v_scale: float = 1.0,
                                   scales_by_position: bool = False):
    """Return copies of an INT8 pool (codes [num_pages, 2, 8, P, 128], bf16
    scale bits [num_pages, 2, 8, P], or [B, 2, 8, max_pages * P] with
    ``scales_by_position``) after appending T tokens per request, each row
    quantised as in kv_append.quantise_int8_rows. Slots and pages are found
    as in kv_append_paged_reference; a token whose slot or page is skipped
    writes no scale either. Tokens are written in (b, t) order."""
    codes = np.array(pool_codes, copy=True)
    scales = np.array(pool_scale_bits, copy=True)
    num_pages, _, H, P, D = codes.shape
    table = np.asarray(block_table)
    B, max_pages = table.shape
    assert H == NUM_KV_HEADS and D == HEAD_DIM
    if scales_by_position:
        assert scales.shape == (B, 2, H, max_pages * P)
    else:
        assert scales.shape == (num_pages, 2, H, P)
    T = np.asarray(k_new_f32).shape[1]
    for b in range(B):
        for t in range(T):
            s = int(positions[b]) + t
            if s < 0 or s >= max_pages * P:
                continue
            page = int(table[b, s // P])
            if not 0 <= page < num_pages:
                continue
            row = s % P
            for plane, (new, scale) in enumerate(((k_new_f32, k_scale), (v_new_f32, v_scale))):
                c, sb = quantise_int8_rows(new[b][t], scale)
                codes[page, plane, :, row, :] = c
                if scales_by_position:
                    scales[b, plane, :, s] = sb
                else:
                    scales[page, plane, :, row] = sb
    return codes, scales
