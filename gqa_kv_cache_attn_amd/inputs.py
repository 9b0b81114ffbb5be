"""Seeded synthetic workloads for single-token GQA decode.

This module is shared by the tests, the smoke entry and the benchmark. It
holds no arithmetic of the decode method itself: it only draws the inputs
(lengths, query, cache) and encodes them into the stored formats, so both the
HIP path and the CPU oracle can consume identical bytes.

Workloads follow the shapes the pages describe: 32 query heads sharing 8 KV
heads at head_dim 128, a ``[batch, 2, 8, capacity, 128]`` cache, per-request
int32 lengths (FlashInfer sm110_gqa_decode article, "input contract"), an
fp8_e4m3 cache that stores ``x / scale`` as ``float8_e4m3fn`` bytes with
per-tensor scales (Thor FP8 KV notes, section 1, patches 1 and 2), and an
INT8 cache with one bf16 scale per (position, KV head) row at 16 query heads
(Qwen3-VL on Jetson Orin doc, "INT8 KV cache").

Recipe: ``torch.Generator`` on the target device seeded with ``seed``; draw
order is lengths (``randint(lo, hi + 1)``), then q (fp32 N(0,1), cast RNE),
then the cache one request at a time (fp32 N(0,1) over both planes, cast RNE;
for fp8 divided by the plane's scale, clamped to +-448, cast to e4m3fn; for
int8 each 128-value row gets the scale max|x| / 127 rounded to bf16, and the
values round(x / scale) clamped to +-127). Slots past a request's length
receive the same N(0,1) draw: garbage the kernel must never read.

Paged workloads (page_size > 0) draw lengths, then q [B, T, Hq, 128], then a
block table (a random permutation of the pool's page ids, so consecutive
slots of a request sit in scattered pages), then the pool page by page with
the same per-dtype encoding; the pool holds a few spare pages no request
uses.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import torch

NUM_Q_HEADS = 32
NUM_KV_HEADS = 8
HEAD_DIM = 128
E4M3_MAX = 448.0

_TORCH_DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    capacity: int
    len_lo: int
    len_hi: int
    q_dtype: str            # "f16" | "bf16"; the output uses the same dtype
    kv_dtype: str           # "f16" | "bf16" | "fp8_e4m3" | "int8"
    q_scale: float = 1.0
    k_scale: float = 1.0
    v_scale: float = 1.0
    seed: int = 0
    num_q_heads: int = NUM_Q_HEADS   # 32, or 16 (2 query heads per KV head)
    page_size: int = 0               # > 0: paged pool of this many slots per page
    q_tokens: int = 1                # query tokens per request (paged workloads)

    def describe(self) -> dict:
        d = {
            "workload": self.name, "batch": self.batch, "capacity": self.capacity,
            "seq_len": [self.len_lo, self.len_hi], "q_heads": self.num_q_heads,
            "kv_heads": NUM_KV_HEADS, "head_dim": HEAD_DIM, "q_dtype": self.q_dtype,
            "kv_dtype": self.kv_dtype, "q_scale": self.q_scale,
            "k_scale": self.k_scale, "v_scale": self.v_scale, "seed": self.seed,
        }
        if self.page_size:
            d.update(page_size=self.page_size, q_tokens=self.q_tokens)
        return d


# The five workloads of the main geometry, then the INT8 row-scaled cache at
# 16 query heads: the doc's 1581-token prompt in a 4096-slot cache, and a
# long-context batch sized like the fp8 one. Seeds are 1000 + (1-based position).
WORKLOADS = [
    Workload("gqa_decode_b1_c64_f16", 1, 64, 64, 64, "f16", "f16", seed=1001),
    Workload("gqa_decode_b1_c1024_f16", 1, 1024, 1024, 1024, "f16", "f16", seed=1002),
    Workload("gqa_decode_b32_c8192_f16_ragged", 32, 8192, 1, 8192, "f16", "f16", seed=1003),
    Workload("gqa_decode_b8_c65536_bf16_long", 8, 65536, 32768, 65536, "bf16", "bf16",
             q_scale=0.5, seed=1004),
    Workload("gqa_decode_b16_c131072_fp8kv_long", 16, 131072, 65536, 131072, "bf16",
             "fp8_e4m3", k_scale=1.0 / 64, v_scale=1.0 / 64, seed=1005),
    Workload("gqa_decode_b1_c4096_int8kv_16q", 1, 4096, 1581, 1581, "bf16", "int8", seed=1006,
             num_q_heads=16),
    Workload("gqa_decode_b16_c131072_int8kv_16q_long", 16, 131072, 65536, 131072, "bf16", "int8",
             seed=1007, num_q_heads=16),
]

# Paged pool, several query tokens per request: the verify pass of a step
# with 2 draft tokens (T = 3) over 16-slot pages, the 64k bf16 shape; a
# single-token fp8 pool of 64-slot pages, the 128k fp8 shape; and an INT8
# pool with row scales at 16 query heads verifying one draft token (T = 2),
# the 128k INT8 shape.
PAGED_WORKLOADS = [
    Workload("gqa_decode_paged_b8_c65536_p16_bf16_t3", 8, 65536, 32768, 65536, "bf16", "bf16",
             q_scale=0.5, seed=1008, page_size=16, q_tokens=3),
    Workload("gqa_decode_paged_b16_c131072_p64_fp8kv_t1", 16, 131072, 65536, 131072, "bf16",
             "fp8_e4m3", k_scale=1.0 / 64, v_scale=1.0 / 64, seed=1009, page_size=64, q_tokens=1),
    Workload("gqa_decode_paged_b16_c131072_p64_int8kv_16q_t2", 16, 131072, 65536, 131072, "bf16",
             "int8", seed=1010, num_q_heads=16, page_size=64, q_tokens=2),
]
WORKLOADS_BY_NAME = {w.name: w for w in WORKLOADS + PAGED_WORKLOADS}


def kv_elem_bytes(kv_dtype: str) -> int:
    return 1 if kv_dtype in ("fp8_e4m3", "int8") else 2


def kv_slot_bytes(kv_dtype: str) -> int:
    """Bytes one cache slot of one KV head holds for K and V together (row scales included)."""
    return 2 * (HEAD_DIM * kv_elem_bytes(kv_dtype) + (2 if kv_dtype == "int8" else 0))


def _encode_fp8(x: torch.Tensor, scale: float) -> torch.Tensor:
    y = (x / scale).clamp_(-E4M3_MAX, E4M3_MAX)
    return y.to(torch.float8_e4m3fn).view(torch.uint8)


def _encode_int8_rows(x: torch.Tensor):
    """Rows of x [..., 128] -> (int8 values, bf16 scales [...]): scale = max|x| / 127 in bf16."""
    scale = (x.abs().amax(dim=-1) / 127.0).clamp_(min=2.0 ** -100).to(torch.bfloat16)
    v = torch.round(x / scale.float().unsqueeze(-1)).clamp_(-127, 127).to(torch.int8)
    return v, scale


def make_inputs(w: Workload, device="cpu", seed: Optional[int] = None,
                seq_lens: Optional[torch.Tensor] = None, capacity: Optional[int] = None,
                batch: Optional[int] = None):
    """Draw one workload. Returns a dict of device tensors plus the scales.

    ``kv`` is fp16/bf16 for 16-bit caches and ``uint8`` (e4m3fn bytes) for fp8.
    ``seq_lens`` overrides the drawn lengths (the draw still happens so the
    rest of the stream is unchanged); ``capacity``/``batch`` override shape.
    """
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed if seed is None else seed)
    B = w.batch if batch is None else batch
    C = w.capacity if capacity is None else capacity
    lo, hi = min(w.len_lo, C), min(w.len_hi, C)
    lens = torch.randint(lo, hi + 1, (B,), generator=gen, device=dev, dtype=torch.int64)
    lens = lens.to(torch.int32)
    if seq_lens is not None:
        lens = seq_lens.to(device=dev, dtype=torch.int32).clone()
    q32 = torch.randn(B, w.num_q_heads, HEAD_DIM, generator=gen, device=dev, dtype=torch.float32)
    q = q32.to(_TORCH_DTYPES[w.q_dtype])
    del q32
    kv_scales = None
    if w.kv_dtype == "fp8_e4m3":
        kv = torch.empty(B, 2, NUM_KV_HEADS, C, HEAD_DIM, device=dev, dtype=torch.uint8)
    elif w.kv_dtype == "int8":
        kv = torch.empty(B, 2, NUM_KV_HEADS, C, HEAD_DIM, device=dev, dtype=torch.int8)
        kv_scales = torch.empty(B, 2, NUM_KV_HEADS, C, device=dev, dtype=torch.bfloat16)
    else:
        kv = torch.empty(B, 2, NUM_KV_HEADS, C, HEAD_DIM, device=dev,
                         dtype=_TORCH_DTYPES[w.kv_dtype])
    for b in range(B):
        x = torch.randn(2, NUM_KV_HEADS, C, HEAD_DIM, generator=gen, device=dev,
                        dtype=torch.float32)
        if w.kv_dtype == "fp8_e4m3":
            kv[b, 0] = _encode_fp8(x[0], w.k_scale)
            kv[b, 1] = _encode_fp8(x[1], w.v_scale)
        elif w.kv_dtype == "int8":
            kv[b], kv_scales[b] = _encode_int8_rows(x)
        else:
            kv[b] = x.to(kv.dtype)
        del x
    return {"q": q, "kv": kv, "kv_scales": kv_scales, "seq_lens": lens, "q_scale": w.q_scale,
            "k_scale": w.k_scale, "v_scale": w.v_scale, "q_dtype": w.q_dtype,
            "kv_dtype": w.kv_dtype}


def _encode_block(x: torch.Tensor, w: Workload):
    """fp32 N(0,1) block [..., 2, 8, S, 128] -> (stored values, bf16 row scales or None)."""
    if w.kv_dtype == "fp8_e4m3":
        return torch.stack([_encode_fp8(x[..., 0, :, :, :], w.k_scale),
                            _encode_fp8(x[..., 1, :, :, :], w.v_scale)], dim=-4), None
    if w.kv_dtype == "int8":
        return _encode_int8_rows(x)
    return x.to(_TORCH_DTYPES[w.kv_dtype]), None


def make_paged_inputs(w: Workload, device="cpu", seed: Optional[int] = None,
                      seq_lens: Optional[torch.Tensor] = None, spare_pages: int = 5,
                      pages_per_draw: int = 4096, scales_by_position: bool = False):
    """Draw one paged workload: q [B, T, Hq, 128], the pool [num_pages, 2, 8, P, 128]
    (+ row scales for int8), block_table [B, max_pages] int32 and the lengths.
    scales_by_position (int8): the same draw, with the row scales moved to
    [B, 2, 8, max_pages * P] (position_scales)."""
    assert w.page_size > 0
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed if seed is None else seed)
    B, C, P, T = w.batch, w.capacity, w.page_size, w.q_tokens
    lo, hi = min(w.len_lo, C), min(w.len_hi, C)
    lens = torch.randint(lo, hi + 1, (B,), generator=gen, device=dev, dtype=torch.int64)
    lens = lens.to(torch.int32)
    if seq_lens is not None:
        lens = seq_lens.to(device=dev, dtype=torch.int32).clone()
    q32 = torch.randn(B, T, w.num_q_heads, HEAD_DIM, generator=gen, device=dev,
                      dtype=torch.float32)
    q = q32.to(_TORCH_DTYPES[w.q_dtype])
    del q32
    max_pages = (C + P - 1) // P
    num_pages = B * max_pages + spare_pages
    perm = torch.randperm(num_pages, generator=gen, device=dev)
    table = perm[:B * max_pages].reshape(B, max_pages).to(torch.int32).contiguous()
    store = {"fp8_e4m3": torch.uint8, "int8": torch.int8}.get(w.kv_dtype)
    pool = torch.empty(num_pages, 2, NUM_KV_HEADS, P, HEAD_DIM, device=dev,
                       dtype=store if store is not None else _TORCH_DTYPES[w.kv_dtype])
    scales = (torch.empty(num_pages, 2, NUM_KV_HEADS, P, device=dev, dtype=torch.bfloat16)
              if w.kv_dtype == "int8" else None)
    for p0 in range(0, num_pages, pages_per_draw):
        n = min(pages_per_draw, num_pages - p0)
        x = torch.randn(n, 2, NUM_KV_HEADS, P, HEAD_DIM, generator=gen, device=dev,
                        dtype=torch.float32)
        vals, sc = _encode_block(x, w)
        pool[p0:p0 + n] = vals
        if scales is not None:
            scales[p0:p0 + n] = sc
        del x, vals, sc
    if scales_by_position:
        assert scales is not None, "scales_by_position needs an int8 pool"
        scales = position_scales(scales, table, P)
    return {"q": q, "kv_pages": pool, "kv_scales": scales, "block_table": table,
            "seq_lens": lens, "q_scale": w.q_scale, "k_scale": w.k_scale, "v_scale": w.v_scale,
            "q_dtype": w.q_dtype, "kv_dtype": w.kv_dtype, "page_size": P,
            "scales_by_position": scales_by_position}


def position_scales(kv_scales: torch.Tensor, block_table: torch.Tensor,
                    page_size: int) -> torch.Tensor:
    """An INT8 pool's row scales moved from the page layout [num_pages, 2, 8, P]
    to the position layout [batch, 2, 8, max_pages * P]: the scale of request
    b's slot j is the one stored beside that slot's row (table entries are
    clamped into the pool, as the kernels clamp them)."""
    B, max_pages = block_table.shape
    ids = block_table.long().clamp(0, kv_scales.shape[0] - 1).reshape(-1)
    g = kv_scales.index_select(0, ids).reshape(B, max_pages, 2, NUM_KV_HEADS, page_size)
    return g.permute(0, 2, 3, 1, 4).reshape(B, 2, NUM_KV_HEADS, max_pages * page_size).contiguous()


def storage_bits(t: torch.Tensor):
    """Host numpy view of a tensor's stored bits (uint16 for 16-bit, uint8 for bytes)."""
    t = t.detach().to("cpu").contiguous()
    if t.dtype in (torch.float16, torch.bfloat16):
        return t.view(torch.int16).numpy().view("uint16")
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return t.view(torch.uint8).numpy()
    if t.dtype == torch.int8:
        return t.numpy()
    raise TypeError(f"unsupported storage dtype {t.dtype}")
