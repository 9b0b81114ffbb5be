"""Seeded synthetic workloads for single-token GQA decode.

This module is shared by the tests, the smoke entry and the benchmark. It
holds no arithmetic of the decode method itself: it only draws the inputs
(lengths, query, cache) and encodes them into the stored formats, so both the
HIP path and the CPU oracle can consume identical bytes.

Workloads follow the shapes the pages describe: 32 query heads sharing 8 KV
heads at head_dim 128, a ``[batch, 2, 8, capacity, 128]`` cache, per-request
int32 lengths (FlashInfer sm110_gqa_decode article, "input contract"), and an
fp8_e4m3 cache that stores ``x / scale`` as ``float8_e4m3fn`` bytes with
per-tensor scales (Thor FP8 KV notes, section 1, patches 1 and 2).

Recipe: ``torch.Generator`` on the target device seeded with ``seed``; draw
order is lengths (``randint(lo, hi + 1)``), then q (fp32 N(0,1), cast RNE),
then the cache one request at a time (fp32 N(0,1) over both planes, cast RNE;
for fp8 divided by the plane's scale, clamped to +-448, cast to e4m3fn).
Slots past a request's length receive the same N(0,1) draw: garbage the
kernel must never read.
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
    kv_dtype: str           # "f16" | "bf16" | "fp8_e4m3"
    q_scale: float = 1.0
    k_scale: float = 1.0
    v_scale: float = 1.0
    seed: int = 0

    def describe(self) -> dict:
        return {
            "workload": self.name, "batch": self.batch, "capacity": self.capacity,
            "seq_len": [self.len_lo, self.len_hi], "q_heads": NUM_Q_HEADS,
            "kv_heads": NUM_KV_HEADS, "head_dim": HEAD_DIM, "q_dtype": self.q_dtype,
            "kv_dtype": self.kv_dtype, "q_scale": self.q_scale,
            "k_scale": self.k_scale, "v_scale": self.v_scale, "seed": self.seed,
        }


# The five workloads, in order. Seeds are 1000 + (1-based position).
WORKLOADS = [
    Workload("gqa_decode_b1_c64_f16", 1, 64, 64, 64, "f16", "f16", seed=1001),
    Workload("gqa_decode_b1_c1024_f16", 1, 1024, 1024, 1024, "f16", "f16", seed=1002),
    Workload("gqa_decode_b32_c8192_f16_ragged", 32, 8192, 1, 8192, "f16", "f16", seed=1003),
    Workload("gqa_decode_b8_c65536_bf16_long", 8, 65536, 32768, 65536, "bf16", "bf16",
             q_scale=0.5, seed=1004),
    Workload("gqa_decode_b16_c131072_fp8kv_long", 16, 131072, 65536, 131072, "bf16",
             "fp8_e4m3", k_scale=1.0 / 64, v_scale=1.0 / 64, seed=1005),
]
WORKLOADS_BY_NAME = {w.name: w for w in WORKLOADS}


def kv_elem_bytes(kv_dtype: str) -> int:
    return 1 if kv_dtype == "fp8_e4m3" else 2


def _encode_fp8(x: torch.Tensor, scale: float) -> torch.Tensor:
    y = (x / scale).clamp_(-E4M3_MAX, E4M3_MAX)
    return y.to(torch.float8_e4m3fn).view(torch.uint8)


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
    q32 = torch.randn(B, NUM_Q_HEADS, HEAD_DIM, generator=gen, device=dev, dtype=torch.float32)
    q = q32.to(_TORCH_DTYPES[w.q_dtype])
    del q32
    if w.kv_dtype == "fp8_e4m3":
        kv = torch.empty(B, 2, NUM_KV_HEADS, C, HEAD_DIM, device=dev, dtype=torch.uint8)
    else:
        kv = torch.empty(B, 2, NUM_KV_HEADS, C, HEAD_DIM, device=dev,
                         dtype=_TORCH_DTYPES[w.kv_dtype])
    for b in range(B):
        x = torch.randn(2, NUM_KV_HEADS, C, HEAD_DIM, generator=gen, device=dev,
                        dtype=torch.float32)
        if w.kv_dtype == "fp8_e4m3":
            kv[b, 0] = _encode_fp8(x[0], w.k_scale)
            kv[b, 1] = _encode_fp8(x[1], w.v_scale)
        else:
            kv[b] = x.to(kv.dtype)
        del x
    return {"q": q, "kv": kv, "seq_lens": lens, "q_scale": w.q_scale,
            "k_scale": w.k_scale, "v_scale": w.v_scale, "q_dtype": w.q_dtype,
            "kv_dtype": w.kv_dtype}


def storage_bits(t: torch.Tensor):
    """Host numpy view of a tensor's stored bits (uint16 for 16-bit, uint8 for bytes)."""
    t = t.detach().to("cpu").contiguous()
    if t.dtype in (torch.float16, torch.bfloat16):
        return t.view(torch.int16).numpy().view("uint16")
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return t.view(torch.uint8).numpy()
    raise TypeError(f"unsupported storage dtype {t.dtype}")
