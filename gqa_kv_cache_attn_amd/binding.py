"""ctypes binding of libgqa_decode.so (argument marshalling only).

Every function here forwards to the C entry point of the same name in
``include/gqa_decode.h``: it takes device pointers from the tensors, the
current (or given) HIP stream, and maps the returned status to an exception.
No step of the decode runs in Python. If the library is missing this module
raises at import: there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

from .build import LIB_PATH

library_path = LIB_PATH

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python -m gqa_kv_cache_attn_amd.build` "
        "(or __graft_entry__.build()) first")

_lib = ctypes.CDLL(LIB_PATH)

GQA_OK, GQA_ERR_INVALID_ARG, GQA_ERR_ALIAS, GQA_ERR_UNSUPPORTED_DEVICE = 0, 1, 2, 3
GQA_ERR_CAPTURE, GQA_ERR_OUT_OF_MEMORY, GQA_ERR_HIP = 4, 5, 6
GQA_F16, GQA_BF16, GQA_FP8_E4M3, GQA_INT8_ROWSCALE = 0, 1, 2, 3
GQA_FLAG_FUSED_COMBINE = 1
GQA_PAGED_SCALES_BY_POSITION = 2
NUM_Q_HEADS, NUM_KV_HEADS, HEAD_DIM = 32, 8, 128
NUM_Q_HEADS_2TO1 = 16

STATUS_NAMES = {
    0: "GQA_OK", 1: "GQA_ERR_INVALID_ARG", 2: "GQA_ERR_ALIAS",
    3: "GQA_ERR_UNSUPPORTED_DEVICE", 4: "GQA_ERR_CAPTURE",
    5: "GQA_ERR_OUT_OF_MEMORY", 6: "GQA_ERR_HIP",
}


class GqaDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("capacity", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("q_dtype", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32), ("k_scale", ctypes.c_float),
        ("v_scale", ctypes.c_float), ("flags", ctypes.c_int32),
    ]


class GqaPagedDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("q_tokens", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("q_dtype", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32), ("k_scale", ctypes.c_float),
        ("v_scale", ctypes.c_float), ("flags", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32),
        ("max_pages", ctypes.c_int32),
    ]


class GqaPlan(ctypes.Structure):
    _fields_ = [
        ("route", ctypes.c_int32), ("num_splits", ctypes.c_int32),
        ("chunk_tokens", ctypes.c_int32), ("num_workgroups", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_uint64), ("fused_merge", ctypes.c_int32),
    ]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


_vp, _i32, _f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
_DescP, _PlanP = ctypes.POINTER(GqaDesc), ctypes.POINTER(GqaPlan)
_PDescP = ctypes.POINTER(GqaPagedDesc)


def _sig(name, restype, argtypes):
    fn = getattr(_lib, name)
    fn.restype, fn.argtypes = restype, argtypes
    return fn


_gqa_decode = _sig("gqa_decode", ctypes.c_int, [_DescP, _vp, _vp, _vp, _f32, _vp, _vp])
_prepare = _sig("prepare_gqa_decode", ctypes.c_int,
                [_DescP, _vp, _vp, _vp, _f32, _vp, _i32, ctypes.POINTER(_vp)])
_launch = _sig("launch_gqa_decode_prepared", ctypes.c_int, [_vp, _vp])
_launch_timed = _sig("launch_gqa_decode_prepared_timed", ctypes.c_int, [_vp, _vp, _vp, _vp, _vp])
_destroy = _sig("gqa_prepared_destroy", None, [_vp])
_ws_bytes = _sig("gqa_prepared_workspace_bytes", ctypes.c_size_t, [_vp])
_prep_plan = _sig("gqa_prepared_plan", ctypes.c_int, [_vp, _PlanP])
_validate = _sig("gqa_validate_args", ctypes.c_int, [_DescP, _vp, _vp, _vp, _f32, _vp, _i32])
_gqa_decode_int8 = _sig("gqa_decode_int8", ctypes.c_int, [_DescP, _vp, _vp, _vp, _vp, _f32, _vp, _vp])
_prepare_int8 = _sig("prepare_gqa_decode_int8", ctypes.c_int,
                     [_DescP, _vp, _vp, _vp, _vp, _f32, _vp, _i32, ctypes.POINTER(_vp)])
_validate_int8 = _sig("gqa_validate_args_int8", ctypes.c_int,
                      [_DescP, _vp, _vp, _vp, _vp, _f32, _vp, _i32])
_plan = _sig("gqa_plan_decode", ctypes.c_int, [_DescP, _i32, _PlanP])
_decode_no_alloc = _sig("gqa_decode_no_alloc", ctypes.c_int,
                        [_DescP, _vp, _vp, _vp, _vp, _f32, _vp, _vp])
_decode_paged = _sig("gqa_decode_paged", ctypes.c_int,
                     [_PDescP, _vp, _vp, _vp, _vp, _vp, _f32, _vp, _vp])
_prepare_paged = _sig("prepare_gqa_decode_paged", ctypes.c_int,
                      [_PDescP, _vp, _vp, _vp, _vp, _vp, _f32, _vp, _i32, ctypes.POINTER(_vp)])
_validate_paged = _sig("gqa_validate_args_paged", ctypes.c_int,
                       [_PDescP, _vp, _vp, _vp, _vp, _vp, _f32, _vp, _i32])
_plan_paged = _sig("gqa_plan_decode_paged", ctypes.c_int, [_PDescP, _i32, _PlanP])
_last_error = _sig("gqa_last_error", ctypes.c_char_p, [])
_append = _sig("gqa_kv_append", ctypes.c_int, [_DescP, _vp, _vp, _vp, _vp, _vp])
_append_paged = _sig("gqa_kv_append_paged", ctypes.c_int, [_PDescP, _vp, _vp, _vp, _vp, _vp, _vp])
_append_int8 = _sig("gqa_kv_append_int8", ctypes.c_int, [_DescP, _vp, _vp, _vp, _vp, _vp, _vp])
_append_paged_int8 = _sig("gqa_kv_append_paged_int8", ctypes.c_int,
                          [_PDescP, _vp, _vp, _vp, _vp, _vp, _vp, _vp])


class GqaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def _check(status: int):
    if status != GQA_OK:
        msg = (_last_error() or b"").decode(errors="replace")
        if status in (GQA_ERR_INVALID_ARG, GQA_ERR_ALIAS):
            err = GqaError(status, msg)
            raise ValueError(str(err)) from err
        raise GqaError(status, msg)


def _dtype_code(t: torch.Tensor, role: str) -> int:
    if t.dtype == torch.float16:
        return GQA_F16
    if t.dtype == torch.bfloat16:
        return GQA_BF16
    if role == "kv" and t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return GQA_FP8_E4M3
    if role == "kv" and t.dtype == torch.int8:
        return GQA_INT8_ROWSCALE
    raise ValueError(f"unsupported {role} dtype {t.dtype}")


def make_desc(q: torch.Tensor, kv: torch.Tensor, k_scale: float = 1.0,
              v_scale: float = 1.0, fused_combine: bool = False) -> GqaDesc:
    if q.dim() != 3 or kv.dim() != 5:
        raise ValueError("q must be [batch, Hq, 128] and kv [batch, 2, 8, capacity, 128]")
    if q.shape[1] not in (NUM_Q_HEADS, NUM_Q_HEADS_2TO1) or q.shape[2] != HEAD_DIM:
        raise ValueError(f"q must be [batch, 32 or 16, 128], got {tuple(q.shape)}")
    if kv.shape[1] != 2 or kv.shape[0] != q.shape[0]:
        raise ValueError(f"kv must be [batch, 2, 8, capacity, 128], got {tuple(kv.shape)}")
    return GqaDesc(batch=q.shape[0], capacity=kv.shape[3], num_q_heads=q.shape[1],
                   num_kv_heads=kv.shape[2], head_dim=kv.shape[4],
                   q_dtype=_dtype_code(q, "q"), kv_dtype=_dtype_code(kv, "kv"),
                   k_scale=k_scale, v_scale=v_scale,
                   flags=GQA_FLAG_FUSED_COMBINE if fused_combine else 0)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


# torch's current-stream lookup that returns the raw handle without building
# a Stream object (about a microsecond less per launch); the public call is
# the fallback where the installed torch lacks it.
_raw_current_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream_handle(stream, device) -> int:
    if stream is None:
        if _raw_current_stream is not None:
            return _raw_current_stream(device.index)
        stream = torch.cuda.current_stream(device)
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check_devices(*ts):
    devs = {t.device for t in ts}
    if len(devs) != 1 or next(iter(devs)).type != "cuda":
        raise ValueError("q, kv, seq_lens and out must be on the same GPU")


def _check_per_request(t: torch.Tensor, batch: int, name: str):
    """seq_lens / positions: int32 [batch], contiguous. The kernels read one
    entry per request, so a shorter tensor would be read past its end."""
    if t.dtype != torch.int32:
        raise ValueError(f"{name} must be int32")
    if t.dim() != 1 or t.shape[0] != batch:
        raise ValueError(f"{name} must be [batch] = [{batch}], got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def gqa_decode(q: torch.Tensor, kv: torch.Tensor, seq_lens: torch.Tensor,
               q_scale: float = 1.0, out: Optional[torch.Tensor] = None,
               k_scale: float = 1.0, v_scale: float = 1.0, stream=None) -> torch.Tensor:
    """Enqueue one decode step on the current stream; returns ``out``."""
    if out is None:
        out = torch.empty_like(q)
    _check_per_request(seq_lens, q.shape[0] if q.dim() > 0 else -1, "seq_lens")
    if out.dtype != q.dtype or out.shape != q.shape:
        raise ValueError("out must match q's shape and dtype")
    _check_devices(q, kv, seq_lens, out)
    desc = make_desc(q, kv, k_scale, v_scale)
    with torch.cuda.device(q.device):
        st = _gqa_decode(ctypes.byref(desc), _ptr(q), _ptr(kv), _ptr(seq_lens), q_scale,
                         _ptr(out), _stream_handle(stream, q.device))
    _check(st)
    return out


def _check_scales(kv: torch.Tensor, kv_scales: torch.Tensor):
    if kv.dtype != torch.int8:
        raise ValueError("the _int8 entry points take an int8 kv")
    if kv_scales.dtype != torch.bfloat16 or tuple(kv_scales.shape) != tuple(kv.shape[:4]):
        raise ValueError(f"kv_scales must be bf16 [batch, 2, 8, capacity] = {tuple(kv.shape[:4])}, "
                         f"got {kv_scales.dtype} {tuple(kv_scales.shape)}")


def gqa_decode_int8(q: torch.Tensor, kv: torch.Tensor, kv_scales: torch.Tensor,
                    seq_lens: torch.Tensor, q_scale: float = 1.0,
                    out: Optional[torch.Tensor] = None, k_scale: float = 1.0,
                    v_scale: float = 1.0, stream=None) -> torch.Tensor:
    """gqa_decode over an int8 cache with bf16 row scales [batch, 2, 8, capacity]."""
    if out is None:
        out = torch.empty_like(q)
    _check_scales(kv, kv_scales)
    _check_per_request(seq_lens, q.shape[0] if q.dim() > 0 else -1, "seq_lens")
    if out.dtype != q.dtype or out.shape != q.shape:
        raise ValueError("out must match q's shape and dtype")
    _check_devices(q, kv, kv_scales, seq_lens, out)
    desc = make_desc(q, kv, k_scale, v_scale)
    with torch.cuda.device(q.device):
        st = _gqa_decode_int8(ctypes.byref(desc), _ptr(q), _ptr(kv), _ptr(kv_scales),
                              _ptr(seq_lens), q_scale, _ptr(out), _stream_handle(stream, q.device))
    _check(st)
    return out


# Bytes of the static device scratch gqa_decode_no_alloc uses as its workspace.
NO_ALLOC_SCRATCH_BYTES = 4 << 20


def gqa_decode_no_alloc(q: torch.Tensor, kv: torch.Tensor, seq_lens: torch.Tensor,
                        q_scale: float, out: torch.Tensor, k_scale: float = 1.0,
                        v_scale: float = 1.0, kv_scales: Optional[torch.Tensor] = None,
                        stream=None) -> torch.Tensor:
    """gqa_decode (or, with kv_scales, gqa_decode_int8) with the library's static
    scratch as the split workspace: nothing is allocated, here or in the library,
    so ``out`` is required. Calls that overlap on one GPU race on the scratch."""
    _check_per_request(seq_lens, q.shape[0] if q.dim() > 0 else -1, "seq_lens")
    if out.dtype != q.dtype or out.shape != q.shape:
        raise ValueError("out must match q's shape and dtype")
    if kv_scales is not None:
        _check_scales(kv, kv_scales)
    desc = make_desc(q, kv, k_scale, v_scale)
    _check_devices(*([q, kv, seq_lens, out] + ([kv_scales] if kv_scales is not None else [])))
    with torch.cuda.device(q.device):
        st = _decode_no_alloc(ctypes.byref(desc), _ptr(q), _ptr(kv), _ptr(kv_scales),
                              _ptr(seq_lens), q_scale, _ptr(out), _stream_handle(stream, q.device))
    _check(st)
    return out


class GqaPrepared:
    """Owner of a prepared handle and of references to its tensors."""

    def __init__(self, handle: int, tensors: dict, desc: GqaDesc):
        self._handle = handle
        self.tensors = tensors   # keeps q/kv/seq_lens/out alive as long as the handle
        self.desc = desc
        self.device = tensors["O"].device

    @property
    def handle(self) -> int:
        if not self._handle:
            raise ValueError("prepared handle already destroyed")
        return self._handle

    @property
    def out(self) -> torch.Tensor:
        return self.tensors["O"]

    @property
    def workspace_bytes(self) -> int:
        return int(_ws_bytes(self.handle))

    @property
    def plan(self) -> dict:
        p = GqaPlan()
        _check(_prep_plan(self.handle, ctypes.byref(p)))
        return p.as_dict()

    def destroy(self):
        if self._handle:
            _destroy(self._handle)
            self._handle = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def prepare_gqa_decode(q: torch.Tensor, kv: torch.Tensor, seq_lens: torch.Tensor,
                       out: torch.Tensor, q_scale: float = 1.0,
                       num_splits: Optional[int] = None, k_scale: float = 1.0,
                       v_scale: float = 1.0, fused_combine: bool = False) -> GqaPrepared:
    """Validate, plan and allocate the split workspace once (outside capture)."""
    _check_per_request(seq_lens, q.shape[0] if q.dim() > 0 else -1, "seq_lens")
    if out.dtype != q.dtype or out.shape != q.shape:
        raise ValueError("out must match q's shape and dtype")
    _check_devices(q, kv, seq_lens, out)
    desc = make_desc(q, kv, k_scale, v_scale, fused_combine)
    h = _vp()
    with torch.cuda.device(q.device):
        st = _prepare(ctypes.byref(desc), _ptr(q), _ptr(kv), _ptr(seq_lens), q_scale, _ptr(out),
                      0 if num_splits is None else int(num_splits), ctypes.byref(h))
    _check(st)
    return GqaPrepared(h.value, {"Q": q, "KV": kv, "sequence_lengths": seq_lens, "O": out}, desc)


def prepare_gqa_decode_int8(q: torch.Tensor, kv: torch.Tensor, kv_scales: torch.Tensor,
                            seq_lens: torch.Tensor, out: torch.Tensor, q_scale: float = 1.0,
                            num_splits: Optional[int] = None, k_scale: float = 1.0,
                            v_scale: float = 1.0, fused_combine: bool = False) -> GqaPrepared:
    """prepare_gqa_decode over an int8 cache with bf16 row scales."""
    _check_scales(kv, kv_scales)
    _check_per_request(seq_lens, q.shape[0] if q.dim() > 0 else -1, "seq_lens")
    if out.dtype != q.dtype or out.shape != q.shape:
        raise ValueError("out must match q's shape and dtype")
    _check_devices(q, kv, kv_scales, seq_lens, out)
    desc = make_desc(q, kv, k_scale, v_scale, fused_combine)
    h = _vp()
    with torch.cuda.device(q.device):
        st = _prepare_int8(ctypes.byref(desc), _ptr(q), _ptr(kv), _ptr(kv_scales), _ptr(seq_lens),
                           q_scale, _ptr(out), 0 if num_splits is None else int(num_splits),
                           ctypes.byref(h))
    _check(st)
    return GqaPrepared(h.value, {"Q": q, "KV": kv, "KV_scales": kv_scales,
                                 "sequence_lengths": seq_lens, "O": out}, desc)


def make_paged_desc(q: torch.Tensor, kv_pages: torch.Tensor, block_table: torch.Tensor,
                    k_scale: float = 1.0, v_scale: float = 1.0,
                    scales_by_position: bool = False) -> GqaPagedDesc:
    """q [batch, T, Hq, 128]; kv_pages [num_pages, 2, 8, page_size, 128];
    block_table [batch, max_pages] int32. scales_by_position: an int8 pool's
    row scales are [batch, 2, 8, max_pages * page_size]."""
    if q.dim() != 4 or kv_pages.dim() != 5 or block_table.dim() != 2:
        raise ValueError("q must be [batch, T, Hq, 128], kv_pages [num_pages, 2, 8, page_size, 128] "
                         "and block_table [batch, max_pages]")
    if kv_pages.shape[1] != 2 or block_table.shape[0] != q.shape[0]:
        raise ValueError(f"bad shapes: q {tuple(q.shape)}, kv_pages {tuple(kv_pages.shape)}, "
                         f"block_table {tuple(block_table.shape)}")
    return GqaPagedDesc(batch=q.shape[0], q_tokens=q.shape[1], num_q_heads=q.shape[2],
                        num_kv_heads=kv_pages.shape[2], head_dim=q.shape[3],
                        q_dtype=_dtype_code(q, "q"), kv_dtype=_dtype_code(kv_pages, "kv"),
                        k_scale=k_scale, v_scale=v_scale,
                        flags=GQA_PAGED_SCALES_BY_POSITION if scales_by_position else 0,
                        page_size=kv_pages.shape[3], num_pages=kv_pages.shape[0],
                        max_pages=block_table.shape[1])


def _paged_scale_shape(kv_pages, block_table, scales_by_position):
    """Shape of an int8 pool's row scales in the chosen layout."""
    if scales_by_position:
        return (block_table.shape[0], 2, NUM_KV_HEADS, block_table.shape[1] * kv_pages.shape[3])
    return tuple(kv_pages.shape[:4])


def _check_paged(q, kv_pages, kv_scales, block_table, seq_lens, out, scales_by_position=False):
    if block_table.dtype != torch.int32:
        raise ValueError("block_table must be int32")
    _check_per_request(seq_lens, q.shape[0] if q.dim() > 0 else -1, "seq_lens")
    if out.dtype != q.dtype or out.shape != q.shape:
        raise ValueError("out must match q's shape and dtype")
    # The pool's rows must be as wide as q's (the kernels step rows at q's
    # head_dim) and hold 8 KV heads; the C side sees only a pointer.
    if q.dim() != 4 or kv_pages.dim() != 5 or kv_pages.shape[1] != 2 or \
            kv_pages.shape[2] != NUM_KV_HEADS or kv_pages.shape[4] != HEAD_DIM or \
            q.shape[3] != HEAD_DIM:
        raise ValueError(f"q must be [batch, T, Hq, {HEAD_DIM}] and kv_pages "
                         f"[num_pages, 2, {NUM_KV_HEADS}, page_size, {HEAD_DIM}], got q "
                         f"{tuple(q.shape)} and kv_pages {tuple(kv_pages.shape)}")
    if (kv_scales is None) != (kv_pages.dtype != torch.int8):
        raise ValueError("kv_scales is required for (and only for) an int8 page pool")
    if scales_by_position and kv_scales is None:
        raise ValueError("scales_by_position needs an int8 page pool and its kv_scales")
    want = _paged_scale_shape(kv_pages, block_table, scales_by_position)
    if kv_scales is not None and (kv_scales.dtype != torch.bfloat16 or
                                  tuple(kv_scales.shape) != want):
        raise ValueError(f"kv_scales must be bf16 {want}")
    ts = [q, kv_pages, block_table, seq_lens, out] + ([kv_scales] if kv_scales is not None else [])
    _check_devices(*ts)


def gqa_decode_paged(q: torch.Tensor, kv_pages: torch.Tensor, block_table: torch.Tensor,
                     seq_lens: torch.Tensor, q_scale: float = 1.0,
                     out: Optional[torch.Tensor] = None, k_scale: float = 1.0,
                     v_scale: float = 1.0, kv_scales: Optional[torch.Tensor] = None,
                     stream=None, scales_by_position: bool = False) -> torch.Tensor:
    """Decode (T query tokens per request, causal among themselves) over a page pool."""
    if out is None:
        out = torch.empty_like(q)
    _check_paged(q, kv_pages, kv_scales, block_table, seq_lens, out, scales_by_position)
    desc = make_paged_desc(q, kv_pages, block_table, k_scale, v_scale, scales_by_position)
    with torch.cuda.device(q.device):
        st = _decode_paged(ctypes.byref(desc), _ptr(q), _ptr(kv_pages), _ptr(kv_scales),
                           _ptr(block_table), _ptr(seq_lens), q_scale, _ptr(out),
                           _stream_handle(stream, q.device))
    _check(st)
    return out


def prepare_gqa_decode_paged(q: torch.Tensor, kv_pages: torch.Tensor, block_table: torch.Tensor,
                             seq_lens: torch.Tensor, out: torch.Tensor, q_scale: float = 1.0,
                             num_splits: Optional[int] = None, k_scale: float = 1.0,
                             v_scale: float = 1.0,
                             kv_scales: Optional[torch.Tensor] = None,
                             scales_by_position: bool = False) -> GqaPrepared:
    """Prepare a paged decode step (workspace allocated once, outside capture)."""
    _check_paged(q, kv_pages, kv_scales, block_table, seq_lens, out, scales_by_position)
    desc = make_paged_desc(q, kv_pages, block_table, k_scale, v_scale, scales_by_position)
    h = _vp()
    with torch.cuda.device(q.device):
        st = _prepare_paged(ctypes.byref(desc), _ptr(q), _ptr(kv_pages), _ptr(kv_scales),
                            _ptr(block_table), _ptr(seq_lens), q_scale, _ptr(out),
                            0 if num_splits is None else int(num_splits), ctypes.byref(h))
    _check(st)
    tensors = {"Q": q, "KV_pages": kv_pages, "block_table": block_table,
               "sequence_lengths": seq_lens, "O": out}
    if kv_scales is not None:
        tensors["KV_scales"] = kv_scales
    return GqaPrepared(h.value, tensors, desc)


def launch_gqa_decode_prepared(prepared: GqaPrepared, stream=None) -> torch.Tensor:
    """Enqueue the prepared step (no allocation, no host sync); returns O."""
    _check(_launch(prepared.handle, _stream_handle(stream, prepared.device)))
    return prepared.out


def launch_gqa_decode_prepared_timed(prepared: GqaPrepared, ev_start, ev_mid, ev_end,
                                     stream=None) -> torch.Tensor:
    """As launch_gqa_decode_prepared, recording three torch.cuda.Events (already
    created, i.e. recorded once) around the attention kernel and the combine."""
    dev = prepared.out.device
    hs = [None if e is None else e.cuda_event for e in (ev_start, ev_mid, ev_end)]
    _check(_launch_timed(prepared.handle, _stream_handle(stream, dev), *hs))
    return prepared.out


def gqa_kv_append(kv: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                  positions: torch.Tensor, k_scale: float = 1.0, v_scale: float = 1.0,
                  stream=None) -> torch.Tensor:
    """Write k_new/v_new [batch, 8, 128] at slot positions[b] of every KV head; returns kv."""
    _check_per_request(positions, k_new.shape[0] if k_new.dim() > 0 else -1, "positions")
    if k_new.shape != v_new.shape or k_new.dtype != v_new.dtype:
        raise ValueError("k_new and v_new must have the same shape and dtype")
    if k_new.dim() != 3 or kv.dim() != 5 or k_new.shape[0] != kv.shape[0]:
        raise ValueError("k_new/v_new must be [batch, 8, 128] and kv [batch, 2, 8, capacity, 128]")
    _check_devices(kv, k_new, v_new, positions)
    desc = GqaDesc(batch=kv.shape[0], capacity=kv.shape[3], num_q_heads=NUM_Q_HEADS,
                   num_kv_heads=k_new.shape[1], head_dim=k_new.shape[2],
                   q_dtype=_dtype_code(k_new, "q"), kv_dtype=_dtype_code(kv, "kv"),
                   k_scale=k_scale, v_scale=v_scale, flags=0)
    if kv.shape[2] != k_new.shape[1] or kv.shape[4] != k_new.shape[2]:
        raise ValueError("kv and k_new disagree on KV heads or head_dim")
    with torch.cuda.device(kv.device):
        st = _append(ctypes.byref(desc), _ptr(k_new), _ptr(v_new), _ptr(positions), _ptr(kv),
                     _stream_handle(stream, kv.device))
    _check(st)
    return kv


def gqa_kv_append_paged(kv_pages: torch.Tensor, block_table: torch.Tensor, k_new: torch.Tensor,
                        v_new: torch.Tensor, positions: torch.Tensor, k_scale: float = 1.0,
                        v_scale: float = 1.0, num_q_heads: int = NUM_Q_HEADS,
                        stream=None) -> torch.Tensor:
    """Write k_new/v_new [batch, T, 8, 128] at slots positions[b] + t of a page pool
    kv_pages [num_pages, 2, 8, page_size, 128] through block_table [batch, max_pages];
    returns kv_pages. num_q_heads is the query-head count of the decode that
    shares the descriptor (T x query heads per KV head must fit its 16 rows)."""
    if block_table.dtype != torch.int32:
        raise ValueError("block_table must be int32")
    _check_per_request(positions, k_new.shape[0] if k_new.dim() > 0 else -1, "positions")
    if k_new.shape != v_new.shape or k_new.dtype != v_new.dtype:
        raise ValueError("k_new and v_new must have the same shape and dtype")
    if k_new.dim() != 4 or kv_pages.dim() != 5 or block_table.dim() != 2 or \
            block_table.shape[0] != k_new.shape[0] or kv_pages.shape[1] != 2:
        raise ValueError("k_new/v_new must be [batch, T, 8, 128], kv_pages "
                         "[num_pages, 2, 8, page_size, 128] and block_table [batch, max_pages]")
    if kv_pages.shape[2] != k_new.shape[2] or kv_pages.shape[4] != k_new.shape[3]:
        raise ValueError("kv_pages and k_new disagree on KV heads or head_dim")
    _check_devices(kv_pages, block_table, k_new, v_new, positions)
    desc = GqaPagedDesc(batch=k_new.shape[0], q_tokens=k_new.shape[1], num_q_heads=num_q_heads,
                        num_kv_heads=k_new.shape[2], head_dim=k_new.shape[3],
                        q_dtype=_dtype_code(k_new, "q"), kv_dtype=_dtype_code(kv_pages, "kv"),
                        k_scale=k_scale, v_scale=v_scale, flags=0, page_size=kv_pages.shape[3],
                        num_pages=kv_pages.shape[0], max_pages=block_table.shape[1])
    with torch.cuda.device(kv_pages.device):
        st = _append_paged(ctypes.byref(desc), _ptr(k_new), _ptr(v_new), _ptr(positions),
                           _ptr(block_table), _ptr(kv_pages), _stream_handle(stream, kv_pages.device))
    _check(st)
    return kv_pages


def gqa_kv_append_int8(kv: torch.Tensor, kv_scales: torch.Tensor, k_new: torch.Tensor,
                       v_new: torch.Tensor, positions: torch.Tensor, k_scale: float = 1.0,
                       v_scale: float = 1.0, num_q_heads: int = NUM_Q_HEADS_2TO1,
                       stream=None) -> torch.Tensor:
    """Quantise k_new/v_new [batch, 8, 128] row by row into an int8 cache kv
    [batch, 2, 8, capacity, 128] and its bf16 row scales kv_scales
    [batch, 2, 8, capacity] at slot positions[b]; returns kv."""
    _check_per_request(positions, k_new.shape[0] if k_new.dim() > 0 else -1, "positions")
    if kv.dtype != torch.int8 or kv_scales.dtype != torch.bfloat16:
        raise ValueError("kv must be int8 and kv_scales bfloat16")
    if k_new.shape != v_new.shape or k_new.dtype != v_new.dtype:
        raise ValueError("k_new and v_new must have the same shape and dtype")
    if k_new.dim() != 3 or kv.dim() != 5 or k_new.shape[0] != kv.shape[0] or \
            tuple(kv_scales.shape) != tuple(kv.shape[:4]):
        raise ValueError("k_new/v_new must be [batch, 8, 128], kv [batch, 2, 8, capacity, 128] "
                         "and kv_scales [batch, 2, 8, capacity]")
    if kv.shape[2] != k_new.shape[1] or kv.shape[4] != k_new.shape[2]:
        raise ValueError("kv and k_new disagree on KV heads or head_dim")
    _check_devices(kv, kv_scales, k_new, v_new, positions)
    desc = GqaDesc(batch=kv.shape[0], capacity=kv.shape[3], num_q_heads=num_q_heads,
                   num_kv_heads=k_new.shape[1], head_dim=k_new.shape[2],
                   q_dtype=_dtype_code(k_new, "q"), kv_dtype=GQA_INT8_ROWSCALE,
                   k_scale=k_scale, v_scale=v_scale, flags=0)
    with torch.cuda.device(kv.device):
        st = _append_int8(ctypes.byref(desc), _ptr(k_new), _ptr(v_new), _ptr(positions), _ptr(kv),
                          _ptr(kv_scales), _stream_handle(stream, kv.device))
    _check(st)
    return kv


def gqa_kv_append_paged_int8(kv_pages: torch.Tensor, kv_scales: torch.Tensor,
                             block_table: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                             positions: torch.Tensor, k_scale: float = 1.0, v_scale: float = 1.0,
                             num_q_heads: int = NUM_Q_HEADS_2TO1, stream=None,
                             scales_by_position: bool = False) -> torch.Tensor:
    """Quantise k_new/v_new [batch, T, 8, 128] row by row into an int8 page pool
    kv_pages [num_pages, 2, 8, page_size, 128] and its bf16 row scales kv_scales
    [num_pages, 2, 8, page_size] (scales_by_position: [batch, 2, 8, max_pages *
    page_size]) at slots positions[b] + t through block_table; returns kv_pages."""
    if block_table.dtype != torch.int32:
        raise ValueError("block_table must be int32")
    _check_per_request(positions, k_new.shape[0] if k_new.dim() > 0 else -1, "positions")
    if kv_pages.dtype != torch.int8 or kv_scales.dtype != torch.bfloat16:
        raise ValueError("kv_pages must be int8 and kv_scales bfloat16")
    if k_new.shape != v_new.shape or k_new.dtype != v_new.dtype:
        raise ValueError("k_new and v_new must have the same shape and dtype")
    if k_new.dim() != 4 or kv_pages.dim() != 5 or block_table.dim() != 2 or \
            block_table.shape[0] != k_new.shape[0] or kv_pages.shape[1] != 2 or \
            tuple(kv_scales.shape) != _paged_scale_shape(kv_pages, block_table,
                                                         scales_by_position):
        raise ValueError("k_new/v_new must be [batch, T, 8, 128], kv_pages "
                         "[num_pages, 2, 8, page_size, 128], kv_scales [num_pages, 2, 8, page_size] "
                         "(by position: [batch, 2, 8, max_pages * page_size]) and block_table "
                         "[batch, max_pages]")
    if kv_pages.shape[2] != k_new.shape[2] or kv_pages.shape[4] != k_new.shape[3]:
        raise ValueError("kv_pages and k_new disagree on KV heads or head_dim")
    _check_devices(kv_pages, kv_scales, block_table, k_new, v_new, positions)
    desc = GqaPagedDesc(batch=k_new.shape[0], q_tokens=k_new.shape[1], num_q_heads=num_q_heads,
                        num_kv_heads=k_new.shape[2], head_dim=k_new.shape[3],
                        q_dtype=_dtype_code(k_new, "q"), kv_dtype=GQA_INT8_ROWSCALE,
                        k_scale=k_scale, v_scale=v_scale,
                        flags=GQA_PAGED_SCALES_BY_POSITION if scales_by_position else 0,
                        page_size=kv_pages.shape[3], num_pages=kv_pages.shape[0],
                        max_pages=block_table.shape[1])
    with torch.cuda.device(kv_pages.device):
        st = _append_paged_int8(ctypes.byref(desc), _ptr(k_new), _ptr(v_new), _ptr(positions),
                                _ptr(block_table), _ptr(kv_pages), _ptr(kv_scales),
                                _stream_handle(stream, kv_pages.device))
    _check(st)
    return kv_pages


def gqa_validate_args(desc: GqaDesc, q_ptr: Optional[int], kv_ptr: Optional[int],
                      lens_ptr: Optional[int], q_scale: float, out_ptr: Optional[int],
                      num_splits: int = 0) -> int:
    """Host-only validation (no device access); returns the raw status code."""
    return int(_validate(ctypes.byref(desc), q_ptr, kv_ptr, lens_ptr, q_scale, out_ptr,
                         num_splits))


def gqa_validate_args_int8(desc: GqaDesc, q_ptr: Optional[int], kv_ptr: Optional[int],
                           scales_ptr: Optional[int], lens_ptr: Optional[int], q_scale: float,
                           out_ptr: Optional[int], num_splits: int = 0) -> int:
    """Host-only validation of an int8-cache call; returns the raw status code."""
    return int(_validate_int8(ctypes.byref(desc), q_ptr, kv_ptr, scales_ptr, lens_ptr, q_scale,
                              out_ptr, num_splits))


def gqa_validate_args_paged(desc: GqaPagedDesc, q_ptr, pool_ptr, scales_ptr, table_ptr, lens_ptr,
                            q_scale: float, out_ptr, num_splits: int = 0) -> int:
    """Host-only validation of a paged call; returns the raw status code."""
    return int(_validate_paged(ctypes.byref(desc), q_ptr, pool_ptr, scales_ptr, table_ptr, lens_ptr,
                               q_scale, out_ptr, num_splits))


def gqa_plan_paged(desc: GqaPagedDesc, num_splits: int = 0) -> dict:
    """Host-only launch plan for a paged descriptor."""
    p = GqaPlan()
    _check(_plan_paged(ctypes.byref(desc), num_splits, ctypes.byref(p)))
    return p.as_dict()


def gqa_plan(desc: GqaDesc, num_splits: int = 0) -> dict:
    """Host-only launch plan for a descriptor."""
    p = GqaPlan()
    _check(_plan(ctypes.byref(desc), num_splits, ctypes.byref(p)))
    return p.as_dict()


def last_error() -> str:
    return (_last_error() or b"").decode(errors="replace")
