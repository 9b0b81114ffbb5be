"""CPU-only checks of the C ABI: the library loads, exports every declared
symbol, and its host-only validation and planning behave as documented.
No device is touched (validation never dereferences a pointer)."""

import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gqa_decode.h")

b = pytest.importorskip("gqa_kv_cache_attn_amd.binding")

OK, INVALID, ALIAS = b.GQA_OK, b.GQA_ERR_INVALID_ARG, b.GQA_ERR_ALIAS
MiB = 1 << 20


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"GQA_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)


def test_header_declares_the_three_page_entry_points():
    names = declared_functions()
    for n in ("gqa_decode", "prepare_gqa_decode", "launch_gqa_decode_prepared"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(b.library_path)
    names = declared_functions()
    # every declaration line was parsed (none slipped past the pattern)
    assert len(names) == sum(ln.startswith("GQA_API ") for ln in open(HEADER)) >= 18
    for n in names:
        assert hasattr(lib, n), n


def desc(batch=2, capacity=1024, q=b.GQA_BF16, kv=b.GQA_BF16, ks=1.0, vs=1.0, hq=32, hkv=8, d=128):
    return b.GqaDesc(batch=batch, capacity=capacity, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                     q_dtype=q, kv_dtype=kv, k_scale=ks, v_scale=vs)


# Fake, well-separated, aligned device addresses: validation only compares them.
Q, KV, LENS, OUT = 1 * 1024 * MiB, 2 * 1024 * MiB, 3 * 1024 * MiB, 4 * 1024 * MiB


def v(d, q=Q, kv=KV, lens=LENS, qs=1.0, out=OUT, ns=0):
    return b.gqa_validate_args(d, q, kv, lens, qs, out, ns)


def test_valid_arguments_pass():
    assert v(desc()) == OK
    assert v(desc(hq=16)) == OK                      # 2 query heads per KV head
    assert v(desc(hq=16, q=b.GQA_F16, kv=b.GQA_FP8_E4M3)) == OK
    assert v(desc(q=b.GQA_F16, kv=b.GQA_F16)) == OK
    assert v(desc(q=b.GQA_BF16, kv=b.GQA_FP8_E4M3, ks=1 / 64, vs=1 / 64)) == OK
    assert v(desc(q=b.GQA_F16, kv=b.GQA_FP8_E4M3)) == OK


@pytest.mark.parametrize("field,value", [("num_q_heads", 24), ("num_q_heads", 8), ("num_q_heads", 64),
                                         ("num_kv_heads", 4), ("head_dim", 64),
                                         ("capacity", 0), ("capacity", -3), ("batch", -1),
                                         ("capacity", (1 << 22) + 1)])
def test_fixed_geometry_and_sizes(field, value):
    d = desc()
    setattr(d, field, value)
    assert v(d) == INVALID
    assert b.last_error()


@pytest.mark.parametrize("q,kv", [(b.GQA_F16, b.GQA_BF16), (b.GQA_BF16, b.GQA_F16),
                                  (b.GQA_FP8_E4M3, b.GQA_FP8_E4M3), (7, b.GQA_BF16),
                                  (b.GQA_INT8_ROWSCALE, b.GQA_INT8_ROWSCALE),
                                  (b.GQA_BF16, 9)])
def test_unsupported_dtype_pairs(q, kv):
    assert v(desc(q=q, kv=kv)) == INVALID


@pytest.mark.parametrize("qs", [0.0, -1.0, math.nan, math.inf, -math.inf])
def test_q_scale_must_be_finite_positive(qs):
    assert v(desc(), qs=qs) == INVALID


@pytest.mark.parametrize("ks,vs", [(0.0, 1.0), (1.0, -2.0), (math.nan, 1.0), (1.0, math.inf)])
def test_fp8_scales_must_be_finite_positive(ks, vs):
    assert v(desc(kv=b.GQA_FP8_E4M3, ks=ks, vs=vs)) == INVALID


def test_scale_on_16bit_cache_is_rejected_not_ignored():
    assert v(desc(ks=0.5)) == INVALID
    assert v(desc(vs=2.0)) == INVALID


@pytest.mark.parametrize("which", ["q", "kv", "lens", "out"])
def test_null_pointers(which):
    args = dict(q=Q, kv=KV, lens=LENS, out=OUT)
    args[which] = None
    assert v(desc(), **args) == INVALID


@pytest.mark.parametrize("which,off", [("q", 8), ("kv", 4), ("out", 2), ("lens", 2)])
def test_misalignment(which, off):
    args = dict(q=Q, kv=KV, lens=LENS, out=OUT)
    args[which] += off
    assert v(desc(), **args) == INVALID


def test_out_aliasing_is_detected_by_address_range():
    d = desc(batch=2, capacity=1024)
    q_bytes = 2 * 32 * 128 * 2
    kv_bytes = 2 * 2 * 8 * 1024 * 128 * 2
    assert v(d, out=Q) == ALIAS
    assert v(d, out=Q + q_bytes - 16) == ALIAS          # tail overlap
    assert v(d, out=Q + q_bytes) == OK                  # adjacent is fine
    assert v(d, out=KV + kv_bytes // 2) == ALIAS        # inside the cache
    assert v(d, out=KV - q_bytes + 16) == ALIAS         # straddles the cache start
    assert v(d, out=LENS - 16) == ALIAS                 # covers the lengths
    assert v(d, q=KV, out=OUT) == OK                    # inputs may overlap each other


def test_batch_zero_is_a_valid_no_op():
    assert v(desc(batch=0), q=None, kv=None, lens=None, out=None) == OK


def test_plan_routes_on_capacity():
    for C in (1, 16, 63, 64):
        p = b.gqa_plan(desc(capacity=C))
        assert p["route"] == 0 and p["num_splits"] == 1 and p["workspace_bytes"] == 0
        assert p["chunk_tokens"] >= C
    for C in (65, 1024, 131072):
        big = C * 2 * 8 // 64 >= 768
        assert b.gqa_plan(desc(capacity=C))["route"] == (2 if big else 1)  # balanced when it fills
        assert b.gqa_plan(desc(capacity=C), 2)["route"] == 1   # explicit split count: chunked


def balanced_ws(B, G=768, rows_per_slot=4):
    # partials: 2 slots per workgroup x rows x (128 + 2) floats | slab prefix [B + 1]
    # and, per (request, KV head), its first-piece slot and last workgroup
    return 2 * G * rows_per_slot * 130 * 4 + ((4 * (B + 1 + 2 * 8 * B) + 255) // 256) * 256


def nominal_balanced_grid(B, C, slot_bytes=2 * 128 * 2):
    """Host-only plans: 256 CUs x 3 workgroups, or (16-bit and INT8 caches)
    one per CU for a single request or at most 256 MiB of K+V at capacity."""
    return 256 if B == 1 or B * 8 * C * slot_bytes <= 256 << 20 else 768


@pytest.mark.parametrize("C", [65, 100, 1000, 1024, 8192, 65536, 131072])
@pytest.mark.parametrize("B", [1, 8, 32, 4096])
def test_auto_plan_is_the_balanced_split(B, C):
    p = b.gqa_plan(desc(batch=B, capacity=C))
    if B * 8 * -(-C // 64) < 768:      # too small to fill the grid: chunked split
        assert p["route"] == 1
        return
    G = nominal_balanced_grid(B, C)
    assert p == {"route": 2, "num_splits": 0, "chunk_tokens": 64, "num_workgroups": G,
                 "workspace_bytes": balanced_ws(B, G), "fused_merge": 0}


def small_chunk(C):
    """Automatic chunk of a problem too small for the balanced split: about an
    eighth of the capacity in 64-slot steps, from 64 to 256 slots."""
    return min(256, max(64, -(-(-(-C // 8)) // 64) * 64))


@pytest.mark.parametrize("B,C", [(1, 65), (1, 128), (1, 500), (1, 1024), (1, 2048), (1, 4096),
                                 (1, 6000), (2, 1024), (4, 1024), (5, 1000), (11, 512),
                                 (40, 128), (47, 65)])
def test_small_automatic_plans_and_the_one_launch_merge(B, C):
    assert B * 8 * -(-C // 64) < 768
    p = b.gqa_plan(desc(batch=B, capacity=C))
    T = small_chunk(C)
    S = -(-C // T)
    one = 1 < S <= 16 and B * 8 * S <= 384
    ctrl = ((B * 8 * 4 + 255) // 256) * 256 if one else 0
    assert p == {"route": 1, "num_splits": S, "chunk_tokens": T, "num_workgroups": B * 8 * S,
                 "workspace_bytes": ctrl + B * 32 * S * 130 * 4 if S > 1 else 0,
                 "fused_merge": int(one)}
    # An explicit split count keeps the two-launch merge unless the flag asks.
    if S > 1:
        assert b.gqa_plan(desc(batch=B, capacity=C), S)["fused_merge"] == 0
    # The paged kernels take no one-launch merge.
    P = 16
    pp = b.gqa_plan_paged(b.GqaPagedDesc(batch=B, q_tokens=1, num_q_heads=32, num_kv_heads=8,
                                         head_dim=128, q_dtype=b.GQA_BF16, kv_dtype=b.GQA_BF16,
                                         k_scale=1.0, v_scale=1.0, flags=0, page_size=P,
                                         num_pages=B * (-(-C // P)), max_pages=-(-C // P)))
    assert pp["fused_merge"] == 0


@pytest.mark.parametrize("kv,slot", [(b.GQA_BF16, 512), (b.GQA_FP8_E4M3, 256),
                                     (b.GQA_INT8_ROWSCALE, 260)])
def test_small_problems_take_one_balanced_workgroup_per_cu(kv, slot):
    """16-bit and INT8 caches; fp8 keeps the resident grid."""
    hq = 16 if kv == b.GQA_INT8_ROWSCALE else 32
    ks = 1 / 64 if kv == b.GQA_FP8_E4M3 else 1.0
    for B, C in [(1, 131072), (1, 1 << 20), (2, 65536), (4, 32768), (16, 4096), (64, 4096),
                 (8, 65536)]:
        p = b.gqa_plan(desc(batch=B, capacity=C, kv=kv, hq=hq, ks=ks, vs=ks))
        assert p["route"] == 2
        small = kv != b.GQA_FP8_E4M3 and (B == 1 or B * 8 * C * slot <= 256 << 20)
        assert p["num_workgroups"] == (256 if small else 768), (B, C)


@pytest.mark.parametrize("C", [65, 1000, 8192, 65536, 131072])
@pytest.mark.parametrize("B", [1, 32, 4097])
def test_chunked_auto_plan_is_consistent(B, C):
    """Beyond 4096 requests, or with the fused merge, auto picks the chunked split."""
    d = desc(batch=B, capacity=C)
    if B <= 4096:
        d.flags = b.GQA_FLAG_FUSED_COMBINE
    p = b.gqa_plan(d)
    S, T = p["num_splits"], p["chunk_tokens"]
    assert p["route"] == 1
    assert T % 16 == 0 and T % 64 == 0
    assert S == -(-C // T)
    assert p["num_workgroups"] == B * 8 * S
    # control words (fused merge: one uint32 counter per (request, KV head)),
    # then FP32 partials (O, then max/sum)
    fused = B <= 4096
    ctrl = ((B * 8 * 4 + 255) // 256) * 256 if fused and S > 1 else 0
    want_ws = ctrl + B * 32 * S * 130 * 4 if S > 1 else 0
    assert p["workspace_bytes"] == want_ws
    assert p["fused_merge"] == int(fused and S > 1)


@pytest.mark.parametrize("C", [100, 1000, 1024, 65536])
def test_explicit_num_splits_is_honoured_exactly_or_rejected(C):
    for n in range(1, 80):
        d = desc(capacity=C)
        st = v(d, ns=n)
        if st == OK:
            p = b.gqa_plan(d, n)
            assert p["num_splits"] == n and p["chunk_tokens"] % 16 == 0
            assert -(-C // p["chunk_tokens"]) == n
        else:
            assert st == INVALID and "num_splits" in b.last_error()
    assert v(desc(capacity=1024), ns=10) == OK        # the article's batch-1 / capacity-1024 split
    assert v(desc(capacity=1024), ns=-1) == INVALID
    assert v(desc(capacity=1024), ns=1025) == INVALID


def test_unknown_flags_are_rejected():
    d = desc()
    d.flags = 2
    assert v(d) == INVALID
    d.flags = b.GQA_FLAG_FUSED_COMBINE
    assert v(d) == OK


def test_error_message_is_thread_local_and_cleared_on_success():
    assert v(desc(), qs=-1.0) == INVALID
    assert "q_scale" in b.last_error()
    assert v(desc()) == OK
    assert b.last_error() == ""


def test_kv_append_rejects_bad_arguments_without_touching_a_device():
    d = desc(batch=2, capacity=16)
    K, V, P, KV_ = (1 << 30), (5 << 30), (3 << 30), (2 << 30)
    app = b._append
    assert app(ctypes.byref(d), None, V, P, KV_, None) == INVALID
    assert app(ctypes.byref(d), K + 4, V, P, KV_, None) == INVALID      # misaligned
    assert app(ctypes.byref(d), KV_ + 4096, V, P, KV_, None) == ALIAS    # k_new inside the cache
    d0 = desc(batch=0)
    assert app(ctypes.byref(d0), None, None, None, None, None) == OK


# ---------------------------------------------------------------- INT8 row-scaled cache
SC = 5 * 1024 * MiB   # fake address of the row scales


def v8(d, q=Q, kv=KV, sc=SC, lens=LENS, qs=1.0, out=OUT, ns=0):
    return b.gqa_validate_args_int8(d, q, kv, sc, lens, qs, out, ns)


@pytest.mark.parametrize("qd", [b.GQA_BF16, b.GQA_F16])
@pytest.mark.parametrize("hq", [16, 32])
def test_int8_valid_arguments_pass(qd, hq):
    assert v8(desc(q=qd, kv=b.GQA_INT8_ROWSCALE, hq=hq)) == OK
    # per-tensor scales multiply on top of the row scales
    assert v8(desc(q=qd, kv=b.GQA_INT8_ROWSCALE, hq=hq, ks=0.5, vs=4.0)) == OK


def test_int8_cache_needs_the_int8_entry_points_and_vice_versa():
    assert v(desc(kv=b.GQA_INT8_ROWSCALE, hq=16)) == INVALID
    assert "int8" in b.last_error()
    assert v8(desc(kv=b.GQA_BF16, hq=16)) == INVALID
    assert v8(desc(kv=b.GQA_FP8_E4M3, hq=16)) == INVALID


def test_int8_scales_pointer_checks():
    d = desc(batch=2, capacity=1024, kv=b.GQA_INT8_ROWSCALE, hq=16)
    assert v8(d, sc=None) == INVALID
    assert v8(d, sc=SC + 2) == INVALID                # scales must be 16-byte aligned
    q_bytes = 2 * 16 * 128 * 2
    sc_bytes = 2 * 2 * 8 * 1024 * 2
    assert v8(d, out=SC + sc_bytes // 2) == ALIAS     # out inside the scales
    assert v8(d, out=SC - q_bytes + 16) == ALIAS
    assert v8(d, out=SC + sc_bytes) == OK
    assert v8(desc(batch=0, kv=b.GQA_INT8_ROWSCALE), q=None, kv=None, sc=None, lens=None,
              out=None) == OK


@pytest.mark.parametrize("hq", [16, 32])
@pytest.mark.parametrize("kv", [b.GQA_BF16, b.GQA_FP8_E4M3, b.GQA_INT8_ROWSCALE])
def test_chunked_workspace_scales_with_query_heads(hq, kv):
    d = desc(batch=3, capacity=5000, kv=kv, hq=hq)
    p = b.gqa_plan(d, 7)
    assert p["route"] == 1 and p["num_splits"] == 7
    assert p["workspace_bytes"] == 3 * hq * 7 * 130 * 4
    # the balanced split's partial slots do not depend on the geometry
    assert b.gqa_plan(desc(batch=8, capacity=65536, kv=kv, hq=hq))["workspace_bytes"] == balanced_ws(8)


def test_int8_chunk_sizing_counts_the_row_scales():
    """Automatic chunks hold about 1 MiB of cache: 64-slot steps of
    64 * 2 * (128 + 2) bytes for INT8 (the row scales included)."""
    d = desc(batch=4097, capacity=65536, kv=b.GQA_INT8_ROWSCALE, hq=16)
    p = b.gqa_plan(d)
    assert p["route"] == 1 and p["chunk_tokens"] == 64 * ((1 << 20) // (64 * 2 * 130))


# ---------------------------------------------------------------- paged cache
POOL, TABLE = 6 * 1024 * MiB, 7 * 1024 * MiB


def pdesc(batch=2, T=1, hq=32, q=b.GQA_BF16, kv=b.GQA_BF16, P=16, num_pages=100, max_pages=8,
          ks=1.0, vs=1.0, flags=0):
    return b.GqaPagedDesc(batch=batch, q_tokens=T, num_q_heads=hq, num_kv_heads=8, head_dim=128,
                          q_dtype=q, kv_dtype=kv, k_scale=ks, v_scale=vs, flags=flags, page_size=P,
                          num_pages=num_pages, max_pages=max_pages)


def vp(d, q=Q, pool=POOL, sc=None, table=TABLE, lens=LENS, qs=1.0, out=OUT, ns=0):
    return b.gqa_validate_args_paged(d, q, pool, sc, table, lens, qs, out, ns)


def test_paged_valid_arguments_pass():
    assert vp(pdesc()) == OK
    assert vp(pdesc(T=4)) == OK
    assert vp(pdesc(T=8, hq=16)) == OK
    assert vp(pdesc(kv=b.GQA_FP8_E4M3, ks=0.25, vs=0.5, P=64)) == OK
    assert vp(pdesc(kv=b.GQA_INT8_ROWSCALE, hq=16, T=3), sc=5 * 1024 * MiB) == OK


@pytest.mark.parametrize("P", [0, 8, 24, 48, 1000, (1 << 16) * 2])
def test_paged_page_size_must_be_a_power_of_two_from_16(P):
    assert vp(pdesc(P=P)) == INVALID
    assert "page_size" in b.last_error()


@pytest.mark.parametrize("hq,T", [(32, 5), (16, 9), (32, 0), (32, -1)])
def test_paged_query_tokens_must_fit_one_mfma_tile(hq, T):
    assert vp(pdesc(hq=hq, T=T)) == INVALID
    assert "q_tokens" in b.last_error()


def test_paged_other_descriptor_checks():
    assert vp(pdesc(num_pages=0)) == INVALID
    assert vp(pdesc(max_pages=0)) == INVALID
    assert vp(pdesc(P=1 << 16, max_pages=65)) == INVALID          # > GQA_MAX_CAPACITY slots
    assert vp(pdesc(flags=1)) == INVALID                            # no one-launch merge here
    assert vp(pdesc(flags=8)) == INVALID
    assert vp(pdesc(ks=0.5)) == INVALID                             # scale on a 16-bit pool
    assert vp(pdesc(kv=b.GQA_INT8_ROWSCALE, hq=16)) == INVALID      # int8 needs its scales
    assert vp(pdesc(), sc=5 * 1024 * MiB) == INVALID                # scales only for int8
    assert vp(pdesc(), table=None) == INVALID
    assert vp(pdesc(), table=TABLE + 2) == INVALID                  # 4-byte alignment
    assert vp(pdesc(), qs=0.0) == INVALID


def test_paged_scales_by_position_flag_is_int8_only_and_sizes_the_scales():
    """GQA_PAGED_SCALES_BY_POSITION: accepted only with an INT8 pool; the
    scales then span batch * 2 * 8 * max_pages * page_size bf16 values, and
    out may not overlap them."""
    POS = b.GQA_PAGED_SCALES_BY_POSITION
    SCALES = 5 * 1024 * MiB
    d = pdesc(batch=2, kv=b.GQA_INT8_ROWSCALE, hq=16, T=2, P=16, num_pages=100, max_pages=8,
              flags=POS)
    assert vp(d, sc=SCALES) == OK
    assert vp(pdesc(flags=POS)) == INVALID and "INT8" in b.last_error()        # bf16 pool
    assert vp(pdesc(kv=b.GQA_FP8_E4M3, ks=0.5, vs=0.5, flags=POS)) == INVALID
    assert vp(pdesc(kv=b.GQA_INT8_ROWSCALE, hq=16, flags=4), sc=SCALES) == INVALID
    assert vp(pdesc(kv=b.GQA_INT8_ROWSCALE, hq=16, flags=POS | 1), sc=SCALES) == INVALID
    by_pos = 2 * 2 * 8 * 8 * 16 * 2        # [batch, 2, 8, max_pages * page_size] bf16
    in_pool = 100 * 2 * 8 * 16 * 2         # [num_pages, 2, 8, page_size] bf16
    assert by_pos < in_pool
    assert vp(d, sc=SCALES, out=SCALES + by_pos - 16) == ALIAS
    assert vp(d, sc=SCALES, out=SCALES + by_pos) == OK
    d0 = pdesc(batch=2, kv=b.GQA_INT8_ROWSCALE, hq=16, T=2, P=16, num_pages=100, max_pages=8)
    assert vp(d0, sc=SCALES, out=SCALES + by_pos) == ALIAS       # the pool layout is larger
    assert vp(d0, sc=SCALES, out=SCALES + in_pool) == OK
    # the append takes the same flag and the same size
    app = b._append_paged_int8
    K, V, POSN = 1 << 30, 3 << 30, 4 << 30
    pool = POOL

    def call(desc_, sc=SCALES, pos=POSN):
        return app(ctypes.byref(desc_), K, V, pos, TABLE, pool, sc, None)

    assert call(d, pos=SCALES + by_pos - 4) == ALIAS
    assert call(d, pos=SCALES + by_pos) not in (INVALID, ALIAS)
    assert call(pdesc(flags=POS)) == INVALID


def test_paged_aliasing_by_address_range():
    d = pdesc(batch=2, T=3, num_pages=100, P=16, max_pages=8)
    q_bytes = 2 * 3 * 32 * 128 * 2
    pool_bytes = 100 * 2 * 8 * 16 * 128 * 2
    assert vp(d, out=Q) == ALIAS
    assert vp(d, out=POOL + pool_bytes - 16) == ALIAS
    assert vp(d, out=POOL + pool_bytes) == OK
    assert vp(d, out=TABLE - q_bytes + 16) == ALIAS                 # covers the block table
    assert vp(d, out=LENS) == ALIAS


def test_paged_plans_use_the_logical_capacity_and_query_rows():
    # capacity = max_pages * page_size = 512 * 16; chunked workspace rows = B * T * Hq * S
    d = pdesc(batch=3, T=2, P=16, max_pages=512)
    p = b.gqa_plan_paged(d, 7)
    assert p["route"] == 1 and p["num_splits"] == 7
    assert p["workspace_bytes"] == 3 * 2 * 32 * 7 * 130 * 4
    # balanced split: 16 partial rows per slot
    p = b.gqa_plan_paged(pdesc(batch=8, T=3, P=16, max_pages=4096))
    assert p["route"] == 2
    assert p["workspace_bytes"] == balanced_ws(8, rows_per_slot=16)
    # short route when the table addresses at most 64 slots
    p = b.gqa_plan_paged(pdesc(batch=3, P=32, max_pages=2))
    assert p["route"] == 0 and p["workspace_bytes"] == 0
    assert vp(pdesc(batch=0), q=None, pool=None, table=None, lens=None, out=None) == OK


def test_paged_append_rejects_bad_arguments_without_touching_a_device():
    d = pdesc(batch=2, T=3, P=16, num_pages=100, max_pages=8)
    K, V, POS = 1 << 30, 5 << 30, 3 << 30
    pool_bytes = 100 * 2 * 8 * 16 * 128 * 2
    app = b._append_paged

    def call(desc_, k=K, v_=V, pos=POS, table=TABLE, pool=POOL):
        return app(ctypes.byref(desc_), k, v_, pos, table, pool, None)

    assert call(d, k=None) == INVALID
    assert call(d, table=None) == INVALID
    assert call(d, k=K + 4) == INVALID                          # 16-byte alignment
    assert call(d, table=TABLE + 2) == INVALID                  # 4-byte alignment
    assert call(d, k=POOL + pool_bytes - 16) == ALIAS           # k_new inside the pool
    assert call(d, table=POOL + 64) == ALIAS                    # block table inside the pool
    # adjacent to the pool is fine: validation passes and only the device check is left
    assert call(d, pos=POOL + pool_bytes) not in (INVALID, ALIAS)
    assert call(pdesc(P=24)) == INVALID and "page_size" in b.last_error()
    assert call(pdesc(T=5)) == INVALID                           # 5 tokens x 4 heads > 16 rows
    assert call(pdesc(kv=b.GQA_INT8_ROWSCALE, hq=16)) == INVALID and "INT8" in b.last_error()
    assert call(pdesc(batch=0), None, None, None, None, None) == OK


def test_int8_append_rejects_bad_arguments_without_touching_a_device():
    """gqa_kv_append_int8 / gqa_kv_append_paged_int8: INT8 descriptors only, a
    2-byte aligned scales buffer that overlaps nothing; the plain forms refuse
    an INT8 cache and name the _int8 form."""
    K, V, P, KV_ = (1 << 30), (5 << 30), (3 << 30), (2 << 30)
    d = desc(batch=2, capacity=16, kv=b.GQA_INT8_ROWSCALE, hq=16)
    cache_bytes = 2 * 2 * 8 * 16 * 128
    scale_bytes = 2 * 2 * 8 * 16 * 2
    app = b._append_int8

    def call(desc_, k=K, v_=V, pos=P, kv=KV_, sc=SC):
        return app(ctypes.byref(desc_), k, v_, pos, kv, sc, None)

    assert call(d, sc=None) == INVALID
    assert call(d, sc=SC + 1) == INVALID                            # 2-byte alignment
    assert call(d, sc=KV_ + cache_bytes - 2) == ALIAS               # scales inside the cache
    assert call(d, k=SC + scale_bytes - 16) == ALIAS                # k_new inside the scales
    assert call(d, pos=SC) == ALIAS
    assert call(d, sc=KV_ + cache_bytes) not in (INVALID, ALIAS)    # adjacent: only the device check
    assert call(desc(batch=2, capacity=16)) == INVALID and "INT8" in b.last_error()
    assert b._append(ctypes.byref(d), K, V, P, KV_, None) == INVALID
    assert "gqa_kv_append_int8" in b.last_error()
    assert call(desc(batch=0, kv=b.GQA_INT8_ROWSCALE, hq=16), None, None, None, None, None) == OK

    pd = pdesc(batch=2, T=2, P=16, num_pages=100, max_pages=8, kv=b.GQA_INT8_ROWSCALE, hq=16)
    pool_bytes = 100 * 2 * 8 * 16 * 128
    pscale_bytes = 100 * 2 * 8 * 16 * 2
    papp = b._append_paged_int8

    def pcall(desc_, k=K, v_=V, pos=P, table=TABLE, pool=POOL, sc=SC):
        return papp(ctypes.byref(desc_), k, v_, pos, table, pool, sc, None)

    assert pcall(pd, sc=None) == INVALID
    assert pcall(pd, sc=SC + 1) == INVALID
    assert pcall(pd, sc=POOL + pool_bytes - 2) == ALIAS
    assert pcall(pd, table=SC + pscale_bytes - 4) == ALIAS          # block table inside the scales
    assert pcall(pd, sc=POOL + pool_bytes) not in (INVALID, ALIAS)
    assert pcall(pdesc(batch=2, T=2)) == INVALID and "INT8" in b.last_error()
    assert b._append_paged(ctypes.byref(pd), K, V, P, TABLE, POOL, None) == INVALID
    assert "gqa_kv_append_paged_int8" in b.last_error()


# ---------------------------------------------------------------- binding shape checks
# The binding checks what the C side cannot see (it gets pointers only):
# per-request tensors must have one entry per request, and a page pool's
# rows must be as wide as q's. These checks run before the device check,
# so CPU tensors reach them; correct shapes fail only at the device check.
import torch  # noqa: E402


def _contig(batch=2, C=64, lens=None, hq=32):
    q = torch.zeros(batch, hq, 128, dtype=torch.float16)
    kv = torch.zeros(batch, 2, 8, C, 128, dtype=torch.float16)
    lens = torch.ones(batch if lens is None else lens, dtype=torch.int32)
    return q, kv, lens, torch.empty_like(q)


def test_binding_rejects_seq_lens_that_do_not_match_the_batch():
    for n in (1, 3):
        q, kv, lens, out = _contig(lens=n)
        with pytest.raises(ValueError, match=r"seq_lens must be \[batch\]"):
            b.gqa_decode(q, kv, lens, 1.0, out)
        with pytest.raises(ValueError, match=r"seq_lens must be \[batch\]"):
            b.prepare_gqa_decode(q, kv, lens, out)
    q, kv, lens, out = _contig()
    with pytest.raises(ValueError, match=r"seq_lens must be \[batch\]"):
        b.gqa_decode(q, kv, lens.reshape(2, 1), 1.0, out)
    with pytest.raises(ValueError, match="int32"):
        b.gqa_decode(q, kv, lens.long(), 1.0, out)
    # right shapes: only the device check is left
    with pytest.raises(ValueError, match="same GPU"):
        b.gqa_decode(q, kv, lens, 1.0, out)
    q8 = torch.zeros(2, 16, 128, dtype=torch.bfloat16)
    kv8 = torch.zeros(2, 2, 8, 64, 128, dtype=torch.int8)
    sc8 = torch.zeros(2, 2, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match=r"seq_lens must be \[batch\]"):
        b.gqa_decode_int8(q8, kv8, sc8, torch.ones(1, dtype=torch.int32), 1.0, torch.empty_like(q8))
    with pytest.raises(ValueError, match=r"seq_lens must be \[batch\]"):
        b.prepare_gqa_decode_int8(q8, kv8, sc8, torch.ones(3, dtype=torch.int32), torch.empty_like(q8))


def _paged(batch=2, T=1, P=16, num_pages=8, max_pages=4, width=128, kv_heads=8):
    q = torch.zeros(batch, T, 32, 128, dtype=torch.bfloat16)
    pool = torch.zeros(num_pages, 2, kv_heads, P, width, dtype=torch.bfloat16)
    table = torch.zeros(batch, max_pages, dtype=torch.int32)
    return q, pool, table, torch.ones(batch, dtype=torch.int32), torch.empty_like(q)


def test_binding_rejects_a_pool_whose_rows_are_not_as_wide_as_q():
    q, pool, table, lens, out = _paged(width=64)
    with pytest.raises(ValueError, match="kv_pages"):
        b.gqa_decode_paged(q, pool, table, lens, 1.0, out)
    with pytest.raises(ValueError, match="kv_pages"):
        b.prepare_gqa_decode_paged(q, pool, table, lens, out)
    q, pool, table, lens, out = _paged(kv_heads=4)
    with pytest.raises(ValueError, match="kv_pages"):
        b.gqa_decode_paged(q, pool, table, lens, 1.0, out)
    q, pool, table, lens, out = _paged()
    with pytest.raises(ValueError, match=r"seq_lens must be \[batch\]"):
        b.gqa_decode_paged(q, pool, table, lens[:1], 1.0, out)
    with pytest.raises(ValueError, match="same GPU"):
        b.gqa_decode_paged(q, pool, table, lens, 1.0, out)


def test_binding_rejects_positions_that_do_not_match_the_batch():
    kv = torch.zeros(2, 2, 8, 64, 128, dtype=torch.float16)
    k_new = torch.zeros(2, 8, 128, dtype=torch.float16)
    short = torch.zeros(1, dtype=torch.int32)
    with pytest.raises(ValueError, match=r"positions must be \[batch\]"):
        b.gqa_kv_append(kv, k_new, k_new.clone(), short)
    kv8 = torch.zeros(2, 2, 8, 64, 128, dtype=torch.int8)
    sc8 = torch.zeros(2, 2, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match=r"positions must be \[batch\]"):
        b.gqa_kv_append_int8(kv8, sc8, k_new, k_new.clone(), short)
    _, pool, table, _, _ = _paged()
    pk = torch.zeros(2, 1, 8, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match=r"positions must be \[batch\]"):
        b.gqa_kv_append_paged(pool, table, pk, pk.clone(), torch.zeros(3, dtype=torch.int32))
    pool8 = torch.zeros(8, 2, 8, 16, 128, dtype=torch.int8)
    psc8 = torch.zeros(8, 2, 8, 16, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match=r"positions must be \[batch\]"):
        b.gqa_kv_append_paged_int8(pool8, psc8, table, pk, pk.clone(), short)
    with pytest.raises(ValueError, match="same GPU"):
        b.gqa_kv_append(kv, k_new, k_new.clone(), torch.zeros(2, dtype=torch.int32))


# ---------------------------------------------------------------- allocation-free decode
def _no_alloc(d, q=Q, kv=KV, sc=None, lens=LENS, qs=1.0, out=OUT):
    return b._decode_no_alloc(ctypes.byref(d), q, kv, sc, lens, qs, out, None)


def test_no_alloc_refuses_what_it_cannot_do_without_touching_a_device():
    # A batch beyond the balanced split's limit takes the chunked split, whose
    # partials ([batch, 32, splits, 128] fp32) far exceed the static scratch:
    # refused with a message that names the sizes, before any device check.
    far = 1 << 42   # addresses far enough apart for a 1.3 TB cache
    assert _no_alloc(desc(batch=5000, capacity=65536, q=b.GQA_F16, kv=b.GQA_F16),
                     q=far, kv=2 * far, lens=3 * far, out=4 * far) == INVALID
    msg = b.last_error()
    assert "static scratch" in msg and str(4 << 20) in msg
    d = desc()
    d.flags = b.GQA_FLAG_FUSED_COMBINE
    assert _no_alloc(d) == INVALID and "flags" in b.last_error()
    assert _no_alloc(desc(), sc=SC) == INVALID and "kv_scales" in b.last_error()
    assert _no_alloc(desc(kv=b.GQA_INT8_ROWSCALE, hq=16)) == INVALID       # INT8 needs its scales
    assert _no_alloc(desc(), out=Q + 64) == ALIAS
    assert _no_alloc(desc(), qs=float("nan")) == INVALID
    assert _no_alloc(desc(batch=0), q=None, kv=None, lens=None, out=None) == OK
    # Valid arguments get as far as the device check (no GPU here).
    assert _no_alloc(desc(batch=8, capacity=65536)) not in (OK, INVALID, ALIAS)
    assert _no_alloc(desc(kv=b.GQA_INT8_ROWSCALE, hq=16), sc=SC) not in (OK, INVALID, ALIAS)
    assert b.NO_ALLOC_SCRATCH_BYTES == 4 << 20
    assert "#define GQA_NO_ALLOC_SCRATCH_BYTES ((size_t)4 << 20)" in open(HEADER).read()


def test_no_alloc_binding_needs_an_output_and_checks_shapes():
    q, kv, lens, out = _contig()
    with pytest.raises(TypeError):
        b.gqa_decode_no_alloc(q, kv, lens, 1.0)                  # no out: it would allocate
    with pytest.raises(ValueError, match=r"seq_lens must be \[batch\]"):
        b.gqa_decode_no_alloc(q, kv, lens[:1], 1.0, out)
    with pytest.raises(ValueError, match="same GPU"):
        b.gqa_decode_no_alloc(q, kv, lens, 1.0, out)
