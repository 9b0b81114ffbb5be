"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI,
compute the oracle on the same seeded inputs, compare to the contract."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from gqa_kv_cache_attn_amd.inputs import Workload, make_inputs, storage_bits  # noqa: F401
from oracle import decode_int8_rows, decode_storage, gqa_decode_head

# Contract tolerances: max-abs error on the output, by KV dtype. An INT8 cache
# with bf16 row scales decodes exactly (int8 and bf16 both widen exactly), like
# a 16-bit cache, so it is held to the 16-bit bound.
ATOL = {"f16": 2e-3, "bf16": 2e-3, "fp8_e4m3": 2e-2, "int8": 2e-3}
# Output ulp exponent offset (mantissa bits) by output dtype.
_MANT = {"f16": 10, "bf16": 7}


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU in this environment")
    name = torch.cuda.get_device_properties(0).gcnArchName
    assert name.startswith("gfx950"), f"expected an MI355X (gfx950), found {name}"


def binding():
    import gqa_kv_cache_attn_amd.binding as b  # fails loudly if the library is not built
    return b


def prepare(inp, out, num_splits=None, fused_combine=False):
    """prepare_gqa_decode, or its _int8 form for an INT8 cache."""
    b = binding()
    if inp["kv_dtype"] == "int8":
        return b.prepare_gqa_decode_int8(inp["q"], inp["kv"], inp["kv_scales"], inp["seq_lens"],
                                         out, inp["q_scale"], num_splits=num_splits,
                                         k_scale=inp["k_scale"], v_scale=inp["v_scale"],
                                         fused_combine=fused_combine)
    return b.prepare_gqa_decode(inp["q"], inp["kv"], inp["seq_lens"], out, inp["q_scale"],
                                num_splits=num_splits, k_scale=inp["k_scale"],
                                v_scale=inp["v_scale"], fused_combine=fused_combine)


def run_decode(inp, path="convenience", num_splits=None, out=None, fused_combine=False):
    b = binding()
    if out is None:
        out = torch.empty_like(inp["q"])
    if path == "convenience":
        if inp["kv_dtype"] == "int8":
            b.gqa_decode_int8(inp["q"], inp["kv"], inp["kv_scales"], inp["seq_lens"],
                              inp["q_scale"], out, k_scale=inp["k_scale"], v_scale=inp["v_scale"])
        else:
            b.gqa_decode(inp["q"], inp["kv"], inp["seq_lens"], inp["q_scale"], out,
                         k_scale=inp["k_scale"], v_scale=inp["v_scale"])
        torch.cuda.synchronize()
        return out, None
    prep = prepare(inp, out, num_splits, fused_combine)
    b.launch_gqa_decode_prepared(prep)
    torch.cuda.synchronize()
    return out, prep


def group_of(inp):
    """Query heads per KV head (4 for 32 query heads, 2 for 16)."""
    return inp["q"].shape[1] // 8


def decoded_kv_rows(inp, b, plane, g, L):
    """Decoded fp64 rows [L, 128] of one (request, plane, KV head) of the cache."""
    kv = inp["kv"]
    if inp["kv_dtype"] == "int8":
        return decode_int8_rows(storage_bits(kv[b, plane, g, :L]),
                                storage_bits(inp["kv_scales"][b, plane, g, :L]))
    return decode_storage(storage_bits(kv[b, plane, g, :L]), inp["kv_dtype"])


def oracle_pairs(inp, pairs):
    """Oracle output rows [G, 128] (fp64) for each (request, KV head) pair."""
    q, kv = inp["q"], inp["kv"]
    lens = inp["seq_lens"].cpu().numpy()
    C = kv.shape[3]
    G = group_of(inp)
    res = {}
    for (b, g) in pairs:
        L = int(lens[b])
        assert 1 <= L <= C, "oracle needs 1 <= L <= capacity"
        qrows = decode_storage(storage_bits(q[b, G * g:G * g + G]), inp["q_dtype"])
        k = decoded_kv_rows(inp, b, 0, g, L)
        v = decoded_kv_rows(inp, b, 1, g, L)
        res[(b, g)] = gqa_decode_head(qrows, k, v, inp["q_scale"], inp["k_scale"], inp["v_scale"])
    return res


def all_pairs(batch):
    return [(b, g) for b in range(batch) for g in range(8)]


def decoded_out(out, q_dtype):
    return decode_storage(storage_bits(out), q_dtype)


def out_ulp(ref, q_dtype):
    """One unit in the last place of the output format at |ref| (normal range)."""
    mag = np.maximum(np.abs(ref), 2.0 ** -14)
    return np.exp2(np.floor(np.log2(mag)) - _MANT[q_dtype])


def compare(out, ref_pairs, inp, label="", contract_only=False):
    """Check the output against the oracle rows.

    contract_only=True: the plain contract, max |err| <= ATOL[kv dtype].
    Otherwise each element may also carry the final rounding to the output
    format, half an output ulp of |ref|: |err| <= ATOL + ulp_out(|ref|) / 2.
    A bf16 output of magnitude >= 0.5 is already off by up to half an ulp
    (>= 2^-9 ~ 1.95e-3) from rounding alone, so short requests with large
    outputs need that on top of the absolute bound; the fp32 arithmetic
    before the rounding has to fit inside ATOL."""
    got_all = decoded_out(out, inp["q_dtype"])
    atol = ATOL[inp["kv_dtype"]]
    G = group_of(inp)
    errs, refs, excess = [], [], []
    for (b, g), ref in ref_pairs.items():
        got = got_all[b, G * g:G * g + G]
        assert np.all(np.isfinite(got)), f"{label}: non-finite output at (b={b}, g={g})"
        err = np.abs(got - ref)
        errs.append(err.max())
        refs.append(np.abs(ref).max())
        excess.append((err - 0.5 * out_ulp(ref, inp["q_dtype"])).max())
    max_err, max_ref = max(errs), max(refs)
    diag = {"max_abs_err": float(max_err), "max_abs_ref": float(max_ref),
            "rel_to_max": float(max_err / max_ref) if max_ref > 0 else 0.0,
            "max_err_minus_half_ulp": float(max(excess))}
    print(f"[parity] {label} {diag}", flush=True)
    if contract_only:
        assert max_err <= atol, f"{label}: max abs err {max_err:.3e} > {atol} ({diag})"
    else:
        assert max(excess) <= atol, f"{label}: |err| - ulp/2 = {max(excess):.3e} > {atol} ({diag})"
    return diag



# ------------------------------------------------------------------ paged cache
def run_paged(inp, path="prepared", num_splits=None, out=None):
    """Run the paged entry points on make_paged_inputs() tensors; returns (out, prepared)."""
    b = binding()
    if out is None:
        out = torch.empty_like(inp["q"])
    args = (inp["q"], inp["kv_pages"], inp["block_table"], inp["seq_lens"])
    kw = dict(k_scale=inp["k_scale"], v_scale=inp["v_scale"], kv_scales=inp["kv_scales"],
              scales_by_position=inp.get("scales_by_position", False))
    if path == "convenience":
        b.gqa_decode_paged(*args, inp["q_scale"], out, **kw)
        torch.cuda.synchronize()
        return out, None
    prep = b.prepare_gqa_decode_paged(*args, out, inp["q_scale"], num_splits=num_splits, **kw)
    b.launch_gqa_decode_prepared(prep)
    torch.cuda.synchronize()
    return out, prep


def paged_oracle_request(inp, b, seq_len=None):
    """Oracle output [T, Hq, 128] (fp64) of request b: its pages decoded from the
    stored bits and relabelled 0..n-1 (relabelling is a pinned invariance)."""
    from oracle.paged import gqa_decode_multi, gqa_decode_paged_reference, int8_rows_by_position
    P = inp["page_size"]
    L = int(inp["seq_lens"][b]) if seq_len is None else seq_len
    n = max(1, -(-L // P))
    ids = inp["block_table"][b, :n].long()
    pages = inp["kv_pages"].index_select(0, ids)
    q = decode_storage(storage_bits(inp["q"][b:b + 1]), inp["q_dtype"])
    if inp.get("scales_by_position"):
        # the scales stay with the request's positions: slots 0 .. n P - 1
        rows = int8_rows_by_position(storage_bits(pages), storage_bits(inp["kv_scales"][b:b + 1, :, :, :n * P]),
                                     np.arange(n)[None, :], [L], P)
        return gqa_decode_multi(q, rows, [L], inp["q_scale"], inp["k_scale"], inp["v_scale"])[0]
    if inp["kv_dtype"] == "int8":
        dec = decode_int8_rows(storage_bits(pages), storage_bits(inp["kv_scales"].index_select(0, ids)))
    else:
        dec = decode_storage(storage_bits(pages), inp["kv_dtype"])
    ref = gqa_decode_paged_reference(q, dec, np.arange(n)[None, :], [L], P, inp["q_scale"],
                                     inp["k_scale"], inp["v_scale"])
    return ref[0]


def compare_paged(out, inp, requests, label=""):
    """Every row of the listed requests against the oracle, to the contract
    bound plus half an output ulp (as compare())."""
    got_all = decoded_out(out, inp["q_dtype"])
    atol = ATOL[inp["kv_dtype"]]
    worst, worst_ref = 0.0, 0.0
    for b in requests:
        ref = paged_oracle_request(inp, b)
        got = got_all[b]
        assert np.all(np.isfinite(got)), f"{label}: non-finite output in request {b}"
        excess = (np.abs(got - ref) - 0.5 * out_ulp(ref, inp["q_dtype"])).max()
        worst = max(worst, float(np.abs(got - ref).max()))
        worst_ref = max(worst_ref, float(np.abs(ref).max()))
        assert excess <= atol, f"{label}: request {b}: |err| - ulp/2 = {excess:.3e} > {atol}"
    print(f"[parity] {label} max_abs_err={worst:.3e} max_abs_ref={worst_ref:.3e}", flush=True)
    return worst
