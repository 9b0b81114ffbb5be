"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI,
compute the oracle on the same seeded inputs, compare to the contract."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from gqa_kv_cache_attn_amd.inputs import Workload, make_inputs, storage_bits  # noqa: F401
from oracle import decode_storage, gqa_decode_head

# Contract tolerances: max-abs error on the output, by KV dtype.
ATOL = {"f16": 2e-3, "bf16": 2e-3, "fp8_e4m3": 2e-2}
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


def run_decode(inp, path="convenience", num_splits=None, out=None, fused_combine=False):
    b = binding()
    if out is None:
        out = torch.empty_like(inp["q"])
    if path == "convenience":
        b.gqa_decode(inp["q"], inp["kv"], inp["seq_lens"], inp["q_scale"], out,
                     k_scale=inp["k_scale"], v_scale=inp["v_scale"])
        torch.cuda.synchronize()
        return out, None
    prep = b.prepare_gqa_decode(inp["q"], inp["kv"], inp["seq_lens"], out, inp["q_scale"],
                                num_splits=num_splits, k_scale=inp["k_scale"],
                                v_scale=inp["v_scale"], fused_combine=fused_combine)
    b.launch_gqa_decode_prepared(prep)
    torch.cuda.synchronize()
    return out, prep


def oracle_pairs(inp, pairs):
    """Oracle output rows [4, 128] (fp64) for each (request, KV head) pair."""
    q, kv = inp["q"], inp["kv"]
    lens = inp["seq_lens"].cpu().numpy()
    C = kv.shape[3]
    res = {}
    for (b, g) in pairs:
        L = int(lens[b])
        assert 1 <= L <= C, "oracle needs 1 <= L <= capacity"
        qrows = decode_storage(storage_bits(q[b, 4 * g:4 * g + 4]), inp["q_dtype"])
        k = decode_storage(storage_bits(kv[b, 0, g, :L]), inp["kv_dtype"])
        v = decode_storage(storage_bits(kv[b, 1, g, :L]), inp["kv_dtype"])
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
    Otherwise each element may also carry one output-format ulp of |ref|:
    |err| <= ATOL + ulp_out(|ref|). A bf16 output of magnitude >= 0.5 is
    already off by up to half an ulp (>= 2^-9 ~ 1.95e-3) from rounding alone,
    so short requests with large outputs need the format's resolution on top
    of the absolute bound."""
    got_all = decoded_out(out, inp["q_dtype"])
    atol = ATOL[inp["kv_dtype"]]
    errs, refs, excess = [], [], []
    for (b, g), ref in ref_pairs.items():
        got = got_all[b, 4 * g:4 * g + 4]
        assert np.all(np.isfinite(got)), f"{label}: non-finite output at (b={b}, g={g})"
        err = np.abs(got - ref)
        errs.append(err.max())
        refs.append(np.abs(ref).max())
        excess.append((err - out_ulp(ref, inp["q_dtype"])).max())
    max_err, max_ref = max(errs), max(refs)
    diag = {"max_abs_err": float(max_err), "max_abs_ref": float(max_ref),
            "rel_to_max": float(max_err / max_ref) if max_ref > 0 else 0.0,
            "max_err_minus_1ulp": float(max(excess))}
    print(f"[parity] {label} {diag}", flush=True)
    if contract_only:
        assert max_err <= atol, f"{label}: max abs err {max_err:.3e} > {atol} ({diag})"
    else:
        assert max(excess) <= atol, f"{label}: |err| - 1 ulp = {max(excess):.3e} > {atol} ({diag})"
    return diag

