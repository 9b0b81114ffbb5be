"""gqa_decode_no_alloc (the allocation-free decode, for callers that cannot
allocate device memory) against gqa_decode / gqa_decode_int8 through the C
ABI: the same plan and kernels, so the outputs must be identical bit for bit,
and both within the contract tolerance of the fp64 oracle. Each case makes two
no-alloc calls in a row on the shared static scratch, the second with a
smaller input, so the second reads nothing the first left behind."""

import ctypes

import pytest
import torch

from gpu_util import Workload, all_pairs, compare, make_inputs, oracle_pairs, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()


def _b():
    import gqa_kv_cache_attn_amd.binding as b
    return b


def _pair(qd, kd, B, C, lo, hi, seed, hq=32):
    ks, vs = (1 / 64, 1 / 32) if kd == "fp8_e4m3" else ((0.5, 2.0) if kd == "int8" else (1.0, 1.0))
    w = Workload(f"noalloc_{qd}_{kd}_B{B}_C{C}", B, C, lo, hi, qd, kd, q_scale=0.75,
                 k_scale=ks, v_scale=vs, seed=seed, num_q_heads=hq)
    return w, make_inputs(w, device="cuda")


def _reference_call(inp, out):
    b = _b()
    if inp["kv_dtype"] == "int8":
        b.gqa_decode_int8(inp["q"], inp["kv"], inp["kv_scales"], inp["seq_lens"], inp["q_scale"],
                          out, k_scale=inp["k_scale"], v_scale=inp["v_scale"])
    else:
        b.gqa_decode(inp["q"], inp["kv"], inp["seq_lens"], inp["q_scale"], out,
                     k_scale=inp["k_scale"], v_scale=inp["v_scale"])


def _no_alloc_call(inp, out):
    _b().gqa_decode_no_alloc(inp["q"], inp["kv"], inp["seq_lens"], inp["q_scale"], out,
                             k_scale=inp["k_scale"], v_scale=inp["v_scale"],
                             kv_scales=inp["kv_scales"])


# (q dtype, kv dtype, query heads, first (B, C, lo, hi), second (B, C, lo, hi)):
# the first input takes the balanced split (its partials fill most of the
# scratch), the second a smaller plan: the chunked split, or the short route.
CASES = [
    ("bf16", "bf16", 32, (4, 20000, 1, 20000), (2, 3000, 1, 3000)),
    ("bf16", "fp8_e4m3", 32, (3, 40000, 20000, 40000), (1, 64, 64, 64)),
    ("f16", "f16", 32, (32, 8192, 1, 8192), (1, 1024, 1024, 1024)),
    ("bf16", "int8", 16, (2, 30000, 1, 30000), (3, 2000, 1, 2000)),
    ("f16", "fp8_e4m3", 16, (5, 9000, 1, 9000), (2, 500, 100, 500)),
]


@pytest.mark.parametrize("qd,kd,hq,first,second", CASES,
                         ids=[f"{c[0]}-{c[1]}-{c[2]}q" for c in CASES])
def test_no_alloc_matches_the_allocating_call_twice_in_a_row(qd, kd, hq, first, second):
    print(f"[case] no_alloc {qd}/{kd}/{hq}q {first} then {second}", flush=True)
    b = _b()
    for i, (B, C, lo, hi) in enumerate((first, second)):
        w, inp = _pair(qd, kd, B, C, lo, hi, seed=500 + 10 * i + len(qd) + hq, hq=hq)
        plan = b.gqa_plan(b.make_desc(inp["q"], inp["kv"], inp["k_scale"], inp["v_scale"]))
        print(f"[plan] call {i}: {plan}", flush=True)
        want = torch.full_like(inp["q"], float("nan"))
        got = torch.full_like(inp["q"], float("nan"))
        _reference_call(inp, want)
        _no_alloc_call(inp, got)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), f"call {i} differs"
        compare(got, oracle_pairs(inp, all_pairs(B) if B * 8 <= 64 else all_pairs(B)[::5]),
                inp, f"{w.name}/no_alloc call {i}")


def test_no_alloc_refuses_an_oversized_plan_and_leaves_out_untouched():
    b = _b()
    # 5000 requests take the chunked split, whose partials exceed the scratch;
    # the check runs before any pointer is used, so fake addresses are enough.
    far = 1 << 42
    d = b.GqaDesc(batch=5000, capacity=65536, num_q_heads=32, num_kv_heads=8, head_dim=128,
                  q_dtype=b.GQA_F16, kv_dtype=b.GQA_F16, k_scale=1.0, v_scale=1.0, flags=0)
    st = b._decode_no_alloc(ctypes.byref(d), far, 2 * far, None, 3 * far, 1.0, 4 * far, None)
    assert st == b.GQA_ERR_INVALID_ARG and "static scratch" in b.last_error()
    # A real call that is refused (a fused-merge flag) enqueues nothing.
    w, inp = _pair("bf16", "bf16", 2, 1000, 1, 1000, seed=9)
    out = torch.full_like(inp["q"], float("nan"))
    d = b.make_desc(inp["q"], inp["kv"], fused_combine=True)
    st = b._decode_no_alloc(ctypes.byref(d), inp["q"].data_ptr(), inp["kv"].data_ptr(), None,
                            inp["seq_lens"].data_ptr(), 1.0, out.data_ptr(),
                            torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == b.GQA_ERR_INVALID_ARG
    assert torch.isnan(out.float()).all()
