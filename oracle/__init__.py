"""CPU oracle for single-token grouped-query decode attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute anything in this package: only the test suite, the graft smoke entry
and the benchmark's ``cpu_baseline`` leg use it. It shares no code with the
HIP library or its Python binding, and imports neither.

Modules:
  gqa_oracle  vectorised fp64 numpy definition of the decode step, plus the
              exact decoders for the stored KV/query formats.
  brute       pure-Python loops (math.fsum / math.exp) for tiny inputs.
  kv_append   the cache write before a decode step (fp8 and INT8 quantise-on-write).
  paged       decode over a paged cache (page pool + block table) with T
              query tokens per request, causal among themselves, and the
              append of T new tokens per request into the pool.

Every function is pinned by ``tests/test_oracle_pins.py`` (and
``tests/test_oracle_pins_paged.py`` for ``paged``) against facts fixed
by the pages or by mathematics (closed forms, invariants, a library special
case, brute force). No function here is "parity unpinned".
"""

from .gqa_oracle import (  # noqa: F401
    HEAD_DIM,
    NUM_KV_HEADS,
    NUM_Q_HEADS,
    GROUP,
    decode_bf16_bits,
    decode_e4m3fn_bits,
    decode_e4m3fn_lookup,
    decode_f16_bits,
    decode_int8_rows,
    decode_storage,
    e4m3fn_table,
    gqa_decode_head,
    gqa_decode_reference,
    gqa_decode_weights,
)
