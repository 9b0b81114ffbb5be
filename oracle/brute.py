"""Pure-Python brute force of the decode step, for tiny inputs only.

TEST INFRASTRUCTURE ONLY. It is deliberately independent of ``gqa_oracle``:
plain nested loops, ``math.fsum`` for every sum and ``math.exp`` for the
explicit softmax ``exp(s_j) / sum_i exp(s_i)`` (no max shift: inputs are
tiny, so nothing overflows). Same definition as the fp64 oracle, written a
second way so the two can pin each other.

Query head h reads KV head h // 4 (FlashInfer sm110_gqa_decode article,
"convenience API": the q.view(batch, 8, 4, 128) grouped view); fp8 scales act
on scores and on the output (Thor FP8 KV notes, patch 2).
"""

from __future__ import annotations

import math


def brute_decode(q, kv, seq_lens, q_scale=1.0, k_scale=1.0, v_scale=1.0):
    """q: nested lists [B][32][128]; kv: [B][2][8][C][128]; returns [B][32][128]."""
    n_q_heads = len(q[0])
    n_kv_heads = len(kv[0][0])
    group = n_q_heads // n_kv_heads
    dim = len(q[0][0])
    c = q_scale * k_scale / math.sqrt(dim)
    out = []
    for b in range(len(q)):
        L = int(seq_lens[b])
        rows_out = []
        for h in range(n_q_heads):
            g = h // group
            scores = [c * math.fsum(q[b][h][d] * kv[b][0][g][j][d] for d in range(dim))
                      for j in range(L)]
            ex = [math.exp(s) for s in scores]
            z = math.fsum(ex)
            rows_out.append([v_scale * math.fsum(ex[j] * kv[b][1][g][j][d] for j in range(L)) / z
                             for d in range(dim)])
        out.append(rows_out)
    return out
