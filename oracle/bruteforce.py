"""Pure-Python brute force of the super-sequence attention (oracle, test infrastructure).

Written straight from the description of the flattened step (Inside vLLM
summary, "PagedAttentionの仕組み"): every K/V token of every sequence sits in
one list; a 0/1 mask built from (sequence id, position) pairs lets a query see
only tokens of its own sequence at positions not after its own.  No paging, no
max subtraction, exact sums with ``math.fsum``.  Tiny inputs only.
"""
from __future__ import annotations

import math
from typing import List, Sequence, Tuple


def ref_bruteforce(q_rows: Sequence, q_seq: Sequence[int], q_pos: Sequence[int],
                   kv_tokens: Sequence[Tuple[int, int, Sequence, Sequence]],
                   scale: float, num_q_heads: int, num_kv_heads: int) -> List[List[List[float]]]:
    """q_rows[r][h][d]: query rows; kv_tokens: (seq, pos, k[hkv][d], v[hkv][d]) for
    every token of the super-sequence (cached or new).  Returns out[r][h][d]."""
    group = num_q_heads // num_kv_heads
    out = []
    for r, qr in enumerate(q_rows):
        row = []
        for h in range(num_q_heads):
            kvh = h // group
            weights, vals = [], []
            for (seq, pos, k, v) in kv_tokens:
                visible = 1 if (seq == q_seq[r] and pos <= q_pos[r]) else 0
                if not visible:
                    continue
                s = scale * math.fsum(float(qr[h][d]) * float(k[kvh][d]) for d in range(len(qr[h])))
                weights.append(math.exp(s))
                vals.append(v[kvh])
            den = math.fsum(weights)
            dim = len(qr[h])
            row.append([math.fsum(w * float(vv[d]) for w, vv in zip(weights, vals)) / den
                        for d in range(dim)])
        out.append(row)
    return out
