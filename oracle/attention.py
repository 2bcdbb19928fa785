"""Reference attention over a paged KV cache, in float64 (oracle, test infrastructure).

The method: all sequences of a step are flattened into one super-sequence;
positions and an attention mask keep every sequence attending only to its own
tokens (Inside vLLM summary, "PagedAttentionの仕組み").  Paging changes where
K/V live, not the result, so for each sequence i this is ordinary causal
multi-head attention over the sequence's own K/V history.

Readings where the pages are silent:
  * causal alignment: the query at absolute position p = context_lens[i] + j
    attends to keys 0..p, itself included (bottom-right alignment for chunks);
  * grouped heads: query head h reads KV head h // (Hq // Hkv);
  * scores are scale * <q, k> and the scale is applied before the max;
  * the output is float64 here (the HIP path writes float32).

For every query row and head:
    s_t = scale * sum_d q[d] * K[t, d]        for t = 0..p
    w_t = exp(s_t - max_t s_t)
    out = sum_t w_t V[t] / sum_t w_t
"""
from __future__ import annotations

from typing import Iterable, Optional, Sequence

import numpy as np


def gather_sequence(cache: np.ndarray, table_row: Sequence[int], length: int,
                    block_size: int = 16) -> np.ndarray:
    """K or V of one sequence, positions 0..length-1, from a [NB, Hkv, bs, D] cache.

    Position t lives in block ``table_row[t // bs]`` at offset ``t % bs``.
    Returns [length, Hkv, D].
    """
    nblk = -(-length // block_size)
    ids = np.asarray(table_row[:nblk], dtype=np.int64)
    pages = cache[ids]  # [nblk, Hkv, bs, D]
    seq = pages.transpose(0, 2, 1, 3).reshape(nblk * block_size, cache.shape[1], cache.shape[3])
    return seq[:length]


def causal_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, positions: Sequence[int],
                     scale: float) -> np.ndarray:
    """Attention of query rows q [n, Hq, D] (absolute positions ``positions``) over
    K, V [L, Hkv, D] of the same sequence; row j sees keys 0..positions[j].
    Returns [n, Hq, D] float64."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    n, hq, d = q.shape
    L, hkv, _ = K.shape
    g = hq // hkv
    pos = np.asarray(positions, dtype=np.int64)
    if n and (pos.max() >= L or pos.min() < 0):
        raise ValueError("query position outside the sequence")
    masked = np.arange(L)[None, :] > pos[:, None]  # [n, L]: key after the query
    out = np.empty((n, hq, d), dtype=np.float64)
    for kvh in range(hkv):
        Kh = K[:, kvh, :]  # [L, D]
        Vh = V[:, kvh, :]
        for hh in range(g):
            h = kvh * g + hh
            s = scale * (q[:, h, :] @ Kh.T)  # [n, L]
            s = np.where(masked, -np.inf, s)
            m = s.max(axis=1, keepdims=True)
            w = np.exp(s - m)
            out[:, h, :] = (w @ Vh) / w.sum(axis=1, keepdims=True)
    return out


def ref_attention_paged(q, k_cache, v_cache, block_tables, seq_lens, query_start_loc,
                        context_lens, scale: float, block_size: int = 16,
                        seqs: Optional[Iterable[int]] = None) -> np.ndarray:
    """Outputs [T, Hq, D] float64 of the step; rows of sequences not in ``seqs`` stay NaN.

    q: [T, Hq, D] float64; caches: [NB, Hkv, bs, D] float64 (already decoded).
    """
    q = np.asarray(q, dtype=np.float64)
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    sl = np.asarray(seq_lens, dtype=np.int64)
    cl = np.asarray(context_lens, dtype=np.int64)
    out = np.full(q.shape, np.nan, dtype=np.float64)
    if seqs is None:
        seqs = range(len(sl))
    for i in seqs:
        r0, r1 = int(qsl[i]), int(qsl[i + 1])
        if r1 == r0:
            continue
        L = int(sl[i])
        if L != int(cl[i]) + (r1 - r0):
            raise ValueError(f"sequence {i}: seq_len != context_len + query_len")
        K = gather_sequence(k_cache, block_tables[i], L, block_size)
        V = gather_sequence(v_cache, block_tables[i], L, block_size)
        pos = int(cl[i]) + np.arange(r1 - r0)
        out[r0:r1] = causal_attention(q[r0:r1], K, V, pos, scale)
    return out


def ref_attention_dense(q_per_seq, k_per_seq, v_per_seq, context_lens, scale: float):
    """Same maths on each sequence's contiguous K/V history (no pool involved).

    q_per_seq[i]: [q_i, Hq, D]; k_per_seq[i], v_per_seq[i]: [L_i, Hkv, D].
    Returns a list of [q_i, Hq, D] float64 arrays.
    """
    outs = []
    for qi, Ki, Vi, c in zip(q_per_seq, k_per_seq, v_per_seq, context_lens):
        n = np.asarray(qi).shape[0]
        outs.append(causal_attention(qi, Ki, Vi, int(c) + np.arange(n), scale))
    return outs
