"""Glue that drives a block pool through a spec's allocation script.

The pool is passed in (the C++ allocator through the Python binding, or the
oracle's reference pool); this module only calls its methods in the order the
script gives and packs the per-step index arrays.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .configs import StepSpec, allocation_script


@dataclass
class StepMeta:
    block_tables: np.ndarray  # [S, max_blocks_per_seq] int32
    slot_mapping: np.ndarray  # [T] int32
    query_start_loc: np.ndarray  # [S+1] int32
    seq_lens: np.ndarray  # [S] int32
    context_lens: np.ndarray  # [S] int32
    max_blocks_per_seq: int


def step_rows(spec: StepSpec):
    """query_start_loc, seq_lens, context_lens of the flattened step (int32)."""
    q = np.array([r.query for r in spec.requests], dtype=np.int64)
    c = np.array([r.context for r in spec.requests], dtype=np.int64)
    qsl = np.zeros(len(q) + 1, dtype=np.int64)
    np.cumsum(q, out=qsl[1:])
    return qsl.astype(np.int32), (c + q).astype(np.int32), c.astype(np.int32)


def run_allocation_script(spec: StepSpec, pool, pad_value: int = -1,
                          width: int | None = None) -> StepMeta:
    """Run the spec's allocation script on ``pool`` and return the step's index arrays.

    Raises RuntimeError if the pool runs out of blocks.
    """
    for op in allocation_script(spec):
        if op[0] == "alloc":
            _, req, done, new = op
            if pool.allocate_slots(req, done, new) is None:
                raise RuntimeError(f"pool exhausted allocating {new} tokens for request {req}")
        elif op[0] == "share":
            _, req, src = op
            pool.share_prefix(req, pool.blocks(src))
        elif op[0] == "free":
            pool.free(op[1])
        else:  # pragma: no cover
            raise ValueError(op)
    qsl, seq_lens, ctx = step_rows(spec)
    w = width if width is not None else spec.max_blocks_per_seq
    bt = np.full((spec.num_seqs, w), pad_value, dtype=np.int32)
    for i, r in enumerate(spec.requests):
        bt[i] = pool.block_table_row(r.key, w, pad_value)
    slots = np.empty(spec.num_tokens, dtype=np.int32)
    for i, r in enumerate(spec.requests):
        if r.query:
            slots[qsl[i]:qsl[i + 1]] = pool.slot_mapping(r.key, r.context, r.query)
    return StepMeta(bt, slots, qsl, seq_lens, ctx, w)
