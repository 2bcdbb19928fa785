"""The five step configurations of the paged-attention hot path, as seeded specs.

A step is one flattened "super-sequence": every request contributes ``query``
new tokens at absolute positions ``context .. context+query-1`` on top of
``context`` tokens already held in the paged KV cache (the flattening and the
per-sequence attention mask are described on page 1, "Inside vLLM" summary,
section on how PagedAttention works).  Block size is 16 tokens (same section).

Draws are seeded and reproducible:
  * lengths come from ``numpy.random.default_rng((cfg_id, 1))``;
  * the free-block queue starts as ``numpy.random.default_rng((cfg_id, 0)).permutation(NB)``.
Uniform integer draws are inclusive of both ends.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

# value-generation key of a shared prompt prefix (distinct from any request key)
PREFIX_KEY = 0x7FFF_0001
# request id under which a shared prefix is first allocated
PREFIX_REQ = -1

CONFIG_NAMES = {
    1: "tiny_fp32",
    2: "decode_bf16",
    3: "chunked_prefill_bf16",
    4: "mixed_8192_bf16",
    5: "long_prefix_bf16",
    6: "verify_bf16",  # an extra workload, not one of the five measured configurations
}


@dataclass
class Request:
    key: int  # request id; also the value-generation key of its private tokens
    context: int  # tokens already cached before the step (c_i)
    query: int  # tokens processed in this step (q_i)
    shares_prefix: bool = False  # first ``prefix_tokens`` positions are the shared prefix

    @property
    def seq_len(self) -> int:
        return self.context + self.query


@dataclass
class StepSpec:
    name: str
    cfg_id: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str  # "f32" or "bf16"
    block_size: int
    num_blocks: int
    scale: float
    requests: List[Request]
    prefix_tokens: int = 0
    initial_order: Optional[np.ndarray] = None
    table_rows: int = 4096
    seed: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return len(self.requests)

    @property
    def num_tokens(self) -> int:
        return sum(r.query for r in self.requests)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def elt_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def blocks_of(self, r: Request) -> int:
        return -(-r.seq_len // self.block_size)

    @property
    def max_blocks_per_seq(self) -> int:
        return max(self.blocks_of(r) for r in self.requests)


def _order(cfg_id: int, nb: int) -> np.ndarray:
    return np.random.default_rng((cfg_id, 0)).permutation(nb).astype(np.int32)


def _blocks(tokens: int, bs: int = 16) -> int:
    return -(-tokens // bs)


def make_config(cfg_id: int) -> StepSpec:
    """Return the seeded spec of step configuration ``cfg_id`` (1..5; 6 is an extra
    short-query workload)."""
    rng = np.random.default_rng((cfg_id, 1))
    if cfg_id == 1:
        # a 17-token fresh prefill (2 blocks) and two 1-token decodes over 5 and 33 cached tokens
        reqs = [Request(0, 0, 17), Request(1, 5, 1), Request(2, 33, 1)]
        nb = 16
        return StepSpec(CONFIG_NAMES[1], 1, 2, 2, 64, "f32", 16, nb, 1.0 / math.sqrt(64), reqs,
                        initial_order=_order(1, nb), table_rows=1024, seed=1)
    if cfg_id == 2:
        ctx = rng.integers(512, 2048, size=64, endpoint=True)
        reqs = [Request(i, int(c), 1) for i, c in enumerate(ctx)]
        nb = 16384
        return StepSpec(CONFIG_NAMES[2], 2, 32, 8, 128, "bf16", 16, nb, 1.0 / math.sqrt(128), reqs,
                        initial_order=_order(2, nb), table_rows=1 << 16, seed=2)
    if cfg_id == 3:
        ctx = [0, 512, 1024, 1536, 0, 512, 1024, 1536]
        reqs = [Request(i, c, 512) for i, c in enumerate(ctx)]
        nb = 1024
        return StepSpec(CONFIG_NAMES[3], 3, 32, 8, 128, "bf16", 16, nb, 1.0 / math.sqrt(128), reqs,
                        initial_order=_order(3, nb), table_rows=1 << 16, seed=3)
    if cfg_id == 4:
        chunk_ctx = rng.integers(0, 4096, size=4, endpoint=True)
        dec_ctx = rng.integers(1024, 8192, size=6144, endpoint=True)
        reqs = [Request(i, int(c), 512) for i, c in enumerate(chunk_ctx)]
        reqs += [Request(4 + i, int(c), 1) for i, c in enumerate(dec_ctx)]
        nb = sum(_blocks(r.seq_len) for r in reqs)
        return StepSpec(CONFIG_NAMES[4], 4, 32, 8, 128, "bf16", 16, nb, 1.0 / math.sqrt(128), reqs,
                        initial_order=_order(4, nb), table_rows=1 << 18, seed=4)
    if cfg_id == 5:
        prefix = 2048
        tails = rng.integers(1024, 30720, size=256, endpoint=True)
        longs = rng.integers(65536, 131072, size=16, endpoint=True)
        reqs = [Request(i, prefix + int(t), 1, shares_prefix=True) for i, t in enumerate(tails)]
        reqs += [Request(256 + i, int(c), 1) for i, c in enumerate(longs)]
        nb = _blocks(prefix)
        for r in reqs:
            nb += _blocks(r.seq_len) - (_blocks(prefix) if r.shares_prefix else 0)
        return StepSpec(CONFIG_NAMES[5], 5, 64, 8, 128, "bf16", 16, nb, 1.0 / math.sqrt(128), reqs,
                        prefix_tokens=prefix, initial_order=_order(5, nb), table_rows=1 << 18, seed=5)
    if cfg_id == 6:
        # speculative-decoding verification: each of 64 sequences checks 4 drafted tokens
        ctx = rng.integers(512, 2048, size=64, endpoint=True)
        reqs = [Request(i, int(c), 4) for i, c in enumerate(ctx)]
        nb = 16384
        return StepSpec(CONFIG_NAMES[6], 6, 32, 8, 128, "bf16", 16, nb, 1.0 / math.sqrt(128), reqs,
                        initial_order=_order(6, nb), table_rows=1 << 16, seed=6)
    raise ValueError(f"unknown config id {cfg_id}")


def random_spec(seed: int, num_seqs: int = 4, max_context: int = 40, max_query: int = 6,
                num_q_heads: int = 4, num_kv_heads: int = 2, head_dim: int = 64,
                dtype: str = "f32", spare_blocks: int = 4, prefix_tokens: int = 0,
                decode_fraction: float = 0.5, name: str = "random") -> StepSpec:
    """A small random step for parity and property tests (any mix of prefill/decode)."""
    rng = np.random.default_rng((1000 + seed, 1))
    reqs = []
    for i in range(num_seqs):
        share = prefix_tokens > 0 and rng.random() < 0.7
        lo = prefix_tokens if share else 0
        c = int(rng.integers(lo, max(lo, max_context) + 1))
        q = 1 if rng.random() < decode_fraction else int(rng.integers(1, max_query + 1))
        if c == 0 and q == 0:
            q = 1
        reqs.append(Request(i, c, q, shares_prefix=share))
    nb = _blocks(prefix_tokens) if prefix_tokens else 0
    for r in reqs:
        nb += _blocks(r.seq_len) - (_blocks(prefix_tokens) if r.shares_prefix else 0)
    nb += spare_blocks
    order = np.random.default_rng((1000 + seed, 0)).permutation(nb).astype(np.int32)
    return StepSpec(name, 1000 + seed, num_q_heads, num_kv_heads, head_dim, dtype, 16, nb,
                    1.0 / math.sqrt(head_dim), reqs, prefix_tokens=prefix_tokens,
                    initial_order=order, table_rows=2048, seed=1000 + seed)


def allocation_script(spec: StepSpec) -> List[Tuple]:
    """The order in which the step's requests ask a block pool for blocks.

    History first (as if earlier steps had run), then the step's new tokens, both in
    super-sequence order.  A shared prefix is allocated once under ``PREFIX_REQ``,
    shared by every request that uses it, then released by ``PREFIX_REQ`` so that
    each prefix block ends with one reference per sharing request.

    Ops: ("alloc", req, num_computed, num_new), ("share", req, src_req), ("free", req).
    """
    ops: List[Tuple] = []
    p = spec.prefix_tokens
    if p:
        ops.append(("alloc", PREFIX_REQ, 0, p))
    for r in spec.requests:
        if r.shares_prefix:
            ops.append(("share", r.key, PREFIX_REQ))
            ops.append(("alloc", r.key, p, r.context - p))
        else:
            ops.append(("alloc", r.key, 0, r.context))
    if p:
        ops.append(("free", PREFIX_REQ))
    for r in spec.requests:
        ops.append(("alloc", r.key, r.context, r.query))
    return ops
