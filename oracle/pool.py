"""Reference block pool (oracle, test infrastructure).

Follows the block-allocation procedure of the Inside vLLM summary, section
"PagedAttentionの仕組み":
  1. a request that will hold ``num_computed + num_new`` tokens needs
     ceil(tokens / block_size) blocks in total, i.e. that many minus the blocks
     it already holds (the page's worked example: 17 tokens -> 2 blocks);
  2. if the free pool cannot supply them, some request has to be preempted and
     recomputed; choosing the victim is scheduler policy, so here the call
     fails with no side effect and the caller decides;
  3. otherwise the first n blocks at the head of ``free_block_queue`` are
     removed and appended to the request's list in ``req_to_blocks``.
Blocks that tokens no longer need go back to the pool (engr-sng explainer,
paragraph on Paging Attention); here ``free`` drops one reference from each of
the request's blocks, in the request's block order, and appends every block
whose count reaches zero to the tail of the queue.  Prefix caching (Inside vLLM
summary, "高度な機能群") lets requests reuse cached KV blocks: ``share_prefix``
appends already-allocated blocks to a request and adds one reference to each.
The prefix cache index (that section, and the architecture overview's block
pool holding it): ``prefix_register`` files a request's full blocks under
caller keys; ``prefix_match`` gives a new request the blocks of its leading
keys, one reference each, up to the first miss.  A block released to zero
references keeps its key and stays findable until the queue hands it out
again (which drops the key); a hit on such a block takes it out of the queue.

Slot of the token at absolute position ``pos`` of a request:
``block_list[pos // block_size] * block_size + pos % block_size``.
"""
from __future__ import annotations

from collections import deque
from typing import Dict, List, Optional

import numpy as np


class RefBlockPool:
    def __init__(self, num_blocks: int, block_size: int = 16, initial_order=None):
        if initial_order is None:
            initial_order = range(num_blocks)
        order = [int(b) for b in initial_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("initial_order must be a permutation of range(num_blocks)")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free_block_queue: deque = deque(order)
        self.req_to_blocks: Dict[int, List[int]] = {}
        self.refcount = [0] * num_blocks
        self.cache: Dict[int, int] = {}  # key -> block
        self.block_key: Dict[int, int] = {}  # block -> key

    # -- allocation ---------------------------------------------------------
    def blocks_needed(self, req: int, num_computed: int, num_new: int) -> int:
        total = num_computed + num_new
        have = len(self.req_to_blocks.get(req, []))
        return max(0, -(-total // self.block_size) - have)

    def allocate_slots(self, req: int, num_computed: int, num_new: int) -> Optional[List[int]]:
        if num_computed < 0 or num_new < 0:
            raise ValueError("token counts must be non-negative")
        n = self.blocks_needed(req, num_computed, num_new)
        if n > len(self.free_block_queue):
            return None  # caller must preempt; nothing changed
        new = [self.free_block_queue.popleft() for _ in range(n)]
        for b in new:
            if b in self.block_key:  # reused: its cached contents go away
                del self.cache[self.block_key.pop(b)]
            self.refcount[b] = 1
        self.req_to_blocks.setdefault(req, []).extend(new)
        return new

    def share_prefix(self, req: int, ids) -> None:
        ids = [int(b) for b in ids]
        for b in ids:
            if not (0 <= b < self.num_blocks) or self.refcount[b] <= 0:
                raise ValueError(f"block {b} is not allocated")
        for b in ids:
            self.refcount[b] += 1
        self.req_to_blocks.setdefault(req, []).extend(ids)

    def free(self, req: int) -> None:
        for b in self.req_to_blocks.pop(req, []):
            self.refcount[b] -= 1
            if self.refcount[b] == 0:
                self.free_block_queue.append(b)

    # -- prefix cache -------------------------------------------------------
    def prefix_match(self, req: int, keys) -> int:
        if self.req_to_blocks.get(req):
            raise ValueError("request already holds blocks")
        hits = 0
        for k in keys:
            b = self.cache.get(int(k))
            if b is None:
                break
            if self.refcount[b] == 0:
                self.free_block_queue.remove(b)
            self.refcount[b] += 1
            self.req_to_blocks.setdefault(req, []).append(b)
            hits += 1
        return hits

    def prefix_register(self, req: int, keys) -> None:
        ids = self.req_to_blocks.get(req, [])
        keys = [int(k) for k in keys]
        if len(keys) > len(ids):
            raise ValueError("request holds fewer blocks than keys")
        for k, b in zip(keys, ids):
            if b in self.block_key and self.block_key[b] != k:
                raise ValueError(f"block {b} is cached under another key")
        for k, b in zip(keys, ids):
            if b in self.block_key or k in self.cache:
                continue
            self.cache[k] = b
            self.block_key[b] = k

    @property
    def num_cached(self) -> int:
        return len(self.cache)

    # -- queries ------------------------------------------------------------
    @property
    def num_free(self) -> int:
        return len(self.free_block_queue)

    def blocks(self, req: int) -> List[int]:
        return list(self.req_to_blocks.get(req, []))

    def block_table_row(self, req: int, width: int, pad_value: int = -1) -> np.ndarray:
        ids = self.req_to_blocks.get(req, [])
        if len(ids) > width:
            raise ValueError("block table row too narrow")
        row = np.full(width, pad_value, dtype=np.int32)
        row[: len(ids)] = ids
        return row

    def slot_mapping(self, req: int, start_pos: int, n: int) -> np.ndarray:
        ids = self.req_to_blocks.get(req, [])
        bs = self.block_size
        out = np.empty(n, dtype=np.int32)
        for j in range(n):
            pos = start_pos + j
            if pos // bs >= len(ids):
                raise ValueError(f"position {pos} has no block")
            out[j] = ids[pos // bs] * bs + pos % bs
        return out
