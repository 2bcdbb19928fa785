"""A multi-step engine loop: continuous batching over a block pool.

The engine of the Inside vLLM summary (techfeed.io, section "エンジンの中核：
スケジューラとKVキャッシュ管理") runs step after step: running requests decode one
token each, waiting requests are admitted and prefilled in chunks under a
per-step token budget (section "高度な機能群", chunked prefill), blocks come
from the free-block queue through allocate_slots, a request that cannot get
its blocks forces the preemption of the most recently admitted running
request, whose blocks are released and which later recomputes its tokens
from scratch, and finished requests release their blocks (section
"PagedAttentionの仕組み").

This module is workload glue like the rest of the package: it decides which
request runs how many tokens each step and calls the pool it is given (the
C++ allocator through the binding, or the oracle's reference pool) in that
order.  It holds none of the method's arithmetic.  Token values are a pure
function of (request key, position) (values.py), so a recomputed request
writes exactly the K/V it wrote before.

With ``prefix_cache`` on, requests that share a system prompt (section
"高度な機能群", Prefix Caching) find its full blocks in the pool's prefix index
when they are admitted, and so do preempted requests find their own released
blocks while the pool has not handed them out again; only the tokens past the
reused blocks are computed.  Block keys stand in for the hash of a block's
tokens chained with its predecessor's: the shared prompt's blocks have keys of
their own, every other block a key of its request and position.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

from .configs import PREFIX_KEY, Request, StepSpec
from .step import StepMeta, step_rows


@dataclass
class EngineRequest:
    key: int
    prompt: int  # prompt tokens
    output: int  # tokens generated after the prompt
    arrival: int  # first step at which it may be admitted
    known: int = 0  # tokens that exist (prompt, then each generated token)
    computed: int = 0  # tokens whose K/V is in the cache
    state: str = "waiting"  # waiting | running | finished
    admitted: int = -1  # admission order of the current run (-1 while waiting)
    preemptions: int = 0
    shares_prefix: bool = False  # starts with the shared system prompt

    @property
    def total(self) -> int:
        return self.prompt + self.output


@dataclass
class EngineConfig:
    num_blocks: int = 56  # tight: preemptions happen (11-38 over seeds 0-2)
    token_budget: int = 96  # tokens per step
    chunk: int = 48  # longest prefill chunk per request and step
    max_running: int = 12
    num_requests: int = 24
    prompt_range: tuple = (1, 160)
    output_range: tuple = (1, 40)
    arrival_span: int = 12  # arrivals spread over steps 0..arrival_span-1
    num_q_heads: int = 8
    num_kv_heads: int = 2
    head_dim: int = 64
    dtype: str = "f32"
    seed: int = 0
    prefix_cache: bool = False  # reuse cached full blocks at admission
    shared_prefix: int = 0  # tokens of a system prompt some requests start with (multiple of 16)
    share_fraction: float = 0.0


@dataclass
class EngineStep:
    index: int
    spec: StepSpec  # the step's requests (key, context, query) in super-sequence order
    meta: StepMeta  # block tables, slots and row arrays of the step
    preempted: List[int] = field(default_factory=list)  # keys preempted while forming it
    finished: List[int] = field(default_factory=list)  # keys that finished with it


class EngineLoop:
    """Forms steps one at a time against ``pool`` (allocate_slots / free / block_table_row /
    slot_mapping, as both pools provide)."""

    def __init__(self, cfg: EngineConfig, pool, table_rows: int = 4096):
        self.cfg = cfg
        self.pool = pool
        rng = np.random.default_rng((cfg.seed, 7))
        self.requests = [
            EngineRequest(key=i,
                          prompt=int(rng.integers(cfg.prompt_range[0], cfg.prompt_range[1] + 1)),
                          output=int(rng.integers(cfg.output_range[0], cfg.output_range[1] + 1)),
                          arrival=int(rng.integers(0, cfg.arrival_span)))
            for i in range(cfg.num_requests)
        ]
        if cfg.shared_prefix:
            share = np.random.default_rng((cfg.seed, 8)).random(cfg.num_requests) < cfg.share_fraction
            for r, sh in zip(self.requests, share):
                if sh:
                    r.shares_prefix = True
                    r.prompt += cfg.shared_prefix
        for r in self.requests:
            r.known = r.prompt
        self.cache_hits = 0  # blocks reused from the prefix index
        self.step_index = 0
        self.admissions = 0
        self.table_rows = table_rows
        self.preemptions = 0

    # -- prefix cache -------------------------------------------------------
    def block_key(self, r: EngineRequest, i: int) -> int:
        """Key of block i of request r (stands in for a chained hash of its tokens)."""
        if r.shares_prefix and (i + 1) * 16 <= self.cfg.shared_prefix:
            return (PREFIX_KEY << 32) | i
        return (1 << 62) | (r.key << 32) | i

    def _reuse_cached(self, r: EngineRequest) -> None:
        """At admission: take over the cached blocks of the request's leading full blocks,
        keeping the block of its last known token private (a step never writes into a
        block another request may read)."""
        n = (r.known - 1) // 16
        if not self.cfg.prefix_cache or n <= 0 or r.computed:
            return
        hits = self.pool.prefix_match(r.key, [self.block_key(r, i) for i in range(n)])
        r.computed = 16 * hits
        self.cache_hits += hits

    # -- step formation ----------------------------------------------------
    def done(self) -> bool:
        return all(r.state == "finished" for r in self.requests)

    def _preempt(self, victim: EngineRequest) -> None:
        self.pool.free(victim.key)
        victim.state = "waiting"
        victim.computed = 0  # recompute every existing token when readmitted
        victim.admitted = -1
        victim.preemptions += 1
        self.preemptions += 1

    def next_step(self) -> Optional[EngineStep]:
        """The next step, or None when every request has finished.  A step may hold no
        request (everything waits for blocks) only if nothing is running."""
        if self.done():
            return None
        cfg = self.cfg
        budget = cfg.token_budget
        sched: List[tuple] = []  # (request, query)
        preempted: List[int] = []

        def want(r: EngineRequest) -> int:
            if r.computed < r.known:  # prefill (or recompute) in chunks
                return min(cfg.chunk, r.known - r.computed)
            return 1  # decode: the newest token

        def try_schedule(r: EngineRequest, q: int) -> bool:
            while self.pool.allocate_slots(r.key, r.computed, q) is None:
                # preempt the latest-admitted running request that is not already in this step
                cands = [x for x in self.requests if x.state == "running" and x is not r
                         and all(x is not s for s, _ in sched)]
                if not cands:
                    return False
                victim = max(cands, key=lambda x: x.admitted)
                self._preempt(victim)
                preempted.append(victim.key)
            return True

        # running requests first, oldest admission first
        for r in sorted((x for x in self.requests if x.state == "running"), key=lambda x: x.admitted):
            if r.state != "running" or budget == 0:
                continue
            q = min(want(r), budget)
            if try_schedule(r, q):
                sched.append((r, q))
                budget -= q
            else:  # nothing left to preempt: this request yields its blocks and waits
                self._preempt(r)
                preempted.append(r.key)
        # then waiting requests in arrival order
        running = sum(1 for x in self.requests if x.state == "running")
        for r in sorted((x for x in self.requests if x.state == "waiting" and x.arrival <= self.step_index
                         and x.key not in preempted), key=lambda x: (x.arrival, x.key)):
            if budget == 0 or running >= cfg.max_running:
                break
            self._reuse_cached(r)
            q = min(want(r), budget)
            # a waiting request never preempts: it is admitted only if its blocks are free
            # (allocation is all or nothing, so a refusal leaves the pool unchanged)
            if self.pool.allocate_slots(r.key, r.computed, q) is None:
                self.pool.free(r.key)  # the blocks it reused wait in the pool again
                r.computed = 0
                break
            r.state = "running"
            r.admitted = self.admissions
            self.admissions += 1
            running += 1
            sched.append((r, q))
            budget -= q

        reqs = [Request(r.key, r.computed, q, shares_prefix=r.shares_prefix) for r, q in sched]
        spec = StepSpec(f"engine step {self.step_index}", 2000 + cfg.seed, cfg.num_q_heads, cfg.num_kv_heads,
                        cfg.head_dim, cfg.dtype, 16, cfg.num_blocks, 1.0 / math.sqrt(cfg.head_dim), reqs,
                        prefix_tokens=cfg.shared_prefix, table_rows=self.table_rows, seed=2000 + cfg.seed)
        qsl, seq_lens, ctx = step_rows(spec)
        width = max([spec.blocks_of(r) for r in reqs], default=1)
        bt = np.full((len(reqs), width), -1, dtype=np.int32)
        slots = np.empty(spec.num_tokens, dtype=np.int32)
        for i, r in enumerate(reqs):
            bt[i] = self.pool.block_table_row(r.key, width, -1)
            slots[qsl[i]:qsl[i + 1]] = self.pool.slot_mapping(r.key, r.context, r.query)
        meta = StepMeta(bt, slots, qsl, seq_lens, ctx, width)
        step = EngineStep(self.step_index, spec, meta, preempted)

        # the step runs: its tokens are now cached; prompts done -> one token generated
        for r, q in sched:
            r.computed += q
            if cfg.prefix_cache and r.computed // 16:  # its full blocks become findable
                self.pool.prefix_register(r.key, [self.block_key(r, i) for i in range(r.computed // 16)])
            if r.computed >= r.prompt and r.known < r.total and r.computed == r.known:
                r.known += 1
            if r.computed >= r.total:
                r.state = "finished"
                self.pool.free(r.key)
                step.finished.append(r.key)
        self.step_index += 1
        return step
