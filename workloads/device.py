"""Device-side step inputs for the GPU tests and the bench (harness glue, torch on the device).

Block ids and slots come from the C++ allocator (through the binding).  The
pre-step cache is filled the way earlier steps would have filled it: each
request's history rows are generated from the seeded tables and written with
pa_reshape_and_cache.  Unused slots hold a NaN pattern, so any read of a slot
the step does not own poisons the output.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

import paged_kv_varlen_reshape_amd as pk
import workloads as W

TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}
BITS_DT = {"f32": torch.int32, "bf16": torch.int16}


def poison_fill(shape, dtype: str, device) -> torch.Tensor:
    p = W.poison_bits(dtype)
    if dtype == "bf16":
        p = p - (1 << 16) if p >= 1 << 15 else p
    t = torch.full(shape, p, dtype=BITS_DT[dtype], device=device)
    return t.view(TORCH_DT[dtype])


@dataclass
class DeviceStep:
    spec: W.StepSpec
    meta: W.StepMeta
    pool: pk.BlockPool
    q: torch.Tensor
    k_new: torch.Tensor
    v_new: torch.Tensor
    slot_mapping: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    block_tables: torch.Tensor
    seq_lens: torch.Tensor
    query_start_loc: torch.Tensor
    context_lens: torch.Tensor

    @property
    def max_query_len(self) -> int:
        return max((r.query for r in self.spec.requests), default=0)

    def reshape(self):
        pk.pa_reshape_and_cache(self.k_new, self.v_new, self.slot_mapping, self.k_cache, self.v_cache)

    def attention(self, out=None, workspace=None):
        return pk.pa_attention(self.q, self.k_cache, self.v_cache, self.block_tables, self.seq_lens,
                               self.query_start_loc, self.context_lens, self.spec.scale, out=out,
                               workspace=workspace, max_query_len=self.max_query_len)

    def workspace(self):
        s = self.spec
        n = pk.pa_attention_workspace_size(s.num_seqs, s.num_tokens, s.num_q_heads, s.num_kv_heads,
                                           s.head_dim, self.meta.max_blocks_per_seq)
        return torch.empty(n, dtype=torch.uint8, device=self.q.device)


def _write_history(spec, pool, kc, vc, device, batch_tokens=1 << 21):
    """Write every request's cached tokens (positions < context) into the caches."""
    prefix_written = False
    pend_k, pend_v, pend_s, n_pend = [], [], [], 0

    def flush():
        nonlocal pend_k, pend_v, pend_s, n_pend
        if not n_pend:
            return
        k = torch.cat(pend_k)
        v = torch.cat(pend_v)
        s = torch.from_numpy(np.concatenate(pend_s)).to(device)
        pk.pa_reshape_and_cache(k, v, s, kc, vc)
        pend_k, pend_v, pend_s, n_pend = [], [], [], 0

    for r in spec.requests:
        start = 0
        if r.shares_prefix and spec.prefix_tokens:
            if prefix_written:
                start = spec.prefix_tokens  # shared blocks already hold the prefix
            prefix_written = True
        for a in range(start, r.context, batch_tokens):
            b = min(r.context, a + batch_tokens)
            pend_k.append(W.kv_values(spec, "k", r, a, b, device))
            pend_v.append(W.kv_values(spec, "v", r, a, b, device))
            pend_s.append(pool.slot_mapping(r.key, a, b - a))
            n_pend += b - a
            if n_pend >= batch_tokens:
                flush()
    flush()


def build_device_step(spec: W.StepSpec, device="cuda", pad_value: Optional[int] = None) -> DeviceStep:
    """Allocate, fill history and stage the step's inputs on the device.

    pad_value: block-table padding; None pads with a block the step never uses
    when the pool has one (so an over-read hits NaN), else -1."""
    pool = pk.BlockPool(spec.num_blocks, spec.block_size, spec.initial_order)
    meta = W.run_allocation_script(spec, pool, pad_value=-1)
    if pad_value is None:
        unused = np.setdiff1d(np.arange(spec.num_blocks), meta.block_tables[meta.block_tables >= 0])
        pad_value = int(unused[0]) if unused.size else -1
    bt = np.where(meta.block_tables < 0, pad_value, meta.block_tables).astype(np.int32)
    meta.block_tables = bt
    shape = (spec.num_blocks, spec.num_kv_heads, spec.block_size, spec.head_dim)
    kc = poison_fill(shape, spec.dtype, device)
    vc = poison_fill(shape, spec.dtype, device)
    _write_history(spec, pool, kc, vc, device)
    qs, ks, vs = [], [], []
    for r in spec.requests:
        if r.query:
            qs.append(W.q_values(spec, r, device))
            ks.append(W.kv_values(spec, "k", r, r.context, r.seq_len, device))
            vs.append(W.kv_values(spec, "v", r, r.context, r.seq_len, device))
    dt = TORCH_DT[spec.dtype]
    D = spec.head_dim
    q = torch.cat(qs) if qs else torch.empty((0, spec.num_q_heads, D), dtype=dt, device=device)
    k_new = torch.cat(ks) if ks else torch.empty((0, spec.num_kv_heads, D), dtype=dt, device=device)
    v_new = torch.cat(vs) if vs else torch.empty((0, spec.num_kv_heads, D), dtype=dt, device=device)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)
    return DeviceStep(spec, meta, pool, q.contiguous(), k_new.contiguous(), v_new.contiguous(),
                      dev(meta.slot_mapping), kc, vc, dev(bt), dev(meta.seq_lens), dev(meta.query_start_loc),
                      dev(meta.context_lens))
