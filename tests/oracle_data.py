"""Host-side step data for oracle tests: every value from the seeded generator,
every block id from the reference pool, every cache write from the oracle scatter."""
from __future__ import annotations

from dataclasses import dataclass
from typing import List

import numpy as np
import torch

import workloads as W
from oracle import RefBlockPool, as_f64, ref_reshape_and_cache


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw element bits of a CPU tensor (uint16 for bf16, uint32 for float32)."""
    t = t.contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy().view(np.uint32)
    raise TypeError(t.dtype)


@dataclass
class OracleStep:
    spec: W.StepSpec
    meta: W.StepMeta
    pool: RefBlockPool
    q: np.ndarray  # [T, Hq, D] bits
    k_new: np.ndarray  # [T, Hkv, D] bits
    v_new: np.ndarray
    k_cache_pre: np.ndarray  # [NB, Hkv, 16, D] bits (history only, rest poison)
    v_cache_pre: np.ndarray
    k_full: List[np.ndarray]  # per sequence [L, Hkv, D] bits, contiguous
    v_full: List[np.ndarray]

    def f64(self, a):
        return as_f64(a, self.spec.dtype)


def build_oracle_step(spec: W.StepSpec, pad_value: int = -1) -> OracleStep:
    pool = RefBlockPool(spec.num_blocks, spec.block_size, spec.initial_order)
    meta = W.run_allocation_script(spec, pool, pad_value=pad_value)
    bdt = np.uint16 if spec.dtype == "bf16" else np.uint32
    shape = (spec.num_blocks, spec.num_kv_heads, spec.block_size, spec.head_dim)
    kc = np.full(shape, W.poison_bits(spec.dtype), dtype=bdt)
    vc = np.full(shape, W.poison_bits(spec.dtype), dtype=bdt)
    q_rows, kn, vn, kf, vf = [], [], [], [], []
    for r in spec.requests:
        k_all = bits(W.kv_values(spec, "k", r, 0, r.seq_len))
        v_all = bits(W.kv_values(spec, "v", r, 0, r.seq_len))
        kf.append(k_all)
        vf.append(v_all)
        if r.context:
            hist_slots = pool.slot_mapping(r.key, 0, r.context)
            kc, vc = ref_reshape_and_cache(k_all[: r.context], v_all[: r.context], hist_slots,
                                           kc, vc, spec.block_size)
        if r.query:
            q_rows.append(bits(W.q_values(spec, r)))
            kn.append(k_all[r.context:])
            vn.append(v_all[r.context:])
    D = spec.head_dim
    q = np.concatenate(q_rows) if q_rows else np.zeros((0, spec.num_q_heads, D), bdt)
    k_new = np.concatenate(kn) if kn else np.zeros((0, spec.num_kv_heads, D), bdt)
    v_new = np.concatenate(vn) if vn else np.zeros((0, spec.num_kv_heads, D), bdt)
    return OracleStep(spec, meta, pool, q, k_new, v_new, kc, vc, kf, vf)
