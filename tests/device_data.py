"""GPU-test helpers: the fp64 oracle on sampled sequences next to the device rows."""
from __future__ import annotations

import numpy as np
import torch

import workloads as W


def oracle_rows(spec: W.StepSpec, seqs, device_out: torch.Tensor, meta: W.StepMeta):
    """fp64 oracle output of sequences `seqs` (dense, from the seeded values) and the
    matching device rows, both as numpy [rows, Hq, D]."""
    from oracle import as_f64, causal_attention
    from oracle_data import bits

    want, got = [], []
    for i in seqs:
        r = spec.requests[i]
        if r.query == 0:
            continue
        q = as_f64(bits(W.q_values(spec, r)), spec.dtype)
        K = as_f64(bits(W.kv_values(spec, "k", r, 0, r.seq_len)), spec.dtype)
        V = as_f64(bits(W.kv_values(spec, "v", r, 0, r.seq_len)), spec.dtype)
        want.append(causal_attention(q, K, V, r.context + np.arange(r.query), spec.scale))
        r0, r1 = int(meta.query_start_loc[i]), int(meta.query_start_loc[i + 1])
        got.append(device_out[r0:r1].double().cpu().numpy())
    return np.concatenate(want), np.concatenate(got)
