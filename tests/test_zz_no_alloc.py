"""pa_attention_noalloc (through the C ABI) against pa_attention on the same steps (GPU).

The no-allocation entry point runs the same checks and kernels with the
library's static per-GPU workspace, so its output must equal pa_attention's
bit for bit, and both must match the fp64 oracle within the contract's
tolerance.  Two calls in a row, the second on a smaller step (the array keeps
the first call's contents), then a third on the larger step again.
"""
import numpy as np
import pytest
import torch

import paged_kv_varlen_reshape_amd as pk
import workloads as W
from workloads.device import build_device_step
from device_data import oracle_rows

pytestmark = pytest.mark.gpu
TOL = {"f32": 1e-5, "bf16": 1e-2}


def _both(ds):
    T, hq, d = ds.q.shape
    ref = ds.attention()
    out = torch.full((T, hq, d), float("nan"), dtype=torch.float32, device=ds.q.device)
    pk.pa_attention_noalloc(ds.q, ds.k_cache, ds.v_cache, ds.block_tables, ds.seq_lens, ds.query_start_loc,
                            ds.context_lens, ds.spec.scale, out=out, max_query_len=ds.max_query_len)
    torch.cuda.synchronize()
    return ref, out


def _check(name, ds, ref, out):
    assert torch.isfinite(out).all(), name
    assert torch.equal(out, ref), f"{name}: no-alloc output differs from pa_attention's"
    spec = ds.spec
    want, got = oracle_rows(spec, range(spec.num_seqs), out, ds.meta)
    err = float(np.abs(want - got).max())
    print(f"no-alloc {name}: equal to pa_attention, max_abs_err vs oracle {err:.3e}", flush=True)
    assert err <= TOL[spec.dtype], err


def test_noalloc_matches_pa_attention_twice_in_a_row():
    # a mixed bf16 step: plan, chunk kernel, row-wise decode and split merge all
    # use the workspace (GQA 4:1, prefix-shared blocks, chunks and decodes)
    big = build_device_step(W.random_spec(900, num_seqs=12, max_context=900, max_query=300, num_q_heads=32,
                                          num_kv_heads=8, head_dim=128, dtype="bf16", prefix_tokens=32,
                                          decode_fraction=0.5))
    big.reshape()
    # a smaller decode-only float32 step (the VALU kernel; fewer rows and ranges)
    small = build_device_step(W.random_spec(901, num_seqs=3, max_context=60, max_query=1, num_q_heads=4,
                                            num_kv_heads=2, head_dim=64, dtype="f32", decode_fraction=1.0))
    small.reshape()
    # and a small self-planned bf16 decode step (the decode kernel writes the header itself)
    tiny = build_device_step(W.random_spec(902, num_seqs=5, max_context=300, max_query=1, num_q_heads=16,
                                           num_kv_heads=2, head_dim=128, dtype="bf16", decode_fraction=1.0))
    tiny.reshape()
    assert small.q.shape[0] < big.q.shape[0] and tiny.q.shape[0] < big.q.shape[0]
    for name, ds in (("mixed bf16", big), ("decode f32 (smaller)", small), ("decode bf16 self-planned", tiny),
                     ("mixed bf16 again", big)):
        ref, out = _both(ds)
        _check(name, ds, ref, out)
