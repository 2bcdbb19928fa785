"""Metadata the kernels had to clamp shows up in the workspace's sticky flag word (GPU).

Metadata is trusted on the device, but no kernel indexes outside its buffers:
a block id outside the pool is read as the nearest valid block, and rows or a
context the block-table row cannot hold are clamped (the cache layout of the
Inside vLLM summary, section "PagedAttentionの仕組み": each request's tokens
live in the blocks of its block list).  Every kernel that clamps sets a bit
that pa_attention_flags reads back.  Each case runs on the kernels it names;
the bad values stay inside what the kernels' own clamps turn into in-bounds
reads, so nothing runs outside a buffer.
"""
import math

import numpy as np
import pytest
import torch

import paged_kv_varlen_reshape_amd as pk
import workloads as W
from workloads.device import build_device_step

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _reset_options():
    yield
    pk.pa_set_option(pk.PA_OPT_DECODE_KERNEL, 0)


def _step(name, reqs, hkv, g, d, dtype, seed):
    nb = sum(-(-r.seq_len // 16) for r in reqs) + 4
    order = np.random.default_rng((seed, 0)).permutation(nb).astype(np.int32)
    return W.StepSpec(name, seed, hkv * g, hkv, d, dtype, 16, nb, 1.0 / math.sqrt(d), reqs, initial_order=order,
                      table_rows=4096, seed=seed)


# (name, requests, kv heads, group, head dim, dtype): which planner and kernels serve the step
CASES = {
    # a small mixed bf16 step: the chunk kernel and the decode kernel plan it themselves
    "self-planned mixed bf16": ([W.Request(0, 0, 150), W.Request(1, 300, 1), W.Request(2, 40, 20),
                                 W.Request(3, 900, 1)], 8, 4, 128, "bf16"),
    # more than 2048 query tokens: the plan kernel, the chunk kernel's queues, the decode kernel
    "planned mixed bf16": ([W.Request(i, 64 * i, 500) for i in range(5)] + [W.Request(5, 700, 1),
                           W.Request(6, 33, 1)], 8, 4, 128, "bf16"),
    # float32: the plan kernel and the VALU row-wise kernel
    "planned mixed f32": ([W.Request(0, 0, 30), W.Request(1, 300, 1), W.Request(2, 77, 1)], 2, 2, 64, "f32"),
}


@pytest.mark.parametrize("case", list(CASES))
def test_block_ids_outside_the_pool_are_flagged(case):
    reqs, hkv, g, d, dtype = CASES[case]
    spec = _step(case, reqs, hkv, g, d, dtype, 800 + len(case))
    ds = build_device_step(spec)
    ds.reshape()
    ws = ds.workspace()
    pk.pa_attention_flags(ws, clear=True)
    ds.attention(workspace=ws)
    assert pk.pa_attention_flags(ws) == 0, "a consistent step sets no flag"
    bt = ds.block_tables.clone()
    for i, r in enumerate(spec.requests):  # a used page of a decode row and of a chunk row
        bt[i, (r.seq_len - 1) // 16] = spec.num_blocks + 7 if i % 2 else -3
    out = pk.pa_attention(ds.q, ds.k_cache, ds.v_cache, bt, ds.seq_lens, ds.query_start_loc, ds.context_lens,
                          spec.scale, workspace=ws, max_query_len=ds.max_query_len)
    torch.cuda.synchronize()
    flags = pk.pa_attention_flags(ws, clear=True)
    print(f"{case}: flags after out-of-pool block ids = {flags}", flush=True)
    assert flags & pk.PA_FLAG_BLOCK_ID and not flags & pk.PA_FLAG_ROWS
    assert pk.pa_attention_flags(ws) == 0, "cleared"
    ds.attention(workspace=ws)
    assert pk.pa_attention_flags(ws) == 0
    del out


@pytest.mark.parametrize("case", list(CASES))
def test_context_past_the_block_table_is_flagged(case):
    reqs, hkv, g, d, dtype = CASES[case]
    spec = _step(case, reqs, hkv, g, d, dtype, 810 + len(case))
    ds = build_device_step(spec, pad_value=-1)
    ds.reshape()
    ws = ds.workspace()
    pk.pa_attention_flags(ws, clear=True)
    ctx = ds.context_lens.clone()
    ctx[1] = ds.block_tables.shape[1] * 16  # no room left for its query row
    pk.pa_attention(ds.q, ds.k_cache, ds.v_cache, ds.block_tables, ds.seq_lens, ds.query_start_loc, ctx, spec.scale,
                    workspace=ws, max_query_len=ds.max_query_len)
    flags = pk.pa_attention_flags(ws, clear=True)
    print(f"{case}: flags after an oversized context = {flags}", flush=True)
    assert flags & pk.PA_FLAG_ROWS


def test_noalloc_workspace_flags():
    reqs, hkv, g, d, dtype = CASES["self-planned mixed bf16"]
    spec = _step("noalloc flags", reqs, hkv, g, d, dtype, 830)
    ds = build_device_step(spec)
    ds.reshape()
    out = torch.empty((spec.num_tokens, spec.num_q_heads, spec.head_dim), dtype=torch.float32, device="cuda")
    pk.pa_attention_flags(None, clear=True)
    pk.pa_attention_noalloc(ds.q, ds.k_cache, ds.v_cache, ds.block_tables, ds.seq_lens, ds.query_start_loc,
                            ds.context_lens, spec.scale, out=out, max_query_len=ds.max_query_len)
    assert pk.pa_attention_flags(None) == 0
    bt = ds.block_tables.clone()
    bt[1, 0] = spec.num_blocks
    pk.pa_attention_noalloc(ds.q, ds.k_cache, ds.v_cache, bt, ds.seq_lens, ds.query_start_loc, ds.context_lens,
                            spec.scale, out=out, max_query_len=ds.max_query_len)
    assert pk.pa_attention_flags(None, clear=True) & pk.PA_FLAG_BLOCK_ID
    assert pk.pa_attention_flags(None) == 0
