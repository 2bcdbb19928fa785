"""The bench's algorithmic work, pinned without the GPU.

The roofline figures divide the work the method itself must do by a kernel's
time, so that work is checked here against counts made another way: the
chunked-prefill workload's causal flops worked out from its definition (8
chunks of 512 rows over 0/512/1024/1536 cached tokens, 32 query heads,
head_dim 128), causal (row, key) pairs counted one by one on small steps, and
unique K/V tokens counted from the block tables the reference pool hands out.
"""
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import workloads as W
from oracle import RefBlockPool

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_chunked_prefill_flops_from_its_definition():
    # a chunk of q rows over c cached tokens has q*c + q(q+1)/2 causal pairs per
    # head; 2 chunks at each of c = 0, 512, 1024, 1536 with q = 512; 4 flops per
    # pair, head_dim and query head (2 for Q.K^T, 2 for P.V)
    pairs = 2 * sum(512 * c + 512 * 513 // 2 for c in (0, 512, 1024, 1536))
    assert pairs == 4_196_352
    assert 4 * 128 * 32 * pairs == 68_753_031_168
    work = bench.algorithmic_work(W.make_config(3), mfma_rows=True)
    assert work["causal_flops"] == 68_753_031_168
    assert work["chunk_flops"] == 68_753_031_168


def _pairs_one_by_one(spec):
    n = 0
    for r in spec.requests:
        for j in range(r.query):
            pos = r.context + j
            n += sum(1 for t in range(r.seq_len) if t <= pos)
    return n


@pytest.mark.parametrize("seed", range(6))
def test_causal_flops_match_pair_count(seed):
    spec = W.random_spec(seed, num_seqs=5, max_context=60, max_query=12, num_q_heads=4, num_kv_heads=2,
                         head_dim=64, decode_fraction=0.4)
    work = bench.algorithmic_work(spec, mfma_rows=True)
    assert work["causal_flops"] == 4 * spec.head_dim * spec.num_q_heads * _pairs_one_by_one(spec)
    # rows split between the kernels: multi-row sequences to the chunk kernel
    chunk_spec_pairs = sum(
        4 * spec.head_dim * spec.num_q_heads * sum(r.context + j + 1 for j in range(r.query))
        for r in spec.requests if r.query > 1)
    assert work["chunk_flops"] == chunk_spec_pairs


@pytest.mark.parametrize("seed,prefix", [(0, 0), (1, 16), (2, 48), (3, 32)])
def test_unique_kv_bytes_match_block_tables(seed, prefix):
    spec = W.random_spec(seed, num_seqs=6, max_context=90, max_query=9, num_q_heads=4, num_kv_heads=2,
                         head_dim=64, prefix_tokens=prefix, decode_fraction=0.5)
    pool = RefBlockPool(spec.num_blocks, spec.block_size, spec.initial_order)
    meta = W.run_allocation_script(spec, pool)
    slots = set()
    for i, r in enumerate(spec.requests):
        for t in range(r.seq_len):
            slots.add((int(meta.block_tables[i, t // 16]), t % 16))
    elt = 4 if spec.dtype == "f32" else 2
    kv_token = 2 * spec.num_kv_heads * spec.head_dim * elt
    work = bench.algorithmic_work(spec, mfma_rows=True)
    assert work["kv_unique_bytes"] == len(slots) * kv_token
    assert work["kv_logical_bytes"] == sum(r.seq_len for r in spec.requests) * kv_token
    if prefix and sum(r.shares_prefix for r in spec.requests) > 1:
        assert work["kv_unique_bytes"] < work["kv_logical_bytes"]


def test_mixed_step_bytes_split_between_kernels():
    # every sequence's K/V is counted by the kernel that serves its rows
    spec = W.random_spec(7, num_seqs=8, max_context=200, max_query=40, num_q_heads=8, num_kv_heads=2,
                         head_dim=128, dtype="bf16", decode_fraction=0.5)
    work = bench.algorithmic_work(spec, mfma_rows=True)
    elt, hq, d = 2, spec.num_q_heads, spec.head_dim
    kv_token = 2 * spec.num_kv_heads * d * elt
    rows = lambda reqs: sum(r.query for r in reqs)
    extra = lambda reqs: rows(reqs) * hq * d * (elt + 4) + sum(-(-r.seq_len // 16) for r in reqs) * 4
    one = [r for r in spec.requests if r.query == 1]
    many = [r for r in spec.requests if r.query > 1]
    assert work["decode_kernel_bytes"] == sum(r.seq_len for r in one) * kv_token + extra(one)
    assert work["chunk_kernel_bytes"] == sum(r.seq_len for r in many) * kv_token + extra(many)


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_step_roofline_sums_kernel_classes_at_their_bounds():
    """The whole-step roofline: row-wise bytes over HBM plus, for the chunk rows, the
    larger of their bytes over HBM and their flops over the matrix cores.  On the
    chunked-prefill configuration (no row-wise rows) that is 68 753 031 168 flops at
    2.5 PFLOP/s = 27.5 us; on a decode-only step it is the bytes over 8 TB/s."""
    w3 = bench.algorithmic_work(W.make_config(3), mfma_rows=True)
    r3 = bench.step_roofline(w3, True, 0.110)
    assert w3["decode_kernel_bytes"] == 0
    assert abs(r3["t_roof_ms"] - 68_753_031_168 / 2.5e15 * 1e3) < 1e-12
    assert abs(r3["frac"] - r3["t_roof_ms"] / 0.110) < 1e-15
    w2 = bench.algorithmic_work(W.make_config(2), mfma_rows=False)
    r2 = bench.step_roofline(w2, False, 0.066, {"gather4k_GBps": 6600.0, "mfma_bf16_random_TFLOPs": 1850.0})
    assert abs(r2["t_roof_ms"] - w2["decode_kernel_bytes"] / 8e12 * 1e3) < 1e-12
    assert abs(r2["t_roof_measured_ms"] - w2["decode_kernel_bytes"] / 6.6e12 * 1e3) < 1e-12
    work = {"decode_kernel_bytes": 8e9, "chunk_kernel_bytes": 1e9, "chunk_flops": 5e12}
    r = bench.step_roofline(work, True, 2.0)
    assert abs(r["t_roof_ms"] - (1.0 + 2.0)) < 1e-12  # 8 GB at 8 TB/s, then 5 TFLOP at 2.5 PFLOP/s
