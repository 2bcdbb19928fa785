"""Multi-step engine loop (continuous batching with chunked prefill, preemption by
recompute and release of finished requests) on the CPU.

* The C++ allocator and the oracle's reference pool, driven by the same loop,
  form identical steps: the same requests, block tables and slots, step after
  step, through every preemption, and both end with every block free.
* The oracle scatter model across steps: each step's new K/V rows are written
  into one persistent host pool (which starts poisoned), and attention gathered
  through the step's block tables equals attention computed directly from each
  request's regenerated K/V (pages are reused by other requests after a
  release, and preempted requests rewrite their tokens into new blocks, so a
  stale or misplaced page shows up here).
"""
import numpy as np
import pytest

import paged_kv_varlen_reshape_amd as pk
import workloads as W
from oracle import RefBlockPool, as_f64, causal_attention, ref_attention_paged, ref_reshape_and_cache
from oracle_data import bits


def _steps(cfg, pool):
    eng = W.EngineLoop(cfg, pool)
    out = []
    while True:
        st = eng.next_step()
        if st is None:
            return out, eng
        out.append(st)
        assert len(out) < 5000, "engine loop does not terminate"


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_cpp_and_reference_pools_form_identical_steps(seed):
    cfg = W.EngineConfig(seed=seed)
    a, ea = _steps(cfg, pk.BlockPool(cfg.num_blocks, 16, None))
    b, eb = _steps(cfg, RefBlockPool(cfg.num_blocks, 16, None))
    assert len(a) == len(b)
    for sa, sb in zip(a, b):
        assert [(r.key, r.context, r.query) for r in sa.spec.requests] == \
               [(r.key, r.context, r.query) for r in sb.spec.requests]
        assert np.array_equal(sa.meta.block_tables, sb.meta.block_tables)
        assert np.array_equal(sa.meta.slot_mapping, sb.meta.slot_mapping)
        assert sa.preempted == sb.preempted and sa.finished == sb.finished
    assert ea.preemptions == eb.preemptions >= 5, "the pool must be tight enough to force preemptions"
    assert all(r.state == "finished" for r in ea.requests)
    assert ea.pool.num_free == eb.pool.num_free == cfg.num_blocks
    # every token of every request was computed at least once; preempted ones more than once
    assert sum(s.spec.num_tokens for s in a) >= sum(r.total for r in ea.requests)


def test_steps_respect_budget_chunk_and_slots():
    cfg = W.EngineConfig(seed=3)
    steps, _ = _steps(cfg, RefBlockPool(cfg.num_blocks, 16, None))
    for st in steps:
        assert st.spec.num_tokens <= cfg.token_budget
        assert all(1 <= r.query <= cfg.chunk for r in st.spec.requests)
        sm = st.meta.slot_mapping
        assert len(np.unique(sm)) == len(sm), "two tokens of a step share a slot"
        assert sm.min() >= 0 and sm.max() < cfg.num_blocks * 16
        # each token's slot lies in the block its table names for that position
        for i, r in enumerate(st.spec.requests):
            pos = r.context + np.arange(r.query)
            s = sm[st.meta.query_start_loc[i]:st.meta.query_start_loc[i + 1]]
            assert np.array_equal(s // 16, st.meta.block_tables[i][pos // 16])
            assert np.array_equal(s % 16, pos % 16)


@pytest.mark.parametrize("seed", [0, 2])
def test_scatter_and_gather_across_steps_match_regenerated_values(seed):
    cfg = W.EngineConfig(seed=seed)
    steps, eng = _steps(cfg, RefBlockPool(cfg.num_blocks, 16, None))
    spec0 = steps[0].spec
    shape = (cfg.num_blocks, cfg.num_kv_heads, 16, cfg.head_dim)
    kc = np.full(shape, W.poison_bits(cfg.dtype), dtype=np.uint32)
    vc = np.full(shape, W.poison_bits(cfg.dtype), dtype=np.uint32)
    worst = 0.0
    for st in steps:
        spec, meta = st.spec, st.meta
        if spec.num_tokens == 0:
            continue
        q = np.concatenate([bits(W.q_values(spec, r)) for r in spec.requests])
        kn = np.concatenate([bits(W.kv_values(spec, "k", r, r.context, r.seq_len)) for r in spec.requests])
        vn = np.concatenate([bits(W.kv_values(spec, "v", r, r.context, r.seq_len)) for r in spec.requests])
        kc, vc = ref_reshape_and_cache(kn, vn, meta.slot_mapping, kc, vc, 16)
        paged = ref_attention_paged(as_f64(q, spec.dtype), as_f64(kc, spec.dtype), as_f64(vc, spec.dtype),
                                    meta.block_tables, meta.seq_lens, meta.query_start_loc, meta.context_lens,
                                    spec.scale)
        for i, r in enumerate(spec.requests):
            K = as_f64(bits(W.kv_values(spec, "k", r, 0, r.seq_len)), spec.dtype)
            V = as_f64(bits(W.kv_values(spec, "v", r, 0, r.seq_len)), spec.dtype)
            want = causal_attention(as_f64(bits(W.q_values(spec, r)), spec.dtype), K, V,
                                    r.context + np.arange(r.query), spec.scale)
            got = paged[meta.query_start_loc[i]:meta.query_start_loc[i + 1]]
            assert np.isfinite(got).all(), f"step {st.index}: request {r.key} read a poisoned slot"
            worst = max(worst, float(np.abs(got - want).max()))
    assert worst <= 1e-12, worst
    assert spec0.seed == steps[-1].spec.seed  # one value table for the whole run
    assert eng.preemptions > 0
