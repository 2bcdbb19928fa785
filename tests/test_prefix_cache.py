"""Prefix cache index of the block pool (CPU).

Pins: a request that starts with the same prompt reuses the cached KV blocks
(Inside vLLM summary, section "高度な機能群", Prefix Caching), a released block
stays findable until the free queue hands it out again, then its key is gone.
Then the C++ pool and the oracle's reference pool in lockstep over random
operation sequences, and the engine loop with prefix caching: identical steps
on both pools, and the oracle scatter model over all steps still gathers
exactly the regenerated K/V (reused blocks hold the tokens their keys name).
"""
import numpy as np
import pytest

import paged_kv_varlen_reshape_amd as pk
import workloads as W
from oracle import RefBlockPool, as_f64, causal_attention, ref_attention_paged, ref_reshape_and_cache
from oracle_data import bits

POOLS = [pk.BlockPool, RefBlockPool]


def _rc(pool, b):
    return pool.refcount(b) if callable(pool.refcount) else pool.refcount[b]


@pytest.mark.parametrize("P", POOLS, ids=["cpp", "ref"])
def test_same_prompt_reuses_released_blocks(P):
    pool = P(8, 16, None)  # queue 0..7
    assert pool.allocate_slots(1, 0, 48) == [0, 1, 2]
    pool.prefix_register(1, [10, 11, 12])
    pool.free(1)  # queue 3..7, 0, 1, 2 (released blocks keep their keys)
    assert pool.num_free == 8 and pool.num_cached == 3
    assert pool.prefix_match(2, [10, 11, 99]) == 2  # the shared prompt's first two blocks
    assert pool.blocks(2) == [0, 1]
    assert pool.num_free == 6  # taken out of the queue
    assert pool.allocate_slots(2, 32, 20) == [3, 4]  # the rest from the head of the queue
    assert [_rc(pool, b) for b in (0, 1, 2)] == [1, 1, 0]


@pytest.mark.parametrize("P", POOLS, ids=["cpp", "ref"])
def test_key_lives_until_the_queue_hands_its_block_out(P):
    pool = P(4, 16, None)
    pool.allocate_slots(1, 0, 16)  # block 0
    pool.prefix_register(1, [7])
    pool.free(1)  # queue 1, 2, 3, 0
    assert pool.allocate_slots(2, 0, 48) == [1, 2, 3]
    assert pool.num_cached == 1  # block 0 still waits in the queue with its key
    pool.free(2)  # queue 0, 1, 2, 3
    assert pool.allocate_slots(3, 0, 16) == [0]  # handed out again: its contents go
    assert pool.num_cached == 0
    assert pool.prefix_match(4, [7]) == 0


@pytest.mark.parametrize("P", POOLS, ids=["cpp", "ref"])
def test_hit_on_a_live_block_shares_it(P):
    pool = P(6, 16, None)
    pool.allocate_slots(1, 0, 40)  # blocks 0, 1, 2
    pool.prefix_register(1, [5, 6])  # its two full blocks
    assert pool.prefix_match(2, [5, 6, 7]) == 2
    assert [_rc(pool, b) for b in (0, 1)] == [2, 2]
    pool.free(1)
    assert [_rc(pool, b) for b in (0, 1, 2)] == [1, 1, 0]
    assert pool.num_free == 4


@pytest.mark.parametrize("P", POOLS, ids=["cpp", "ref"])
def test_register_and_match_refusals_change_nothing(P):
    pool = P(4, 16, None)
    pool.allocate_slots(1, 0, 32)
    pool.prefix_register(1, [1, 2])
    err = pk.PAError if P is pk.BlockPool else ValueError
    with pytest.raises(err):
        pool.prefix_register(1, [1, 3])  # block 1 is cached under key 2
    with pytest.raises(err):
        pool.prefix_register(1, [1, 2, 3])  # more keys than blocks
    with pytest.raises(err):
        pool.prefix_match(1, [1])  # request already holds blocks
    assert pool.num_cached == 2 and pool.blocks(1) == [0, 1] and pool.num_free == 2
    pool.allocate_slots(2, 0, 16)  # block 2
    pool.prefix_register(2, [1])  # key 1 already names block 0: block 2 stays unindexed
    assert pool.num_cached == 2


@pytest.mark.parametrize("seed", range(6))
def test_random_operations_agree_with_reference(seed):
    rng = np.random.default_rng(seed)
    nb = int(rng.integers(8, 40))
    order = rng.permutation(nb).astype(np.int32)
    a, b = pk.BlockPool(nb, 16, order), RefBlockPool(nb, 16, order)
    live, next_req = {}, 0  # req -> tokens held
    for _ in range(400):
        op = rng.random()
        if op < 0.35 or not live:  # a new request, maybe reusing cached blocks
            req, next_req = next_req, next_req + 1
            keys = [int(k) for k in rng.integers(0, 12, size=int(rng.integers(0, 5)))]
            ha, hb = a.prefix_match(req, keys), b.prefix_match(req, keys)
            assert ha == hb
            live[req] = 16 * ha
        elif op < 0.65:  # grow
            req = int(rng.choice(list(live)))
            new = int(rng.integers(1, 40))
            ra, rb = a.allocate_slots(req, live[req], new), b.allocate_slots(req, live[req], new)
            assert ra == rb
            if ra is not None:
                live[req] += new
        elif op < 0.85:  # register full blocks under fresh or colliding keys
            req = int(rng.choice(list(live)))
            n = live[req] // 16
            keys = [int(k) for k in rng.integers(0, 12, size=n)]
            ea = eb = None
            try:
                a.prefix_register(req, keys)
            except pk.PAError:
                ea = True
            try:
                b.prefix_register(req, keys)
            except ValueError:
                eb = True
            assert ea == eb
        else:  # release
            req = int(rng.choice(list(live)))
            a.free(req)
            b.free(req)
            del live[req]
        assert a.num_free == b.num_free and a.num_cached == b.num_cached
        for req in live:
            assert a.blocks(req) == b.blocks(req)


def _run(cfg, pool):
    eng = W.EngineLoop(cfg, pool)
    steps = []
    while True:
        st = eng.next_step()
        if st is None:
            return steps, eng
        steps.append(st)
        assert len(steps) < 5000


@pytest.mark.parametrize("seed", [0, 1])
def test_engine_with_prefix_cache_agrees_with_reference(seed):
    cfg = W.EngineConfig(seed=seed, prefix_cache=True, shared_prefix=48, share_fraction=0.7)
    sa, ea = _run(cfg, pk.BlockPool(cfg.num_blocks, 16, None))
    sb, eb = _run(cfg, RefBlockPool(cfg.num_blocks, 16, None))
    assert len(sa) == len(sb) and ea.cache_hits == eb.cache_hits > 0
    for x, y in zip(sa, sb):
        assert [(r.key, r.context, r.query) for r in x.spec.requests] == \
               [(r.key, r.context, r.query) for r in y.spec.requests]
        assert np.array_equal(x.meta.block_tables, y.meta.block_tables)
        assert np.array_equal(x.meta.slot_mapping, y.meta.slot_mapping)
    # fewer tokens computed than without reuse
    plain, _ = _run(W.EngineConfig(seed=seed, shared_prefix=48, share_fraction=0.7),
                    RefBlockPool(cfg.num_blocks, 16, None))
    assert sum(s.spec.num_tokens for s in sa) < sum(s.spec.num_tokens for s in plain)


def test_reused_blocks_hold_the_tokens_their_keys_name():
    cfg = W.EngineConfig(seed=3, prefix_cache=True, shared_prefix=48, share_fraction=0.7)
    steps, eng = _run(cfg, RefBlockPool(cfg.num_blocks, 16, None))
    assert eng.cache_hits > 0
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
