"""Pins of the oracle against facts that do not come from the oracle itself.

Each check takes the implementation under test as arguments so that the same
checks can be run against deliberately broken copies (see test_oracle_mutants).
Every check raises AssertionError on failure.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

import workloads as W
from oracle import RefBlockPool, ref_bruteforce
from oracle_data import build_oracle_step

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def rng_qkv(seed, n, L, hq, hkv, d):
    r = np.random.default_rng(seed)
    return r.standard_normal((n, hq, d)), r.standard_normal((L, hkv, d)), r.standard_normal((L, hkv, d))


# --------------------------------------------------------------------------- pool pins
def pin_block_count(pool_cls=RefBlockPool):
    g = golden("block_count.json")
    for case in g["cases"]:
        pool = pool_cls(64, g["block_size"], None)
        got = pool.allocate_slots(7, 0, case["tokens"])
        assert got is not None and len(got) == case["blocks"], (case, got)


def pin_head_of_queue(pool_cls=RefBlockPool):
    order = np.random.default_rng(5).permutation(40)
    pool = pool_cls(40, 16, order)
    a = pool.allocate_slots(1, 0, 40)  # 3 blocks
    assert list(a) == list(order[:3])
    b = pool.allocate_slots(2, 0, 17)  # 2 blocks, next in line
    assert list(b) == list(order[3:5])
    # growing a request only takes the difference
    c = pool.allocate_slots(1, 40, 9)  # ceil(49/16)=4 -> 1 more
    assert list(c) == [order[5]]
    assert pool.num_free == 34
    assert pool.blocks(1) == list(order[:3]) + [order[5]]


def pin_exhaustion(pool_cls=RefBlockPool):
    order = np.arange(6)[::-1].copy()
    pool = pool_cls(6, 16, order)
    assert pool.allocate_slots(1, 0, 64) is not None  # 4 blocks
    before = pool.num_free
    assert pool.allocate_slots(2, 0, 48) is None  # needs 3, only 2 left
    assert pool.num_free == before and pool.blocks(2) == []
    assert pool.allocate_slots(2, 0, 32) is not None


def pin_fifo_release(pool_cls=RefBlockPool):
    order = np.arange(8)
    pool = pool_cls(8, 16, order)
    pool.allocate_slots(1, 0, 32)  # [0, 1]
    pool.allocate_slots(2, 0, 32)  # [2, 3]
    pool.free(1)  # 0, 1 go to the tail: queue 4 5 6 7 0 1
    got = pool.allocate_slots(3, 0, 96)  # 6 blocks
    assert list(got) == [4, 5, 6, 7, 0, 1]


def pin_refcount(pool_cls=RefBlockPool):
    pool = pool_cls(10, 16, np.arange(10))
    pool.allocate_slots(-1, 0, 32)  # prefix owner: [0, 1]
    pref = pool.blocks(-1)
    for r in (1, 2, 3):
        pool.share_prefix(r, pref)
        pool.allocate_slots(r, 32, 1)  # one private block each
    pool.free(-1)
    assert pool.num_free == 10 - 2 - 3
    pool.free(1)
    pool.free(2)
    assert pool.num_free == 10 - 2 - 1  # prefix still held by request 3
    pool.free(3)
    assert pool.num_free == 10


def pin_tiny_allocation(pool_cls=RefBlockPool):
    g = golden("tiny_fp32_allocation.json")
    spec = W.make_config(1)
    pool = pool_cls(spec.num_blocks, spec.block_size, spec.initial_order)
    meta = W.run_allocation_script(spec, pool)
    assert meta.seq_lens.tolist() == g["seq_lens"]
    assert meta.context_lens.tolist() == g["context_lens"]
    assert meta.query_start_loc.tolist() == g["query_start_loc"]
    for i, pos in enumerate(g["queue_positions"]):
        nblk = g["blocks_per_seq"][i]
        assert meta.block_tables[i, :nblk].tolist() == [int(spec.initial_order[p]) for p in pos]
    assert pool.num_free == g["free_after"]


# --------------------------------------------------------------------------- layout pins
def pin_cache_layout(scatter_fn, gather_fn):
    g = golden("cache_layout.json")
    nb, hkv, bs, d = g["num_blocks"], g["num_kv_heads"], g["block_size"], g["head_dim"]
    T = nb * bs
    # token n carries the value n*1000 + head*10 + dim, stored at slot = n
    k = np.array([[[n * 1000 + h * 10 + dd for dd in range(d)] for h in range(hkv)] for n in range(T)],
                 dtype=np.uint32)
    cache = np.zeros((nb, hkv, bs, d), dtype=np.uint32)
    kc, _ = scatter_fn(k, k, np.arange(T, dtype=np.int32), cache, cache, bs)
    flat = kc.reshape(-1)
    for e in g["entries"]:
        assert flat[e["flat"]] == e["slot"] * 1000 + e["head"] * 10 + e["dim"], e
    # gather with the identity table reads the tokens back in order
    seq = gather_fn(kc, list(range(nb)), T, bs)
    assert np.array_equal(seq, k)
    # a negative slot stores nothing
    kc2, _ = scatter_fn(k[:2], k[:2], np.array([-1, 5], dtype=np.int32), cache, cache, bs)
    assert kc2.sum() == k[1].sum() and np.array_equal(kc2[0, :, 5, :], k[1])


def pin_scatter_gather_dense(spec, scatter_fn, gather_fn):
    """Writing each sequence's tokens through the pool's slots and gathering them back
    through the block table gives the sequence's contiguous K history."""
    st = build_oracle_step(spec)
    kc, vc = scatter_fn(st.k_new, st.v_new, st.meta.slot_mapping, st.k_cache_pre, st.v_cache_pre,
                        spec.block_size)
    for i, r in enumerate(spec.requests):
        ks = gather_fn(kc, st.meta.block_tables[i], r.seq_len, spec.block_size)
        vs = gather_fn(vc, st.meta.block_tables[i], r.seq_len, spec.block_size)
        assert np.array_equal(ks, st.k_full[i]) and np.array_equal(vs, st.v_full[i]), i


# --------------------------------------------------------------------------- attention pins
def _paged_out(spec, attn_fn, gather_fn, scatter_fn, order=None):
    if order is not None:
        spec.initial_order = order
    st = build_oracle_step(spec)
    kc, vc = scatter_fn(st.k_new, st.v_new, st.meta.slot_mapping, st.k_cache_pre, st.v_cache_pre,
                        spec.block_size)
    kc, vc, q = st.f64(kc), st.f64(vc), st.f64(st.q)
    out = np.zeros(q.shape)
    m = st.meta
    for i, r in enumerate(spec.requests):
        r0, r1 = m.query_start_loc[i], m.query_start_loc[i + 1]
        if r1 == r0:
            continue
        K = gather_fn(kc, m.block_tables[i], r.seq_len, spec.block_size)
        V = gather_fn(vc, m.block_tables[i], r.seq_len, spec.block_size)
        out[r0:r1] = attn_fn(q[r0:r1], K, V, r.context + np.arange(r1 - r0), spec.scale)
    return out, st


def pin_bruteforce(attn_fn, gather_fn, scatter_fn, seeds=(0, 1, 2)):
    specs = [W.make_config(1)] + [W.random_spec(s, num_seqs=3, max_context=20, max_query=4,
                                                num_q_heads=4, num_kv_heads=2, head_dim=8)
                                  for s in seeds]
    for spec in specs:
        out, st = _paged_out(spec, attn_fn, gather_fn, scatter_fn)
        q = st.f64(st.q)
        q_seq, q_pos, toks = [], [], []
        for i, r in enumerate(spec.requests):
            for j in range(r.query):
                q_seq.append(i)
                q_pos.append(r.context + j)
            kf, vf = st.f64(st.k_full[i]), st.f64(st.v_full[i])
            for t in range(r.seq_len):
                toks.append((i, t, kf[t].tolist(), vf[t].tolist()))
        bf = np.array(ref_bruteforce(q.tolist(), q_seq, q_pos, toks, spec.scale,
                                     spec.num_q_heads, spec.num_kv_heads))
        assert np.abs(bf - out).max() <= 1e-12, (spec.name, np.abs(bf - out).max())


def pin_sdpa(attn_fn, seeds=(0, 1, 2, 3)):
    """Equal to torch's CPU attention routine in float64 with an explicit boolean mask."""
    for s in seeds:
        r = np.random.default_rng(100 + s)
        hkv = int(r.choice([1, 2, 4]))
        g = int(r.choice([1, 2, 4]))
        hq, d = hkv * g, int(r.choice([8, 16, 64]))
        L = int(r.integers(1, 70))
        n = int(r.integers(1, L + 1))
        c = L - n
        q, K, V = rng_qkv(200 + s, n, L, hq, hkv, d)
        scale = float(r.uniform(0.05, 0.5))
        out = attn_fn(q, K, V, c + np.arange(n), scale)
        qt = torch.from_numpy(q).permute(1, 0, 2)  # [hq, n, d]
        Kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(g, dim=0).contiguous()
        Vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(g, dim=0).contiguous()
        mask = torch.from_numpy(np.arange(L)[None, :] <= (c + np.arange(n))[:, None])
        ref = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, attn_mask=mask, scale=scale)
        assert np.abs(ref.permute(1, 0, 2).numpy() - out).max() <= 1e-12


def pin_closed_forms(attn_fn):
    r = np.random.default_rng(7)
    # one visible key: the output is that key's value row, exactly
    q, K, V = rng_qkv(1, 1, 1, 4, 2, 16)
    out = attn_fn(q, K, V, [0], 0.3)
    for h in range(4):
        assert np.array_equal(out[0, h], V[0, h // 2])
    # all keys equal: every visible value weighs the same, out = mean of visible V rows
    L = 9
    q, _, V = rng_qkv(2, 3, L, 2, 1, 8)
    K = np.tile(r.standard_normal((1, 1, 8)), (L, 1, 1))
    pos = [2, 5, 8]
    out = attn_fn(q, K, V, pos, 0.7)
    for j, p in enumerate(pos):
        assert np.allclose(out[j, 0], V[: p + 1, 0].mean(axis=0), rtol=0, atol=1e-14)
    # scale 0: same thing with arbitrary keys
    q, K, V = rng_qkv(3, 2, 6, 2, 2, 8)
    out = attn_fn(q, K, V, [3, 5], 0.0)
    assert np.allclose(out[0, 1], V[:4, 1].mean(axis=0), atol=1e-14)
    assert np.allclose(out[1, 0], V[:6, 0].mean(axis=0), atol=1e-14)
    # two keys: softmax of two scores in closed form
    q = np.zeros((1, 1, 2)); q[0, 0] = [1.0, 0.0]
    K = np.array([[[2.0, 5.0]], [[0.0, -1.0]]])
    V = np.array([[[1.0, 0.0]], [[0.0, 1.0]]])
    out = attn_fn(q, K, V, [1], 0.5)  # scores 1.0 and 0.0
    w0 = math.exp(1.0) / (math.exp(1.0) + 1.0)
    assert abs(out[0, 0, 0] - w0) < 1e-15 and abs(out[0, 0, 1] - (1 - w0)) < 1e-15
    # grouped heads equal plain multi-head attention on repeat-interleaved K/V
    q, K, V = rng_qkv(4, 5, 12, 8, 2, 16)
    pos = np.arange(7, 12)
    a = attn_fn(q, K, V, pos, 0.25)
    b = attn_fn(q, np.repeat(K, 4, axis=1), np.repeat(V, 4, axis=1), pos, 0.25)
    assert np.abs(a - b).max() <= 1e-14


def pin_decode_is_last_prefill_row(attn_fn):
    """A decode at context t equals the last row of a fresh prefill over t+1 tokens."""
    q, K, V = rng_qkv(11, 20, 20, 4, 2, 32)
    full = attn_fn(q, K, V, np.arange(20), 0.2)
    for t in (0, 7, 19):
        dec = attn_fn(q[t:t + 1], K[: t + 1], V[: t + 1], [t], 0.2)
        assert np.abs(dec - full[t:t + 1]).max() <= 1e-14


def pin_chunked_equals_full(attn_fn):
    """A chunk over cached context c equals rows c..c+q-1 of a full prefill over c+q tokens."""
    q, K, V = rng_qkv(12, 40, 40, 4, 4, 16)
    full = attn_fn(q, K, V, np.arange(40), 0.3)
    for c, n in ((0, 13), (13, 16), (29, 11)):
        ch = attn_fn(q[c:c + n], K[: c + n], V[: c + n], c + np.arange(n), 0.3)
        assert np.abs(ch - full[c:c + n]).max() <= 1e-14


def pin_permutation_invariance(attn_fn, gather_fn, scatter_fn):
    """Another initial order of the free queue gives other physical blocks, same outputs."""
    mk = lambda: W.random_spec(5, num_seqs=4, max_context=50, max_query=5, head_dim=16, spare_blocks=6)
    a, st_a = _paged_out(mk(), attn_fn, gather_fn, scatter_fn)
    other = np.random.default_rng(99).permutation(mk().num_blocks).astype(np.int32)
    b, st_b = _paged_out(mk(), attn_fn, gather_fn, scatter_fn, order=other)
    assert not np.array_equal(st_a.meta.block_tables, st_b.meta.block_tables)
    assert np.abs(a - b).max() <= 1e-12


def pin_isolation(attn_fn, gather_fn, scatter_fn):
    """Changing other sequences' Q and K/V leaves a sequence's rows unchanged."""
    spec = W.random_spec(6, num_seqs=4, max_context=30, max_query=4, head_dim=16)
    st = build_oracle_step(spec)
    kc, vc = scatter_fn(st.k_new, st.v_new, st.meta.slot_mapping, st.k_cache_pre, st.v_cache_pre, 16)
    kc, vc, q = st.f64(kc), st.f64(vc), st.f64(st.q)
    m = st.meta

    def run(kc, vc, q):
        out = np.zeros(q.shape)
        for i, r in enumerate(spec.requests):
            r0, r1 = m.query_start_loc[i], m.query_start_loc[i + 1]
            K = gather_fn(kc, m.block_tables[i], r.seq_len, 16)
            V = gather_fn(vc, m.block_tables[i], r.seq_len, 16)
            out[r0:r1] = attn_fn(q[r0:r1], K, V, r.context + np.arange(r1 - r0), spec.scale)
        return out

    base = run(kc, vc, q)
    keep = 1
    own = set(m.block_tables[keep][: spec.blocks_of(spec.requests[keep])].tolist())
    kc2, vc2, q2 = kc.copy(), vc.copy(), q.copy()
    for b in range(spec.num_blocks):
        if b not in own:
            kc2[b] = np.random.default_rng(b).standard_normal(kc2[b].shape) * 5
            vc2[b] = np.random.default_rng(b + 1000).standard_normal(vc2[b].shape) * 5
    r0, r1 = m.query_start_loc[keep], m.query_start_loc[keep + 1]
    q2[:r0] += 3.0
    q2[r1:] -= 2.0
    pert = run(kc2, vc2, q2)
    assert np.array_equal(pert[r0:r1], base[r0:r1])
    assert not np.allclose(pert[:r0], base[:r0]) or r0 == 0


def pin_prefix_sharing(attn_fn, gather_fn, scatter_fn):
    """Requests reading a shared, ref-counted prefix get the same output as with private copies."""
    spec = W.random_spec(7, num_seqs=5, max_context=60, max_query=3, head_dim=16, prefix_tokens=32)
    shared, st = _paged_out(spec, attn_fn, gather_fn, scatter_fn)
    assert any(r.shares_prefix for r in spec.requests)
    # private copies: each request's contiguous history holds its own copy of the prefix
    outs = []
    for i, r in enumerate(spec.requests):
        q = st.f64(st.q)[st.meta.query_start_loc[i]:st.meta.query_start_loc[i + 1]]
        outs.append(attn_fn(q, st.f64(st.k_full[i]), st.f64(st.v_full[i]),
                            r.context + np.arange(r.query), spec.scale))
    dense = np.concatenate(outs)
    assert np.abs(dense - shared).max() <= 1e-12
    # and the shared blocks really are shared
    pref_blocks = [tuple(st.meta.block_tables[i][:2]) for i, r in enumerate(spec.requests) if r.shares_prefix]
    assert len(set(pref_blocks)) == 1


def pin_order(attn_fn, gather_fn, scatter_fn):
    """Permuting the sequences of the super-sequence permutes the output rows alike."""
    spec = W.random_spec(8, num_seqs=5, max_context=25, max_query=4, head_dim=16)
    a, st = _paged_out(spec, attn_fn, gather_fn, scatter_fn)
    perm = [3, 0, 4, 2, 1]
    spec2 = W.random_spec(8, num_seqs=5, max_context=25, max_query=4, head_dim=16)
    spec2.requests = [spec2.requests[p] for p in perm]
    b, st2 = _paged_out(spec2, attn_fn, gather_fn, scatter_fn)
    qsl, qsl2 = st.meta.query_start_loc, st2.meta.query_start_loc
    for new_i, old_i in enumerate(perm):
        ra = a[qsl[old_i]:qsl[old_i + 1]]
        rb = b[qsl2[new_i]:qsl2[new_i + 1]]
        assert np.abs(ra - rb).max() <= 1e-12
