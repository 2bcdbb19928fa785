"""HIP path vs the fp64 oracle on the same seeded inputs (GPU).

Cache scatter: bit-exact, whole pool (poisoned background included).
Attention: max-abs error <= 1e-5 for float32 steps and <= 1e-2 for bf16 steps
(inputs bf16, fp32 accumulation), on every row of the small configurations and
on sampled sequences of the full-size ones, launched exactly as the bench does.
"""
import numpy as np
import pytest
import torch

import paged_kv_varlen_reshape_amd as pk
import workloads as W
from workloads.device import build_device_step
from device_data import oracle_rows
from oracle import ref_reshape_and_cache
from oracle_data import build_oracle_step

pytestmark = pytest.mark.gpu
TOL = {"f32": 1e-5, "bf16": 1e-2}


def _host_bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy().view(
        np.uint16 if t.dtype == torch.bfloat16 else np.uint32)


def _check_attention(spec, ds, out, seqs=None):
    torch.cuda.synchronize()
    assert torch.isfinite(out).all(), "non-finite output (over-read of a poisoned slot?)"
    seqs = range(spec.num_seqs) if seqs is None else seqs
    want, got = oracle_rows(spec, seqs, out, ds.meta)
    err = np.abs(want - got).max() if want.size else 0.0
    print(f"[{spec.name}] rows={want.shape[0]} max_abs_err={err:.3e}", flush=True)
    assert err <= TOL[spec.dtype], err
    return err


@pytest.fixture(autouse=True)
def _reset_options():
    yield
    pk.pa_set_option(pk.PA_OPT_FORCE_ROWWISE, 0)
    pk.pa_set_option(pk.PA_OPT_SPLIT_TOKENS, 0)
    pk.pa_set_option(pk.PA_OPT_TARGET_ITEMS, 0)
    pk.pa_set_option(pk.PA_OPT_DECODE_BUFFERS, 0)
    pk.pa_set_option(pk.PA_OPT_DECODE_KERNEL, 0)
    pk.pa_set_option(pk.PA_OPT_VERIFY_ROWS, 0)
    pk.pa_set_option(pk.PA_OPT_CHUNK_KERNEL, 0)


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_reshape_and_cache_bit_exact_whole_pool(cfg):
    spec = W.make_config(cfg)
    print(f"reshape parity cfg{cfg}", flush=True)
    ds = build_device_step(spec, pad_value=-1)
    ds.reshape()
    torch.cuda.synchronize()
    st = build_oracle_step(spec)
    kc, vc = ref_reshape_and_cache(st.k_new, st.v_new, st.meta.slot_mapping, st.k_cache_pre, st.v_cache_pre, 16)
    assert np.array_equal(st.meta.block_tables, ds.meta.block_tables)
    assert np.array_equal(_host_bits(ds.k_cache), kc)
    assert np.array_equal(_host_bits(ds.v_cache), vc)


def test_reshape_skips_negative_slots_and_empty_call():
    spec = W.random_spec(21, num_seqs=4, dtype="bf16", head_dim=128)
    ds = build_device_step(spec)
    before = _host_bits(ds.k_cache).copy()
    sm = ds.slot_mapping.clone()
    sm[::2] = -1
    pk.pa_reshape_and_cache(ds.k_new, ds.v_new, sm, ds.k_cache, ds.v_cache)
    torch.cuda.synchronize()
    st = build_oracle_step(spec)
    kc, _ = ref_reshape_and_cache(st.k_new, st.v_new, sm.cpu().numpy(), before, before, 16)
    assert np.array_equal(_host_bits(ds.k_cache), kc)
    pk.pa_reshape_and_cache(ds.k_new[:0], ds.v_new[:0], sm[:0], ds.k_cache, ds.v_cache)


@pytest.mark.parametrize("cfg", [1, 2, 3, 6])
def test_attention_matches_oracle_every_row(cfg):
    spec = W.make_config(cfg)
    print(f"attention parity cfg{cfg}", flush=True)
    ds = build_device_step(spec)
    ds.reshape()
    out = ds.attention()
    _check_attention(spec, ds, out)


@pytest.mark.parametrize("seed", range(12))
def test_attention_random_steps(seed):
    r = np.random.default_rng(seed)
    dtype = ["f32", "bf16"][seed % 2]
    hkv = int(r.choice([1, 2, 4]))
    g = int(r.choice([1, 2, 4, 8]))
    d = int(r.choice([64, 128]))
    spec = W.random_spec(seed, num_seqs=int(r.integers(1, 9)), max_context=int(r.integers(1, 300)),
                         max_query=int(r.integers(1, 40)), num_q_heads=hkv * g, num_kv_heads=hkv, head_dim=d,
                         dtype=dtype, prefix_tokens=int(r.choice([0, 16, 48])), decode_fraction=0.5)
    print(f"random step seed={seed} {dtype} hkv={hkv} g={g} d={d} seqs={spec.num_seqs}", flush=True)
    ds = build_device_step(spec)
    ds.reshape()
    for split in (0, 16, 48):
        pk.pa_set_option(pk.PA_OPT_SPLIT_TOKENS, split)
        out = ds.attention()
        _check_attention(spec, ds, out)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("g", [1, 2, 4, 8])
def test_chunk_kernel_long_items_every_group(d, g):
    """The MFMA chunk kernel on items of many key tiles: unmasked and masked
    tiles, the hand-over to the next item during an item's last tiles, zeroed V
    tails and mid-block chunk starts, for every GQA group size and head dim."""
    seed = 200 + 10 * (d // 64) + g
    spec = W.random_spec(seed, num_seqs=3, max_context=700, max_query=300, num_q_heads=2 * g, num_kv_heads=2,
                         head_dim=d, dtype="bf16", decode_fraction=0.0)
    print(f"chunk items seed={seed} d={d} g={g} (context, query)="
          f"{[(r.context, r.query) for r in spec.requests]}", flush=True)
    ds = build_device_step(spec)
    ds.reshape()
    _check_attention(spec, ds, ds.attention())


@pytest.mark.parametrize("case", ["ties sorted", "too many to sort", "all-chunk beyond 2048 sorted", "mixed sorted"])
def test_self_planned_chunk_orders(case):
    """Steps the chunk kernel plans by itself: tiles ranked longest first in
    LDS (equal tiles by index) and taken in zigzag rounds when the items take
    more than one round of the grid, or in sequence order when there are too
    many sequences to rank (or one round); every tile is computed exactly once
    either way."""
    import math
    if case == "ties sorted":            # 40 identical sequences: every key count tied 40 ways
        reqs = [W.Request(i, 100, 70) for i in range(40)]
    elif case == "too many to sort":     # 70 sequences > the ranking limit
        reqs = [W.Request(i, 13 * i, 8) for i in range(70)]
    elif case == "all-chunk beyond 2048 sorted":  # 4200 tokens, every sequence a chunk
        reqs = [W.Request(i, [0, 64, 500, 1000, 33, 700][i], 700) for i in range(6)]
    else:                                # chunks next to decodes, more items than one grid round
        reqs = [W.Request(i, 17 * i, 40 if i < 40 else 1) for i in range(60)]
    nb = sum(-(-r.seq_len // 16) for r in reqs) + 4
    seed = 2400 + len(reqs)
    order = np.random.default_rng(seed).permutation(nb).astype(np.int32)
    spec = W.StepSpec(f"self-plan {case}", seed, 32, 8, 128, "bf16", 16, nb, 1.0 / math.sqrt(128.0), reqs,
                      initial_order=order, table_rows=4096, seed=seed)
    print(f"self-planned chunk order: {case}, {len(reqs)} sequences, {sum(r.query for r in reqs)} tokens", flush=True)
    ds = build_device_step(spec)
    ds.reshape()
    _check_attention(spec, ds, ds.attention())


@pytest.mark.parametrize("hkv,g", [(8, 4), (16, 2)])
def test_chunk_kernel_xcd_queues(hkv, g):
    """Kv-head counts that split evenly over the per-XCD work queues (one or two
    kv heads per queue) on ragged multi-tile items: every (tile, kv head) item
    is taken exactly once."""
    seed = 300 + hkv
    spec = W.random_spec(seed, num_seqs=4, max_context=900, max_query=260, num_q_heads=hkv * g, num_kv_heads=hkv,
                         head_dim=128, dtype="bf16", decode_fraction=0.0)
    print(f"xcd queues seed={seed} hkv={hkv} g={g} (context, query)="
          f"{[(r.context, r.query) for r in spec.requests]}", flush=True)
    ds = build_device_step(spec)
    ds.reshape()
    _check_attention(spec, ds, ds.attention())


def test_chunk_and_decode_over_very_long_contexts():
    """A 200-row chunk over 40000 cached tokens (about 630 key tiles per item,
    with the next item claimed during its last tiles), a decode over 100000
    tokens cut into many ranges, and a short 5-row chunk, GQA 8:1 with one kv head."""
    reqs = [W.Request(0, 40000, 200), W.Request(1, 100000, 1), W.Request(2, 37, 5)]
    nb = sum(-(-r.seq_len // 16) for r in reqs) + 4
    order = np.random.default_rng((77, 0)).permutation(nb).astype(np.int32)
    spec = W.StepSpec("long-contexts", 77, 8, 1, 128, "bf16", 16, nb, 1.0 / np.sqrt(128.0), reqs,
                      initial_order=order, seed=77)
    ds = build_device_step(spec)
    ds.reshape()
    _check_attention(spec, ds, ds.attention())


@pytest.mark.parametrize("kernel,nbuf", [(1, 1), (1, 2), (2, 2), (2, 3), (2, 4)])
@pytest.mark.parametrize("seed", [100, 101, 102, 103])
def test_bf16_decode_kernels_match_oracle(seed, kernel, nbuf):
    """Both row-wise kernels for bf16 (VALU with one or two page buffers, MFMA with
    two to four),
    every group size, ranges both shorter and longer than a row."""
    r = np.random.default_rng(seed)
    hkv = [1, 2, 4, 2][seed % 4]
    g = [1, 2, 4, 8][seed % 4]
    d = [64, 128][(seed // 2) % 2]
    spec = W.random_spec(seed, num_seqs=int(r.integers(3, 9)), max_context=int(r.integers(40, 400)),
                         max_query=int(r.integers(2, 24)), num_q_heads=hkv * g, num_kv_heads=hkv, head_dim=d,
                         dtype="bf16", prefix_tokens=16, decode_fraction=0.6)
    print(f"bf16 decode kernel={kernel} nbuf={nbuf} seed={seed} hkv={hkv} g={g} d={d}", flush=True)
    ds = build_device_step(spec)
    ds.reshape()
    pk.pa_set_option(pk.PA_OPT_DECODE_KERNEL, kernel)
    pk.pa_set_option(pk.PA_OPT_DECODE_BUFFERS, nbuf)
    for rowwise in (0, 1):
        pk.pa_set_option(pk.PA_OPT_FORCE_ROWWISE, rowwise)
        for split in (0, 16, 80):
            pk.pa_set_option(pk.PA_OPT_SPLIT_TOKENS, split)
            _check_attention(spec, ds, ds.attention())


@pytest.mark.parametrize("seed", range(8))
def test_self_planned_decode_ranges(seed):
    """Decode-only bf16 steps small enough for the MFMA decode kernel to plan
    itself: contexts from 0 (one-page pairs) to a few thousand tokens, ranges from
    one page (every pair cut) to 512 pages (a range over many pairs, and over more
    than 64 pages of one pair), two to four pages in flight per wavefront, every
    group size and both head sizes."""
    import math
    r = np.random.default_rng((seed, 7))
    g = [1, 2, 4, 8][seed % 4]
    hkv = [2, 1][(seed // 4) % 2]
    d = [64, 128][(seed // 2) % 2]
    n = int(r.integers(20, 120))
    ctx = np.where(r.random(n) < 0.4, r.integers(0, 40, n), r.integers(40, 3000, n))
    reqs = [W.Request(i, int(c), 1) for i, c in enumerate(ctx)]
    nb = sum(-(-(int(c) + 1) // 16) for c in ctx) + 4
    order = np.random.default_rng((seed, 8)).permutation(nb).astype(np.int32)
    spec = W.StepSpec("self-planned decode", 3000 + seed, hkv * g, hkv, d, "bf16", 16, nb, 1.0 / math.sqrt(d),
                      reqs, initial_order=order, table_rows=2048, seed=3000 + seed)
    print(f"self-planned decode seed={seed} g={g} hkv={hkv} d={d} seqs={n}", flush=True)
    ds = build_device_step(spec)
    ds.reshape()
    assert ds.max_query_len == 1
    for nbuf in (2, 3, 4):  # pages in flight per wavefront
        pk.pa_set_option(pk.PA_OPT_DECODE_BUFFERS, nbuf)
        for split in (0, 16, 256, 1024, 8192):
            pk.pa_set_option(pk.PA_OPT_SPLIT_TOKENS, split)
            _check_attention(spec, ds, ds.attention())


def test_many_sequences_plan_fallbacks():
    """More sequences than the plan keeps in registers and more rows than its
    LDS range search holds: both fallback paths, checked on sampled sequences."""
    spec = W.random_spec(40, num_seqs=9000, max_context=70, max_query=3, num_q_heads=4, num_kv_heads=2,
                         head_dim=64, dtype="f32", decode_fraction=0.3)
    assert spec.num_tokens > 8192
    print(f"many sequences: {spec.num_seqs} seqs, {spec.num_tokens} rows", flush=True)
    ds = build_device_step(spec)
    ds.reshape()
    seqs = sorted(np.random.default_rng(40).choice(spec.num_seqs, 200, replace=False).tolist()) + [spec.num_seqs - 1]
    for split in (0, 16):
        pk.pa_set_option(pk.PA_OPT_SPLIT_TOKENS, split)
        _check_attention(spec, ds, ds.attention(), seqs)


@pytest.mark.parametrize("seed", range(8))
def test_short_queries_share_pages(seed):
    """Sequences with 2..16/G query rows as one row-wise record (their rows share every
    page, one MFMA column per row and head) against the oracle; with the grouping off
    (chunk kernel), capped at 3 rows, and with range lengths that cut the records."""
    r = np.random.default_rng(seed)
    g = [1, 2, 4, 8][seed % 4]
    hkv = [2, 1][(seed // 4) % 2]
    d = [64, 128][(seed // 2) % 2]
    spec = W.random_spec(200 + seed, num_seqs=int(r.integers(4, 12)), max_context=int(r.integers(20, 400)),
                         max_query=8, num_q_heads=hkv * g, num_kv_heads=hkv, head_dim=d, dtype="bf16",
                         prefix_tokens=16, decode_fraction=0.3)
    print(f"short queries seed={seed} g={g} hkv={hkv} d={d} q={[x.query for x in spec.requests]}", flush=True)
    ds = build_device_step(spec)
    ds.reshape()
    for vr in (16, 1, 3):  # the cap 16 / G, off (chunk kernel), at most 3 rows
        pk.pa_set_option(pk.PA_OPT_VERIFY_ROWS, vr)
        for split in (0, 16, 48):
            pk.pa_set_option(pk.PA_OPT_SPLIT_TOKENS, split)
            _check_attention(spec, ds, ds.attention())


@pytest.mark.parametrize("seed", range(8))
def test_self_planned_short_query_records(seed):
    """Small steps whose sequences all have at most 16 / G query rows (speculative-
    decoding verification), records on: the MFMA decode kernel plans the records by
    itself (no plan or chunk kernel) -- contexts from 0 to a few thousand tokens,
    every group size and head size, ranges that cut records.  Then the same step with
    a max_query_len hint below the longest sequences' rows: those become several
    records each (or, past the self-planned size, take the planned path)."""
    import math
    r = np.random.default_rng((seed, 11))
    g = [1, 2, 4, 8][seed % 4]
    hkv = [2, 1][(seed // 4) % 2]
    d = [64, 128][(seed // 2) % 2]
    cap = 16 // g
    for case in ("fits", "hint too low"):
        n = int(r.integers(8, 64))
        hi = cap if case == "fits" else 3 * cap
        n = min(n, 500 // hi)
        ctx = np.where(r.random(n) < 0.3, r.integers(0, 40, n), r.integers(40, 3000, n))
        qs = r.integers(1, hi + 1, n)
        if case == "hint too low":
            qs[0] = hi  # at least one sequence longer than the hint
        reqs = [W.Request(i, int(c), int(q)) for i, (c, q) in enumerate(zip(ctx, qs))]
        nb = sum(-(-(int(c) + int(q)) // 16) for c, q in zip(ctx, qs)) + 4
        order = np.random.default_rng((seed, 12)).permutation(nb).astype(np.int32)
        spec = W.StepSpec(f"short-query records {case}", 3100 + seed, hkv * g, hkv, d, "bf16", 16, nb,
                          1.0 / math.sqrt(d), reqs, initial_order=order, table_rows=2048, seed=3100 + seed)
        print(f"short-query records seed={seed} case={case} g={g} hkv={hkv} d={d} seqs={n} "
              f"tokens={spec.num_tokens} max_q={int(qs.max())}", flush=True)
        ds = build_device_step(spec)
        ds.reshape()
        # 0: automatic (records in the one-row workspace layout, fewer and longer
        # ranges); 16: on request (the cap, a workspace laid out for it)
        for vr in (0, 16):
            pk.pa_set_option(pk.PA_OPT_VERIFY_ROWS, vr)
            for split in (0, 16, 256):
                pk.pa_set_option(pk.PA_OPT_SPLIT_TOKENS, split)
                if case == "fits":
                    out = ds.attention()
                else:
                    out = pk.pa_attention(ds.q, ds.k_cache, ds.v_cache, ds.block_tables, ds.seq_lens,
                                          ds.query_start_loc, ds.context_lens, spec.scale, max_query_len=cap)
                _check_attention(spec, ds, out)


def test_short_query_configuration_as_records():
    """The short-query configuration (64 sequences x 4 query rows over contexts of
    512-2048, GQA 4:1) with records on, every row against the oracle."""
    spec = W.make_config(6)
    ds = build_device_step(spec)
    ds.reshape()
    pk.pa_set_option(pk.PA_OPT_VERIFY_ROWS, 4)
    _check_attention(spec, ds, ds.attention())


def test_max_query_len_hint_never_changes_results():
    """<= 1 sends every row to the row-wise kernel: exact for a decode step,
    within tolerance (other kernel) for a mixed step given a wrong hint; a hint
    with T = S * hint sends every row to the chunk kernel, right or wrong."""
    dec = build_device_step(W.make_config(2))
    dec.reshape()
    a = dec.attention().clone()
    b = pk.pa_attention(dec.q, dec.k_cache, dec.v_cache, dec.block_tables, dec.seq_lens, dec.query_start_loc,
                        dec.context_lens, dec.spec.scale, max_query_len=dec.q.shape[0])
    torch.cuda.synchronize()
    assert dec.max_query_len == 1 and torch.equal(a, b)
    spec = W.make_config(3)
    mix = build_device_step(spec)
    mix.reshape()
    assert mix.max_query_len > 1
    out = pk.pa_attention(mix.q, mix.k_cache, mix.v_cache, mix.block_tables, mix.seq_lens, mix.query_start_loc,
                          mix.context_lens, spec.scale, max_query_len=1)
    _check_attention(spec, mix, out)
    # T = S * hint sends every row to the chunk kernel; a wrong hint of that kind (a
    # one-row sequence next to longer ones) must still get every row computed
    import math
    for d, g in ((128, 4), (64, 8), (128, 1)):
        reqs = [W.Request(i, c, q) for i, (c, q) in enumerate([(40, 1), (300, 5), (0, 1), (17, 5), (1000, 3),
                                                                 (5, 3)])]
        nb = sum(-(-(r.context + r.query) // 16) for r in reqs) + 4
        order = np.random.default_rng(d + g).permutation(nb).astype(np.int32)
        sp = W.StepSpec("wrong hint", 4000 + d + g, 2 * g, 2, d, "bf16", 16, nb, 1.0 / math.sqrt(d), reqs,
                        initial_order=order, table_rows=2048, seed=4000 + d + g)
        ds = build_device_step(sp)
        ds.reshape()
        assert ds.q.shape[0] == 6 * 3 and ds.max_query_len == 5
        for hint in (3, 5):  # 3: every row to the chunk kernel (T = 6 * 3); 5: the usual routing
            out = pk.pa_attention(ds.q, ds.k_cache, ds.v_cache, ds.block_tables, ds.seq_lens, ds.query_start_loc,
                                  ds.context_lens, sp.scale, max_query_len=hint)
            _check_attention(sp, ds, out)


@pytest.mark.parametrize("kernel", [2, 1])
def test_forced_rowwise_every_split_matches_oracle(kernel):
    """Every row of the chunked-prefill step (8 chunks of 512 rows) routed
    row-wise, on the MFMA (2) and the VALU (1) row-wise kernel, with ranges of
    16, 256 and 4096 tokens' worth of pages and the automatic ranges: each
    output against the oracle on every row."""
    spec = W.make_config(3)
    ds = build_device_step(spec)
    ds.reshape()
    pk.pa_set_option(pk.PA_OPT_FORCE_ROWWISE, 1)
    pk.pa_set_option(pk.PA_OPT_DECODE_KERNEL, kernel)
    want = None
    for split in (0, 16, 256, 4096):
        pk.pa_set_option(pk.PA_OPT_SPLIT_TOKENS, split)
        out = ds.attention()
        torch.cuda.synchronize()
        assert torch.isfinite(out).all()
        if want is None:
            want, got = oracle_rows(spec, range(spec.num_seqs), out, ds.meta)
        else:
            got = out.double().cpu().numpy()
        err = float(np.abs(want - got).max())
        print(f"forced row-wise kernel={kernel} split={split} max_abs_err={err:.3e}", flush=True)
        assert err <= TOL[spec.dtype], (split, err)


def test_deterministic_bitwise():
    spec = W.make_config(2)
    ds = build_device_step(spec)
    ds.reshape()
    a = ds.attention().clone()
    b = ds.attention().clone()
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_block_permutation_invariance_on_gpu():
    spec = W.make_config(2)
    a = build_device_step(spec)
    a.reshape()
    oa = a.attention().clone()
    spec2 = W.make_config(2)
    spec2.initial_order = np.random.default_rng(77).permutation(spec2.num_blocks).astype(np.int32)
    b = build_device_step(spec2)
    b.reshape()
    ob = b.attention()
    torch.cuda.synchronize()
    assert not np.array_equal(a.meta.block_tables, b.meta.block_tables)
    assert torch.equal(oa, ob)  # same work decomposition, only addresses differ


def test_sequences_without_query_rows_and_padding():
    spec = W.random_spec(30, num_seqs=6, dtype="bf16", head_dim=128, num_q_heads=8, num_kv_heads=2)
    spec.requests[1].query = 0
    spec.requests[4].query = 0
    ds = build_device_step(spec, pad_value=-1)
    ds.reshape()
    out = ds.attention()
    _check_attention(spec, ds, out)


def test_empty_step_is_a_no_op():
    spec = W.random_spec(31, num_seqs=2, dtype="bf16", head_dim=128, num_q_heads=8, num_kv_heads=2)
    ds = build_device_step(spec)
    out = torch.full((0, 8, 128), 0.0, device="cuda")
    pk.pa_attention(ds.q[:0], ds.k_cache, ds.v_cache, ds.block_tables, ds.seq_lens[:0], ds.query_start_loc[:1],
                    ds.context_lens[:0], 0.1, out=out)
    torch.cuda.synchronize()


@pytest.mark.slow
@pytest.mark.parametrize("cfg", [4, 5])
def test_full_size_configs_sampled(cfg):
    """The full-size mixed (4) and long-context prefix-shared (5) steps, launched as
    the bench launches them.  Attention against the oracle on the sampled subsets:
    all 4 chunks and 256 decodes of the mixed step; 32 prefix-sharing decodes and
    2 of the 16 long ones of the long-context step.  The scatter: K and V of every
    slot the step writes equal the step's new rows, bit for bit."""
    spec = W.make_config(cfg)
    print(f"full-size cfg{cfg}: building {spec.num_blocks} blocks", flush=True)
    ds = build_device_step(spec)
    ds.reshape()
    out = ds.attention()
    torch.cuda.synchronize()
    rng = np.random.default_rng(cfg)
    if cfg == 4:
        seqs = list(range(4)) + sorted(rng.choice(np.arange(4, spec.num_seqs), 256, replace=False).tolist())
    else:
        seqs = (sorted(rng.choice(256, 32, replace=False).tolist())
                + sorted((256 + rng.choice(16, 2, replace=False)).tolist()))
    print(f"full-size cfg{cfg}: oracle on {len(seqs)} sequences", flush=True)
    _check_attention(spec, ds, out, seqs)
    # scatter of this step: every written slot holds the step's row, bit for bit
    sm = ds.meta.slot_mapping.astype(np.int64)
    assert (sm >= 0).all() and np.unique(sm).size == sm.size
    blk, off = torch.from_numpy(sm // 16).cuda(), torch.from_numpy(sm % 16).cuda()
    for cache, new in ((ds.k_cache, ds.k_new), (ds.v_cache, ds.v_new)):
        got = cache[blk, :, off, :]
        assert torch.equal(got.view(torch.int16), new.view(torch.int16))
    del ds
    torch.cuda.empty_cache()


@pytest.mark.parametrize("block", range(4))
def test_random_steps_under_random_options(block):
    """Seeded random steps (1-600 sequences, contexts up to 3000, queries up to
    300 rows, decode fractions 0-1, shared prefixes, every group size, kv-head
    count and head size, bf16 and fp32) under random option combinations
    (records automatic / off / on request, the eight-wavefront chunk kernel,
    split lengths, forced row-wise, the VALU decode kernel) and max_query_len
    hints that are right or wrong: sampled sequences against the oracle."""
    for c in range(10):
        seed = 9000 + 10 * block + c
        r = np.random.default_rng(seed)
        g = int(r.choice([1, 2, 4, 8]))
        hkv = int(r.choice([1, 2, 4, 8]))
        d = int(r.choice([64, 128]))
        dtype = "bf16" if r.random() < 0.8 else "f32"
        n = int(r.choice([1, 3, 17, 64, 200, 600]))
        spec = W.random_spec(seed, num_seqs=n, max_context=int(r.choice([1, 30, 300, 3000])),
                             max_query=int(r.choice([1, 2, 4, 9, 40, 300])), num_q_heads=hkv * g,
                             num_kv_heads=hkv, head_dim=d, dtype=dtype, prefix_tokens=int(r.choice([0, 16, 48])),
                             decode_fraction=float(r.choice([0.0, 0.5, 0.9, 1.0])))
        opts = {pk.PA_OPT_VERIFY_ROWS: int(r.choice([0, 0, 1, 16])), pk.PA_OPT_CHUNK_KERNEL: int(r.choice([0, 0, 0, 2])),
                pk.PA_OPT_SPLIT_TOKENS: int(r.choice([0, 0, 16, 48])), pk.PA_OPT_FORCE_ROWWISE: int(r.random() < 0.1),
                pk.PA_OPT_DECODE_KERNEL: int(r.random() < 0.15)}
        for k, v in opts.items():
            pk.pa_set_option(k, v)
        ds = build_device_step(spec)
        ds.reshape()
        hint = ds.max_query_len if r.random() < 0.8 else int(r.choice([1, 2, 4, spec.num_tokens]))
        print(f"random step seed={seed} {dtype} g={g} hkv={hkv} d={d} seqs={n} tokens={spec.num_tokens} "
              f"hint={hint} options={list(opts.values())}", flush=True)
        out = pk.pa_attention(ds.q, ds.k_cache, ds.v_cache, ds.block_tables, ds.seq_lens, ds.query_start_loc,
                              ds.context_lens, spec.scale, max_query_len=hint)
        seqs = sorted(r.choice(spec.num_seqs, min(spec.num_seqs, 24), replace=False).tolist())
        _check_attention(spec, ds, out, seqs)
        for k in opts:
            pk.pa_set_option(k, 0)
        del ds, out
        torch.cuda.empty_cache()
