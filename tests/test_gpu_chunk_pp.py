"""The eight-wavefront chunk kernel (chunk_pp) against the fp64 oracle (GPU).

chunk_pp computes the same rows as the four-wavefront chunk kernel: causal
attention of each chunk row over its own sequence's keys 0..c+j, read through
the block table (Inside vLLM summary, techfeed.io, section "PagedAttentionの仕組み";
chunked prefill over cached tokens, section "高度な機能群").  Its items are 256
query rows long and its two wavefront groups alternate products and softmax,
so these cases reach what is particular to it: items of many key tiles with
the hand-over to the next item, the first step (no P.V) and the last (no S),
tiles of odd and even parity, masked diagonal tiles, zeroed V tails, chunk
starts in the middle of a page, every head size and group size, the per-XCD
queues, and a wrong block id clamped and flagged.  PA_OPT_CHUNK_KERNEL = 2
sends every step with chunk rows to it (the plan kernel plans them).
"""
import math

import numpy as np
import pytest
import torch

import paged_kv_varlen_reshape_amd as pk
import workloads as W
from workloads.device import build_device_step
from device_data import oracle_rows

pytestmark = pytest.mark.gpu
TOL = 1e-2  # bf16 inputs, fp32 accumulation


@pytest.fixture(autouse=True)
def _chunk_pp():
    pk.pa_set_option(pk.PA_OPT_CHUNK_KERNEL, 2)
    pk.pa_set_option(pk.PA_OPT_VERIFY_ROWS, 1)  # short queries stay chunk rows too
    yield
    pk.pa_set_option(pk.PA_OPT_CHUNK_KERNEL, 0)
    pk.pa_set_option(pk.PA_OPT_VERIFY_ROWS, 0)
    pk.pa_set_option(pk.PA_OPT_SPLIT_TOKENS, 0)


def _check(spec, ds, out, seqs=None):
    torch.cuda.synchronize()
    assert torch.isfinite(out).all(), "non-finite output"
    seqs = range(spec.num_seqs) if seqs is None else seqs
    want, got = oracle_rows(spec, seqs, out, ds.meta)
    err = float(np.abs(want - got).max()) if want.size else 0.0
    print(f"[{spec.name}] rows={want.shape[0]} max_abs_err={err:.3e}", flush=True)
    assert err <= TOL, err
    return err


def _spec(name, reqs, hkv, g, d, seed, scale=None):
    nb = sum(-(-r.seq_len // 16) for r in reqs) + 4
    order = np.random.default_rng((seed, 0)).permutation(nb).astype(np.int32)
    return W.StepSpec(name, seed, hkv * g, hkv, d, "bf16", 16, nb, 1.0 / math.sqrt(d) if scale is None else scale,
                      reqs, initial_order=order, table_rows=4096, seed=seed)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("g", [1, 2, 4, 8])
def test_long_items_every_group(d, g):
    """Random chunks of up to 300 rows over up to 700 cached tokens: items of
    one to a dozen key tiles, ragged last items, every group size and head dim."""
    seed = 1200 + 10 * (d // 64) + g
    spec = W.random_spec(seed, num_seqs=3, max_context=700, max_query=300, num_q_heads=2 * g, num_kv_heads=2,
                         head_dim=d, dtype="bf16", decode_fraction=0.0)
    print(f"chunk_pp items seed={seed} d={d} g={g} (context, query)="
          f"{[(r.context, r.query) for r in spec.requests]}", flush=True)
    ds = build_device_step(spec)
    ds.reshape()
    _check(spec, ds, ds.attention())


@pytest.mark.parametrize("reqs", [
    [(0, 1), (0, 64), (0, 65), (15, 1), (16, 63)],        # one key tile, no P.V before the last step
    [(0, 256), (64, 256), (1, 255), (127, 129)],          # whole items, items ending mid-tile
    [(17, 300), (3000, 40), (5, 513)],                    # odd/even tile counts, long masked-free runs
])
def test_item_boundaries(reqs):
    """Chosen (context, query) pairs for the first and last steps of an item,
    both buffer parities and mid-page starts (group size 4, 256/4 = 64 tokens
    per item)."""
    rq = [W.Request(i, c, q) for i, (c, q) in enumerate(reqs)]
    spec = _spec("chunk_pp boundaries", rq, 2, 4, 128, 1300 + sum(c + q for c, q in reqs))
    print(f"chunk_pp boundaries {reqs}", flush=True)
    ds = build_device_step(spec)
    ds.reshape()
    _check(spec, ds, ds.attention())


@pytest.mark.parametrize("hkv,g", [(8, 4), (16, 2), (8, 8)])
def test_xcd_queues(hkv, g):
    """Kv-head counts that split over the per-XCD queues, ragged multi-tile items:
    every (tile, kv head) item is taken exactly once."""
    seed = 1400 + hkv + g
    spec = W.random_spec(seed, num_seqs=4, max_context=900, max_query=600, num_q_heads=hkv * g,
                         num_kv_heads=hkv, head_dim=128, dtype="bf16", decode_fraction=0.0)
    print(f"chunk_pp xcd queues seed={seed} hkv={hkv} g={g} (context, query)="
          f"{[(r.context, r.query) for r in spec.requests]}", flush=True)
    ds = build_device_step(spec)
    ds.reshape()
    _check(spec, ds, ds.attention())


@pytest.mark.parametrize("seed", range(6))
def test_mixed_steps_with_decodes(seed):
    """Chunks next to decodes: chunk_pp takes the chunk rows, the row-wise
    kernel the rest, under several decode range lengths."""
    r = np.random.default_rng(1500 + seed)
    hkv = int(r.choice([1, 2, 4]))
    g = int(r.choice([1, 2, 4, 8]))
    d = int(r.choice([64, 128]))
    spec = W.random_spec(1500 + seed, num_seqs=int(r.integers(2, 9)), max_context=int(r.integers(1, 600)),
                         max_query=int(r.integers(2, 200)), num_q_heads=hkv * g, num_kv_heads=hkv, head_dim=d,
                         dtype="bf16", prefix_tokens=int(r.choice([0, 16, 48])), decode_fraction=0.5)
    print(f"chunk_pp mixed seed={seed} hkv={hkv} g={g} d={d} seqs={spec.num_seqs}", flush=True)
    ds = build_device_step(spec)
    ds.reshape()
    for split in (0, 48):
        pk.pa_set_option(pk.PA_OPT_SPLIT_TOKENS, split)
        _check(spec, ds, ds.attention())


@pytest.mark.parametrize("cfg", [3, 6])
def test_configurations(cfg):
    """The chunked-prefill configuration (8 chunks of 512 over 0..1536 cached
    tokens) and the short-query one (64 x 4 rows) on chunk_pp, every row."""
    spec = W.make_config(cfg)
    print(f"chunk_pp configuration {cfg}", flush=True)
    ds = build_device_step(spec)
    ds.reshape()
    _check(spec, ds, ds.attention())


def test_very_long_context():
    """A 200-row chunk over 40000 cached tokens (about 630 key tiles per item)
    next to a decode over 100000 tokens and a 5-row chunk, GQA 8:1."""
    reqs = [W.Request(0, 40000, 200), W.Request(1, 100000, 1), W.Request(2, 37, 5)]
    spec = _spec("chunk_pp long", reqs, 1, 8, 128, 1600)
    ds = build_device_step(spec)
    ds.reshape()
    _check(spec, ds, ds.attention())


@pytest.mark.parametrize("scale", [0.0, -0.0883883, 8.0])
def test_scales(scale):
    """Zero, negative and large scales (the sign or the zero folded into Q, the
    positive factor applied to the raw maxima): every weight of a row equal at
    scale 0, reversed order at a negative scale, one-hot-like at 8."""
    reqs = [W.Request(0, 0, 150), W.Request(1, 200, 77), W.Request(2, 5, 300), W.Request(3, 90, 1)]
    spec = _spec("chunk_pp scales", reqs, 2, 4, 128, 1700, scale=scale)
    ds = build_device_step(spec)
    ds.reshape()
    _check(spec, ds, ds.attention())


def test_repeat_is_bitwise_identical():
    """The same step twice gives the same bits (the queue order may differ, the
    arithmetic of each row does not)."""
    spec = W.make_config(3)
    ds = build_device_step(spec)
    ds.reshape()
    a = ds.attention().clone()
    b = ds.attention()
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_out_of_pool_block_id_is_clamped_and_flagged():
    """A block-table entry past the pool is read as the last block (no access
    outside the pool) and sets PA_FLAG_BLOCK_ID; a clean step leaves it clear."""
    reqs = [W.Request(0, 100, 300), W.Request(1, 40, 70)]
    spec = _spec("chunk_pp flags", reqs, 2, 4, 128, 1800)
    ds = build_device_step(spec)
    ds.reshape()
    ws = ds.workspace()
    pk.pa_attention_flags(ws, clear=True)
    ds.attention(workspace=ws)
    assert pk.pa_attention_flags(ws, clear=True) == 0
    bt = ds.block_tables.clone()
    bt[0, 3] = spec.num_blocks + 5
    pk.pa_attention(ds.q, ds.k_cache, ds.v_cache, bt, ds.seq_lens, ds.query_start_loc, ds.context_lens, spec.scale,
                    workspace=ws, max_query_len=ds.max_query_len)
    flags = pk.pa_attention_flags(ws, clear=True)
    print(f"chunk_pp flags after a bad block id: {flags}", flush=True)
    assert flags & pk.PA_FLAG_BLOCK_ID
