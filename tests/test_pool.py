"""The C++ block allocator against the pages' procedure and the oracle pool,
block for block, plus the host metadata validator (CPU only)."""
import numpy as np
import pytest

import paged_kv_varlen_reshape_amd as pk
import pins
import workloads as W
from oracle import RefBlockPool


@pytest.mark.parametrize("pin", [pins.pin_block_count, pins.pin_head_of_queue, pins.pin_exhaustion,
                                 pins.pin_fifo_release, pins.pin_refcount, pins.pin_tiny_allocation])
def test_cpp_pool_meets_the_pins(pin):
    pin(pk.BlockPool)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5, 6])
def test_cpp_pool_equals_reference_on_configs(cfg):
    spec = W.make_config(cfg)
    a, b = pk.BlockPool(spec.num_blocks, 16, spec.initial_order), RefBlockPool(spec.num_blocks, 16, spec.initial_order)
    ma, mb = W.run_allocation_script(spec, a), W.run_allocation_script(spec, b)
    assert np.array_equal(ma.block_tables, mb.block_tables)
    assert np.array_equal(ma.slot_mapping, mb.slot_mapping)
    assert a.num_free == b.num_free
    if cfg in (4, 5):
        assert a.num_free == 0  # pool sized to fit exactly
    if cfg == 5:
        shared = ma.block_tables[0][:128]
        assert all(a.refcount(int(x)) == 256 for x in shared)
        assert all(np.array_equal(ma.block_tables[i][:128], shared) for i in range(256))


def test_cpp_pool_random_ops_match_reference():
    rng = np.random.default_rng(3)
    nb = 200
    order = rng.permutation(nb)
    a, b = pk.BlockPool(nb, 16, order), RefBlockPool(nb, 16, order)
    held = {}
    for step in range(3000):
        op = rng.integers(0, 10)
        req = int(rng.integers(0, 25))
        if op < 6:
            done = held.get(req, 0)
            new = int(rng.integers(0, 40))
            ra, rb = a.allocate_slots(req, done, new), b.allocate_slots(req, done, new)
            assert ra == rb
            if ra is not None:
                held[req] = done + new
        elif op < 8:
            a.free(req)
            b.free(req)
            held.pop(req, None)
        else:
            src = int(rng.integers(0, 25))
            if req not in held and src in held and src != req:
                ids = b.blocks(src)[:2]
                a.share_prefix(req, ids)
                b.share_prefix(req, ids)
                held[req] = 16 * len(ids)
        assert a.num_free == b.num_free
        for r in range(25):
            assert a.blocks(r) == b.blocks(r)


def test_pool_rejects_bad_arguments():
    with pytest.raises(pk.PAError):
        pk.BlockPool(4, 16, [0, 1, 1, 2])
    with pytest.raises(pk.PAError):
        pk.BlockPool(0)
    p = pk.BlockPool(4)
    with pytest.raises(pk.PAError):
        p.share_prefix(1, [3])  # not allocated
    with pytest.raises(pk.PAError):
        p.slot_mapping(1, 0, 1)  # no block
    p.allocate_slots(1, 0, 20)
    with pytest.raises(pk.PAError):
        p.block_table_row(1, 1)
    assert p.allocate_slots(2, 0, 100) is None and p.num_free == 2


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_validator_accepts_configs(cfg):
    spec = W.make_config(cfg)
    m = W.run_allocation_script(spec, pk.BlockPool(spec.num_blocks, 16, spec.initial_order))
    pk.pa_validate_metadata(m.block_tables, m.seq_lens, m.query_start_loc, m.context_lens, m.slot_mapping,
                            spec.num_blocks)


def test_validator_catches_each_corruption():
    spec = W.make_config(1)
    m = W.run_allocation_script(spec, pk.BlockPool(spec.num_blocks, 16, spec.initial_order))
    args = dict(block_tables=m.block_tables, seq_lens=m.seq_lens, query_start_loc=m.query_start_loc,
                context_lens=m.context_lens, slot_mapping=m.slot_mapping)
    bad = []
    x = dict(args); x["seq_lens"] = m.seq_lens + np.array([1, 0, 0], np.int32); bad.append(x)
    x = dict(args); bt = m.block_tables.copy(); bt[2, 1] = 99; x["block_tables"] = bt; bad.append(x)
    x = dict(args); bt = m.block_tables.copy(); bt[0, 0] = -1; x["block_tables"] = bt; bad.append(x)
    x = dict(args); sm = m.slot_mapping.copy(); sm[1] = sm[0]; x["slot_mapping"] = sm; bad.append(x)
    x = dict(args); sm = m.slot_mapping.copy(); sm[3] = 16 * 16; x["slot_mapping"] = sm; bad.append(x)
    x = dict(args); q = m.query_start_loc.copy(); q[0] = 1; x["query_start_loc"] = q; bad.append(x)
    x = dict(args); x["block_tables"] = m.block_tables[:, :2]; bad.append(x)  # too narrow for 34 tokens
    for b in bad:
        with pytest.raises(pk.PAError):
            pk.pa_validate_metadata(num_blocks=spec.num_blocks, **b)
