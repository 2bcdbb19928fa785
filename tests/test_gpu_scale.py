"""Scales other than 1/sqrt(D), through every attention kernel, against the oracle (GPU).

Every row's weights are softmax(scale * <q, K_t>) over its visible keys, the
scale applied before the maximum (Inside vLLM summary, techfeed.io, section
"PagedAttentionの仕組み": each sequence attends to its own tokens under
positions and a mask; where the scale sits is this repository's reading, the
same one the oracle takes).  The library accepts any finite scale, so a zero,
a negative and a large one must come out right on each kernel:
  * the MFMA chunk kernels (rows of multi-row sequences, bf16: four
    wavefronts per workgroup, and eight in two alternating groups),
  * the MFMA row-wise decode kernel (decode rows, bf16; every row when forced),
  * the VALU row-wise kernel (float32 steps; bf16 rows on request).
At scale 0 every weight is equal, so each row is also checked against the
closed form: the mean of the V rows it sees, computed straight from the seeded
values with no softmax involved.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import paged_kv_varlen_reshape_amd as pk
import workloads as W
from workloads.device import build_device_step
from device_data import oracle_rows

pytestmark = pytest.mark.gpu
TOL = {"f32": 1e-5, "bf16": 1e-2}


@pytest.fixture(autouse=True)
def _reset_options():
    yield
    pk.pa_set_option(pk.PA_OPT_FORCE_ROWWISE, 0)
    pk.pa_set_option(pk.PA_OPT_DECODE_KERNEL, 0)
    pk.pa_set_option(pk.PA_OPT_SPLIT_TOKENS, 0)
    pk.pa_set_option(pk.PA_OPT_CHUNK_KERNEL, 0)


def _mixed_spec(dtype, d, g, seed):
    """Chunks over no context (the causal diagonal in almost every key tile), over
    context that starts mid-page, long enough for several key tiles and a ragged
    last query tile, next to decodes (one of them the very first token)."""
    reqs = [W.Request(0, 0, 150), W.Request(1, 37, 1), W.Request(2, 200, 77), W.Request(3, 0, 1),
            W.Request(4, 1000, 1), W.Request(5, 5, 3), W.Request(6, 330, 1)]
    nb = sum(-(-r.seq_len // 16) for r in reqs) + 4
    order = np.random.default_rng((seed, 0)).permutation(nb).astype(np.int32)
    return W.StepSpec(f"scale-{dtype}-d{d}-g{g}", seed, 2 * g, 2, d, dtype, 16, nb, 1.0 / math.sqrt(d), reqs,
                      initial_order=order, table_rows=4096, seed=seed)


def _mean_of_visible_v(spec):
    """Closed form at scale 0: row j of sequence i is the mean of V[0..c_i + j]."""
    from oracle import as_f64
    from oracle_data import bits

    g = spec.num_q_heads // spec.num_kv_heads
    rows = []
    for r in spec.requests:
        V = as_f64(bits(W.kv_values(spec, "v", r, 0, r.seq_len)), spec.dtype)  # [L, Hkv, D]
        csum = np.cumsum(V, axis=0)
        for j in range(r.query):
            p = r.context + j
            rows.append(np.repeat(csum[p] / (p + 1), g, axis=0))  # [Hq, D]
    return np.stack(rows)


# (kernel routing name, FORCE_ROWWISE, DECODE_KERNEL, CHUNK_KERNEL): which kernels compute the rows
ROUTES = {
    "chunk+decode_mfma": (0, 2, 1),
    "chunk_pp+decode_mfma": (0, 2, 2),
    "chunk+decode_valu": (0, 1, 1),
    "all_decode_mfma": (1, 2, 0),
    "all_decode_valu": (1, 1, 0),
}


@pytest.mark.parametrize("d,g", [(128, 4), (64, 8), (128, 1)])
@pytest.mark.parametrize("route", list(ROUTES))
def test_bf16_scales_every_kernel(route, d, g):
    spec = _mixed_spec("bf16", d, g, 600 + d + g)
    rowwise, kernel, chunk = ROUTES[route]
    print(f"scales bf16 route={route} d={d} g={g}", flush=True)
    ds = build_device_step(spec)
    ds.reshape()
    pk.pa_set_option(pk.PA_OPT_FORCE_ROWWISE, rowwise)
    pk.pa_set_option(pk.PA_OPT_DECODE_KERNEL, kernel)
    pk.pa_set_option(pk.PA_OPT_CHUNK_KERNEL, chunk)
    for scale in (0.0, -1.0 / math.sqrt(d), -0.6, 2.0, 8.0):
        for split in (0, 48):
            pk.pa_set_option(pk.PA_OPT_SPLIT_TOKENS, split)
            out = pk.pa_attention(ds.q, ds.k_cache, ds.v_cache, ds.block_tables, ds.seq_lens, ds.query_start_loc,
                                  ds.context_lens, scale, max_query_len=ds.max_query_len)
            torch.cuda.synchronize()
            assert torch.isfinite(out).all(), f"non-finite output at scale {scale}"
            sp = dataclasses.replace(spec, scale=scale)
            want, got = oracle_rows(sp, range(sp.num_seqs), out, ds.meta)
            err = float(np.abs(want - got).max())
            print(f"  scale={scale:+.4f} split={split} max_abs_err={err:.3e}", flush=True)
            assert err <= TOL["bf16"], (scale, split, err)
            if scale == 0.0:
                mean_err = float(np.abs(_mean_of_visible_v(spec) - got).max())
                assert mean_err <= TOL["bf16"], ("closed form", mean_err)


@pytest.mark.parametrize("d,g", [(64, 1), (128, 4)])
def test_f32_scales_valu_kernel(d, g):
    spec = _mixed_spec("f32", d, g, 700 + d + g)
    print(f"scales f32 d={d} g={g}", flush=True)
    ds = build_device_step(spec)
    ds.reshape()
    for scale in (0.0, -1.0 / math.sqrt(d), -0.3, 1.0):
        out = pk.pa_attention(ds.q, ds.k_cache, ds.v_cache, ds.block_tables, ds.seq_lens, ds.query_start_loc,
                              ds.context_lens, scale, max_query_len=ds.max_query_len)
        torch.cuda.synchronize()
        assert torch.isfinite(out).all()
        sp = dataclasses.replace(spec, scale=scale)
        want, got = oracle_rows(sp, range(sp.num_seqs), out, ds.meta)
        err = float(np.abs(want - got).max())
        print(f"  scale={scale:+.4f} max_abs_err={err:.3e}", flush=True)
        assert err <= TOL["f32"], (scale, err)
        if scale == 0.0:
            assert float(np.abs(_mean_of_visible_v(spec) - got).max()) <= TOL["f32"]


def test_zero_scale_on_the_chunked_prefill_step():
    """Configuration-shaped chunk rows (8 chunks of 512 over 0..1536 cached tokens,
    every query tile and the whole causal diagonal) at scale 0 and at a negative
    scale, on the chunk kernel alone."""
    spec = W.make_config(3)
    ds = build_device_step(spec)
    ds.reshape()
    seqs = [0, 3, 5]
    for scale in (0.0, -1.0 / math.sqrt(128)):
        out = pk.pa_attention(ds.q, ds.k_cache, ds.v_cache, ds.block_tables, ds.seq_lens, ds.query_start_loc,
                              ds.context_lens, scale, max_query_len=ds.max_query_len)
        torch.cuda.synchronize()
        assert torch.isfinite(out).all()
        sp = dataclasses.replace(spec, scale=scale)
        want, got = oracle_rows(sp, seqs, out, ds.meta)
        err = float(np.abs(want - got).max())
        print(f"chunked prefill scale={scale:+.4f} max_abs_err={err:.3e}", flush=True)
        assert err <= TOL["bf16"], (scale, err)
