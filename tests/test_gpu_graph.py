"""The whole step (scatter, plan, kernels, merge) captured in a HIP graph.

The library allocates nothing, clears its counters with kernels (no memset
nodes) and never synchronises, so a step can be captured once per batch shape
and replayed.  Each replay must reproduce the eager step bit for bit (the
kernels are deterministic), with eager work and synchronisations between the
replays, and the replayed output is checked against the fp64 oracle on every
row (max-abs 1e-5 for float32 steps, 1e-2 for bf16).
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


def _specs():
    yield "decode bf16", W.make_config(2)
    yield "chunked prefill bf16", W.make_config(3)
    yield "short queries bf16", W.make_config(6)  # self-planned multi-row records
    yield "mixed f32", W.random_spec(50, num_seqs=6, max_context=200, max_query=30, num_q_heads=8, num_kv_heads=2,
                                     head_dim=64, dtype="f32", prefix_tokens=16, decode_fraction=0.5)
    yield "mixed bf16", W.random_spec(51, num_seqs=7, max_context=300, max_query=40, num_q_heads=16,
                                      num_kv_heads=2, head_dim=128, dtype="bf16", prefix_tokens=32,
                                      decode_fraction=0.5)


@pytest.mark.parametrize("name,spec", list(_specs()), ids=[n for n, _ in _specs()])
def test_step_replays_from_a_graph(name, spec):
    print(f"graph replay: {name}", flush=True)
    ds = build_device_step(spec)
    out = torch.empty((spec.num_tokens, spec.num_q_heads, spec.head_dim), dtype=torch.float32, device="cuda")
    ws = ds.workspace()
    ds.reshape()
    ref = ds.attention(out=torch.empty_like(out), workspace=ws).clone()
    torch.cuda.synchronize()
    assert torch.isfinite(ref).all()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture stream's side
        ds.reshape()
        ds.attention(out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ds.reshape()
        ds.attention(out=out, workspace=ws)

    rng = np.random.default_rng(7)
    junk = torch.randn(256, 256, device="cuda")
    for rep in range(4):
        out.fill_(float("nan"))
        ws.fill_(int(rng.integers(0, 256)))  # the step must not rely on workspace contents
        junk = torch.tanh(junk @ junk.t() * 1e-3)  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {rep} differs from the eager step"
    want, got = oracle_rows(spec, range(spec.num_seqs), out, ds.meta)
    err = float(np.abs(want - got).max())
    print(f"graph replay {name}: max_abs_err vs oracle {err:.3e}", flush=True)
    assert err <= TOL[spec.dtype], err
