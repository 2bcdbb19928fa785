"""Multi-step engine loop on the GPU: continuous batching with chunked prefill,
preemption by recompute and block reuse (and, in two cases, the pool's prefix
index: requests reuse the cached blocks of a shared system prompt and their own
released blocks), all steps writing into one persistent device pool through
pa_reshape_and_cache and reading it through pa_attention.

Every step's output is compared with the fp64 oracle computed from each
request's regenerated K/V (max-abs 1e-5 for fp32, 1e-2 for bf16), and after
the last step the whole device pool must equal the oracle's scatter model of
all steps bit for bit.
"""
import numpy as np
import pytest
import torch

import paged_kv_varlen_reshape_amd as pk
import workloads as W
from oracle import as_f64, causal_attention, ref_reshape_and_cache
from oracle_data import bits
from workloads.device import BITS_DT, poison_fill

pytestmark = pytest.mark.gpu
TOL = {"f32": 1e-5, "bf16": 1e-2}


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


@pytest.mark.parametrize("dtype,hq,hkv,d,seed,cache", [("f32", 8, 2, 64, 0, False), ("bf16", 8, 2, 128, 1, False),
                                                      ("f32", 8, 2, 64, 2, True), ("bf16", 8, 2, 128, 3, True)])
def test_engine_loop_matches_oracle_every_step(dtype, hq, hkv, d, seed, cache):
    """With ``cache`` the pool's prefix index is on and 70 % of the requests start with a
    48-token system prompt: reused blocks must hold the K/V their keys name."""
    cfg = W.EngineConfig(num_q_heads=hq, num_kv_heads=hkv, head_dim=d, dtype=dtype, seed=seed,
                         prefix_cache=cache, shared_prefix=48 if cache else 0, share_fraction=0.7 if cache else 0.0)
    eng = W.EngineLoop(cfg, pk.BlockPool(cfg.num_blocks, 16, None))
    shape = (cfg.num_blocks, hkv, 16, d)
    kc = poison_fill(shape, dtype, "cuda")
    vc = poison_fill(shape, dtype, "cuda")
    bdt = np.uint16 if dtype == "bf16" else np.uint32
    hk = np.full(shape, W.poison_bits(dtype), dtype=bdt)  # host scatter model
    hv = np.full(shape, W.poison_bits(dtype), dtype=bdt)
    worst, nsteps = 0.0, 0
    while True:
        st = eng.next_step()
        if st is None:
            break
        spec, meta = st.spec, st.meta
        if spec.num_tokens == 0:
            continue
        nsteps += 1
        reqs = spec.requests
        q = torch.cat([W.q_values(spec, r, "cuda") for r in reqs])
        kn = torch.cat([W.kv_values(spec, "k", r, r.context, r.seq_len, "cuda") for r in reqs])
        vn = torch.cat([W.kv_values(spec, "v", r, r.context, r.seq_len, "cuda") for r in reqs])
        pk.pa_reshape_and_cache(kn, vn, _i32(meta.slot_mapping), kc, vc)
        out = pk.pa_attention(q, kc, vc, _i32(meta.block_tables), _i32(meta.seq_lens),
                              _i32(meta.query_start_loc), _i32(meta.context_lens), spec.scale,
                              max_query_len=max(r.query for r in reqs))
        hk, hv = ref_reshape_and_cache(bits(kn.cpu()), bits(vn.cpu()), meta.slot_mapping, hk, hv, 16)
        got = out.double().cpu().numpy()
        assert np.isfinite(got).all(), f"step {st.index}: non-finite output"
        for i, r in enumerate(reqs):
            K = as_f64(bits(W.kv_values(spec, "k", r, 0, r.seq_len)), dtype)
            V = as_f64(bits(W.kv_values(spec, "v", r, 0, r.seq_len)), dtype)
            want = causal_attention(as_f64(bits(W.q_values(spec, r)), dtype), K, V,
                                    r.context + np.arange(r.query), spec.scale)
            err = float(np.abs(got[meta.query_start_loc[i]:meta.query_start_loc[i + 1]] - want).max())
            worst = max(worst, err)
            assert err <= TOL[dtype], f"step {st.index} request {r.key}: {err:.3e}"
    torch.cuda.synchronize()
    print(f"engine {dtype} cache={cache}: {nsteps} steps, {eng.preemptions} preemptions, "
          f"{eng.cache_hits} reused blocks, max_abs_err={worst:.3e}", flush=True)
    assert eng.preemptions > 0
    assert (eng.cache_hits > 0) == cache
    assert np.array_equal(kc.view(BITS_DT[dtype]).cpu().numpy().view(bdt), hk)
    assert np.array_equal(vc.view(BITS_DT[dtype]).cpu().numpy().view(bdt), hv)
