"""The Python binding rejects inconsistent tensors before any pointer reaches the
library (CPU: the checks run before the device check)."""
import pytest
import torch

import paged_kv_varlen_reshape_amd as pk


def _step(T=5, S=2, hq=8, hkv=2, d=64, nb=16, mbps=4, dtype=torch.bfloat16):
    return dict(q=torch.zeros(T, hq, d, dtype=dtype), k_cache=torch.zeros(nb, hkv, 16, d, dtype=dtype),
                v_cache=torch.zeros(nb, hkv, 16, d, dtype=dtype),
                block_tables=torch.zeros(S, mbps, dtype=torch.int32), seq_lens=torch.ones(S, dtype=torch.int32),
                query_start_loc=torch.zeros(S + 1, dtype=torch.int32),
                context_lens=torch.zeros(S, dtype=torch.int32), scale=0.125)


def _call(**kw):
    args = _step()
    args.update(kw)
    return pk.pa_attention(**args)


def test_consistent_cpu_tensors_reach_the_device_check():
    with pytest.raises(ValueError, match="device tensor"):
        _call()


@pytest.mark.parametrize("bad,match", [
    (dict(k_cache=torch.zeros(16, 2, 16, 128, dtype=torch.bfloat16),
          v_cache=torch.zeros(16, 2, 16, 128, dtype=torch.bfloat16)), "head_dim"),
    (dict(v_cache=torch.zeros(8, 2, 16, 64, dtype=torch.bfloat16)), "v_cache"),
    (dict(k_cache=torch.zeros(16, 2, 16, 64, dtype=torch.float32),
          v_cache=torch.zeros(16, 2, 16, 64, dtype=torch.float32)), "dtype"),
    (dict(block_tables=torch.zeros(3, 4, dtype=torch.int32)), "block_tables"),
    (dict(block_tables=torch.zeros(8, dtype=torch.int32)), "block_tables"),
    (dict(query_start_loc=torch.zeros(2, dtype=torch.int32)), "query_start_loc"),
    (dict(context_lens=torch.zeros(3, dtype=torch.int32)), "context_lens"),
    (dict(seq_lens=torch.ones(2, dtype=torch.int64)), "int32"),
    (dict(out=torch.zeros(5, 8, 64, dtype=torch.bfloat16)), "out"),
    (dict(out=torch.zeros(4, 8, 64, dtype=torch.float32)), "out"),
    (dict(q=torch.zeros(5, 8, dtype=torch.bfloat16)), "q must be"),
])
def test_inconsistent_tensors_are_rejected(bad, match):
    with pytest.raises(ValueError, match=match):
        _call(**bad)


def test_scatter_rejects_mismatched_tensors():
    k = torch.zeros(3, 2, 64, dtype=torch.bfloat16)
    kc = torch.zeros(8, 2, 16, 64, dtype=torch.bfloat16)
    slots = torch.zeros(3, dtype=torch.int32)
    with pytest.raises(ValueError, match="shape"):
        pk.pa_reshape_and_cache(k, k, slots, kc, torch.zeros(8, 2, 16, 128, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="dtype"):
        pk.pa_reshape_and_cache(k, k, slots, kc.float(), kc.float())
    with pytest.raises(ValueError, match="slot_mapping"):
        pk.pa_reshape_and_cache(k, k, torch.zeros(2, dtype=torch.int32), kc, kc)
