"""The oracle pinned against the pages' worked example, closed forms, a library
routine, brute force and the invariants the method guarantees (CPU only)."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import RefBlockPool, causal_attention, gather_sequence, ref_reshape_and_cache
from oracle import ref_attention_dense, ref_attention_paged, bf16_bits_to_f64, f32_to_bf16_bits_rne
import pins
from oracle_data import build_oracle_step

A, G, S = causal_attention, gather_sequence, ref_reshape_and_cache


def test_block_count_worked_example():
    pins.pin_block_count()


def test_pool_head_of_queue():
    pins.pin_head_of_queue()


def test_pool_exhaustion_has_no_side_effect():
    pins.pin_exhaustion()


def test_pool_release_goes_to_tail():
    pins.pin_fifo_release()


def test_pool_refcounted_prefix():
    pins.pin_refcount()


def test_tiny_step_allocation_by_hand():
    pins.pin_tiny_allocation()


def test_cache_layout_golden():
    pins.pin_cache_layout(S, G)


@pytest.mark.parametrize("cfg", [1, 3])
def test_scatter_then_gather_is_contiguous_history(cfg):
    pins.pin_scatter_gather_dense(W.make_config(cfg), S, G)


def test_scatter_gather_random_and_prefix():
    pins.pin_scatter_gather_dense(W.random_spec(3, num_seqs=6, max_context=70, prefix_tokens=32), S, G)


def test_paged_equals_bruteforce():
    pins.pin_bruteforce(A, G, S)


def test_equals_torch_sdpa_float64():
    pins.pin_sdpa(A)


def test_closed_forms():
    pins.pin_closed_forms(A)


def test_decode_is_last_prefill_row():
    pins.pin_decode_is_last_prefill_row(A)


def test_chunked_equals_full_prefill():
    pins.pin_chunked_equals_full(A)


def test_block_permutation_invariance():
    pins.pin_permutation_invariance(A, G, S)


def test_isolation_between_sequences():
    pins.pin_isolation(A, G, S)


def test_prefix_sharing_equals_private_copies():
    pins.pin_prefix_sharing(A, G, S)


def test_sequence_order_permutes_rows():
    pins.pin_order(A, G, S)


def test_paged_api_matches_dense_api():
    spec = W.random_spec(9, num_seqs=5, max_context=45, max_query=6, head_dim=16, prefix_tokens=16)
    st = build_oracle_step(spec)
    kc, vc = S(st.k_new, st.v_new, st.meta.slot_mapping, st.k_cache_pre, st.v_cache_pre, 16)
    m = st.meta
    paged = ref_attention_paged(st.f64(st.q), st.f64(kc), st.f64(vc), m.block_tables, m.seq_lens,
                                m.query_start_loc, m.context_lens, spec.scale)
    qs = [st.f64(st.q)[m.query_start_loc[i]:m.query_start_loc[i + 1]] for i in range(spec.num_seqs)]
    dense = ref_attention_dense(qs, [st.f64(k) for k in st.k_full], [st.f64(v) for v in st.v_full],
                                m.context_lens, spec.scale)
    assert np.abs(np.concatenate(dense) - paged).max() <= 1e-12


def test_paged_rejects_inconsistent_lengths():
    spec = W.random_spec(10, num_seqs=2)
    st = build_oracle_step(spec)
    m = st.meta
    bad = m.seq_lens.copy()
    bad[0] += 1
    with pytest.raises(ValueError):
        ref_attention_paged(st.f64(st.q), st.f64(st.k_cache_pre), st.f64(st.v_cache_pre),
                            m.block_tables, bad, m.query_start_loc, m.context_lens, spec.scale)


def test_bf16_widening_is_exact():
    # exact powers of two, signs, subnormal and the largest finite bf16
    bits = np.array([0x3F80, 0xBF80, 0x4000, 0x0001, 0x7F7F, 0x0000, 0x8000], dtype=np.uint16)
    want = [1.0, -1.0, 2.0, 2.0 ** -133, (2 - 2 ** -7) * 2.0 ** 127, 0.0, -0.0]
    got = bf16_bits_to_f64(bits)
    assert got.tolist() == want
    # rounding to nearest, ties to even
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20], dtype=np.float32)
    assert f32_to_bf16_bits_rne(x).tolist() == [0x3F80, 0x3F82, 0x3F81]


def test_generator_values_are_device_independent_bits():
    """The seeded tables round-trip to bits and the row hash is pure integer maths."""
    spec = W.make_config(2)
    r = spec.requests[3]
    a = W.kv_values(spec, "k", r, 0, 40)
    b = W.kv_values(spec, "k", r, 0, 40)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert float(a.float().std()) == pytest.approx(1.0, abs=0.1)
