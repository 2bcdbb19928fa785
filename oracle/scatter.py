"""Reference cache scatter (oracle, test infrastructure).

Before attention reads the paged cache, each new token's K and V rows are
written into the slot its request's block table gives it (the super-sequence
flattening of the Inside vLLM summary, "PagedAttentionの仕組み").

Cache layout (a convention of this implementation; the pages fix none):
``cache[block, kv_head, offset, dim]`` with ``offset = slot % block_size`` and
``block = slot // block_size``, so one (block, kv_head) page of 16 tokens is a
contiguous run of ``16 * head_dim`` elements.  A negative slot means "do not
store this token".  The copy is of raw element bits.
"""
from __future__ import annotations

import numpy as np


def ref_reshape_and_cache(k, v, slot_mapping, k_cache, v_cache, block_size: int = 16):
    """Return copies of ``k_cache``/``v_cache`` with the step's rows written in.

    k, v: [T, Hkv, D] element bits (any integer dtype); caches: [NB, Hkv, bs, D].
    """
    k = np.asarray(k)
    v = np.asarray(v)
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    nb = kc.shape[0]
    for n, s in enumerate(np.asarray(slot_mapping).tolist()):
        if s < 0:
            continue
        block, offset = divmod(s, block_size)
        if block >= nb:
            raise IndexError(f"slot {s} beyond the pool")
        kc[block, :, offset, :] = k[n]
        vc[block, :, offset, :] = v[n]
    return kc, vc
