"""The pins are strong enough: a plausible mistake planted in a copy of the oracle
(wrong index, dropped term, transposed operand, wrong queue end) fails at least
one of them.  All on the CPU; the real oracle is untouched."""
from collections import deque

import numpy as np
import pytest

import pins
from oracle import RefBlockPool, causal_attention, gather_sequence, ref_reshape_and_cache

G, S = gather_sequence, ref_reshape_and_cache


def _attn(mistake):
    def attn(q, K, V, positions, scale):
        q = np.asarray(q, float); K = np.asarray(K, float); V = np.asarray(V, float)
        n, hq, d = q.shape
        L, hkv, _ = K.shape
        g = hq // hkv
        pos = np.asarray(positions)
        if mistake == "exclude_self":
            masked = np.arange(L)[None, :] >= pos[:, None]
        else:
            masked = np.arange(L)[None, :] > pos[:, None]
        out = np.empty((n, hq, d))
        for h in range(hq):
            kvh = h % hkv if mistake == "gqa_modulo" else h // g
            Kh, Vh = K[:, kvh], V[:, kvh]
            if mistake == "swap_kv":
                Kh, Vh = Vh, Kh
            sc = 1.0 if mistake == "no_scale" else scale
            s = sc * (q[:, h] @ Kh.T)
            s = np.where(masked, -np.inf, s)
            w = np.exp(s - s.max(axis=1, keepdims=True))
            den = (~masked).sum(axis=1, keepdims=True) if mistake == "count_norm" else w.sum(axis=1, keepdims=True)
            if mistake == "drop_first_key":
                w[:, 0] = 0.0
            out[:, h] = (w @ Vh) / den
        return out
    return attn


def _gather_swapped(cache, row, length, bs=16):
    nblk = -(-length // bs)
    pages = cache[np.asarray(row[:nblk])]
    # forgets that head comes before offset in a page
    return pages.reshape(nblk * bs, cache.shape[1], cache.shape[3])[:length]


def _gather_wrong_block(cache, row, length, bs=16):
    nblk = -(-length // bs)
    ids = np.asarray(row[:nblk])[::-1]
    pages = cache[ids]
    return pages.transpose(0, 2, 1, 3).reshape(nblk * bs, cache.shape[1], cache.shape[3])[:length]


def _scatter_swapped(k, v, slots, kc, vc, bs=16):
    kc = np.array(kc, copy=True); vc = np.array(vc, copy=True)
    hkv = kc.shape[1]
    for n, s in enumerate(np.asarray(slots).tolist()):
        if s < 0:
            continue
        b, o = divmod(s, bs)
        flat_k = kc[b].reshape(-1, kc.shape[3]); flat_v = vc[b].reshape(-1, vc.shape[3])
        for h in range(hkv):
            flat_k[o * hkv + h] = k[n, h]  # token-major page instead of head-major
            flat_v[o * hkv + h] = v[n, h]
    return kc, vc


class _TailPool(RefBlockPool):
    def allocate_slots(self, req, done, new):
        n = self.blocks_needed(req, done, new)
        if n > len(self.free_block_queue):
            return None
        got = [self.free_block_queue.pop() for _ in range(n)]
        for b in got:
            self.refcount[b] = 1
        self.req_to_blocks.setdefault(req, []).extend(got)
        return got


class _FloorPool(RefBlockPool):
    def blocks_needed(self, req, done, new):
        return max(0, (done + new) // self.block_size + 1 - len(self.req_to_blocks.get(req, [])))


class _FreeToHeadPool(RefBlockPool):
    def free(self, req):
        for b in self.req_to_blocks.pop(req, []):
            self.refcount[b] -= 1
            if self.refcount[b] == 0:
                self.free_block_queue.appendleft(b)


class _NoRefcountPool(RefBlockPool):
    def free(self, req):
        for b in self.req_to_blocks.pop(req, []):
            if self.refcount[b] > 0:
                self.refcount[b] = 0
                self.free_block_queue.append(b)


class _PartialPool(RefBlockPool):
    def allocate_slots(self, req, done, new):
        n = self.blocks_needed(req, done, new)
        got = []
        while n and self.free_block_queue:
            got.append(self.free_block_queue.popleft()); n -= 1
        self.req_to_blocks.setdefault(req, []).extend(got)
        for b in got:
            self.refcount[b] = 1
        return None if n else got


def _fails(*checks):
    for c in checks:
        try:
            c()
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            return True
    return False


def _attn_checks(a):
    return [lambda: pins.pin_closed_forms(a), lambda: pins.pin_sdpa(a),
            lambda: pins.pin_bruteforce(a, G, S), lambda: pins.pin_decode_is_last_prefill_row(a)]


@pytest.mark.parametrize("mistake", ["exclude_self", "gqa_modulo", "swap_kv", "no_scale",
                                     "count_norm", "drop_first_key"])
def test_attention_mutant_is_caught(mistake):
    with np.errstate(all="ignore"):
        assert _fails(*_attn_checks(_attn(mistake)))


def test_real_oracle_passes_the_same_checks():
    assert not _fails(*_attn_checks(causal_attention))


@pytest.mark.parametrize("gather", [_gather_swapped, _gather_wrong_block])
def test_gather_mutant_is_caught(gather):
    assert _fails(lambda: pins.pin_cache_layout(S, gather),
                  lambda: pins.pin_bruteforce(causal_attention, gather, S))


def test_scatter_mutant_is_caught():
    assert _fails(lambda: pins.pin_cache_layout(_scatter_swapped, G))


@pytest.mark.parametrize("pool_cls", [_TailPool, _FloorPool, _FreeToHeadPool, _NoRefcountPool, _PartialPool])
def test_pool_mutant_is_caught(pool_cls):
    assert _fails(lambda: pins.pin_block_count(pool_cls), lambda: pins.pin_head_of_queue(pool_cls),
                  lambda: pins.pin_exhaustion(pool_cls), lambda: pins.pin_fifo_release(pool_cls),
                  lambda: pins.pin_refcount(pool_cls), lambda: pins.pin_tiny_allocation(pool_cls))
