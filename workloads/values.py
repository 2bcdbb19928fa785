"""Seeded Q/K/V element values, identical on the host and on the device.

Every (tensor, sequence key, absolute position, head) picks one row of a
seeded table of ``table_rows`` vectors of length ``head_dim``; the row index
is a 32-bit integer hash of those four fields.  The tables are drawn once on
the host (``torch.randn`` from a seeded CPU generator, then rounded to the
step's dtype) and copied to the device as raw bits, and the hash uses only
integer tensor ops, so the values a GPU pool holds and the values the oracle
regenerates on the host are the same bits.

Element values are N(0, 1) draws rounded to the step dtype; a table of 2**16
or more rows keeps distinct tokens' vectors effectively independent for the
attention maths (repeats only re-use a vector at unrelated positions).
"""
from __future__ import annotations

from functools import lru_cache

import torch

from .configs import PREFIX_KEY, Request, StepSpec

_M32 = 0xFFFFFFFF
_TENSOR_ID = {"q": 1, "k": 2, "v": 3}


def _mix32(x: torch.Tensor) -> torch.Tensor:
    """32-bit integer finaliser on int64 tensors holding values in [0, 2**32)."""
    x = x ^ (x >> 16)
    x = (x * 0x45D9F3B) & _M32
    x = x ^ (x >> 16)
    x = (x * 0x45D9F3B) & _M32
    x = x ^ (x >> 16)
    return x


@lru_cache(maxsize=16)
def _table_cpu(seed: int, tensor: str, rows: int, dim: int, dtype: str) -> torch.Tensor:
    g = torch.Generator().manual_seed(seed * 1000 + _TENSOR_ID[tensor])
    t = torch.randn(rows, dim, generator=g, dtype=torch.float32)
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def value_table(spec: StepSpec, tensor: str, device="cpu") -> torch.Tensor:
    """Table [table_rows, head_dim] in the step dtype (torch.float32 or torch.bfloat16)."""
    t = _table_cpu(spec.seed, tensor, spec.table_rows, spec.head_dim, spec.dtype)
    return t if str(device) == "cpu" else t.to(device)


def _row_index(spec: StepSpec, tensor: str, keys: torch.Tensor, pos: torch.Tensor,
               heads: int) -> torch.Tensor:
    """Row indices [n, heads] for (key, pos) pairs given as int64 tensors [n]."""
    base = _mix32(torch.full_like(keys, (spec.seed * 0x9E37 + _TENSOR_ID[tensor]) & _M32))
    h = _mix32(base ^ (keys & _M32))
    h = _mix32(h ^ (pos & _M32))
    hd = torch.arange(heads, dtype=torch.int64, device=keys.device)
    h = _mix32(h[:, None] ^ hd[None, :])
    return h & (spec.table_rows - 1)


def kv_key_for(spec: StepSpec, req: Request, pos: torch.Tensor) -> torch.Tensor:
    """Value key of each K/V position of ``req``: the shared prefix has a key of its own."""
    keys = torch.full_like(pos, req.key)
    if req.shares_prefix and spec.prefix_tokens:
        keys = torch.where(pos < spec.prefix_tokens, torch.full_like(pos, PREFIX_KEY), keys)
    return keys


def kv_rows(spec: StepSpec, tensor: str, keys: torch.Tensor, pos: torch.Tensor) -> torch.Tensor:
    assert tensor in ("k", "v")
    return _row_index(spec, tensor, keys, pos, spec.num_kv_heads)


def q_rows(spec: StepSpec, keys: torch.Tensor, pos: torch.Tensor) -> torch.Tensor:
    return _row_index(spec, "q", keys, pos, spec.num_q_heads)


def kv_values(spec: StepSpec, tensor: str, req: Request, pos_start: int, pos_end: int,
              device="cpu") -> torch.Tensor:
    """K or V of ``req`` at positions [pos_start, pos_end): [n, Hkv, D] in the step dtype."""
    pos = torch.arange(pos_start, pos_end, dtype=torch.int64, device=device)
    idx = kv_rows(spec, tensor, kv_key_for(spec, req, pos), pos)
    return value_table(spec, tensor, device)[idx]


def q_values(spec: StepSpec, req: Request, device="cpu") -> torch.Tensor:
    """Q rows of ``req`` for this step (positions context..seq_len-1): [q, Hq, D]."""
    pos = torch.arange(req.context, req.seq_len, dtype=torch.int64, device=device)
    idx = q_rows(spec, torch.full_like(pos, req.key), pos)
    return value_table(spec, "q", device)[idx]


def poison_bits(dtype: str) -> int:
    """Bit pattern of a quiet NaN in the step dtype, used to fill unused cache slots."""
    return 0x7FC0 if dtype == "bf16" else 0x7FC00000
