"""ctypes binding of libpa.so: argument marshalling only.

Every step of the hot path runs in the HIP kernels behind the C ABI declared
in include/pa.h; this module turns torch tensors into device pointers and the
current HIP stream, and numpy arrays into host pointers.  It raises if the
library is missing: there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import List, Optional

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpa.so")

PA_OK = 0
PA_ERR_INVALID = -1
PA_ERR_UNSUPPORTED = -2
PA_ERR_HIP = -3
PA_ERR_WORKSPACE = -4
PA_ERR_NO_BLOCKS = -5
PA_F32 = 0
PA_BF16 = 1
PA_OPT_FORCE_ROWWISE = 1
PA_OPT_SPLIT_TOKENS = 2
PA_OPT_TARGET_ITEMS = 3
PA_OPT_DECODE_BUFFERS = 4
PA_OPT_DECODE_KERNEL = 5
PA_OPT_VERIFY_ROWS = 6
PA_OPT_CHUNK_KERNEL = 7
PA_FLAG_BLOCK_ID = 1
PA_FLAG_ROWS = 2
PA_K_RESHAPE, PA_K_PLAN, PA_K_CHUNK, PA_K_DECODE, PA_K_MERGE, PA_K_COUNT = range(6)
KERNEL_NAMES = ["reshape_and_cache", "plan", "chunk_mfma", "decode", "split_merge"]  # PA_K_* kinds

_i32, _i64, _f32, _vp, _sz = C.c_int32, C.c_int64, C.c_float, C.c_void_p, C.c_size_t
_pi32 = C.POINTER(C.c_int32)
_pu64 = C.POINTER(C.c_uint64)

# name -> (restype, argtypes); mirrors include/pa.h
SIGNATURES = {
    "pa_reshape_and_cache": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i64, _i32, _vp]),
    "pa_attention_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "pa_attention": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _f32, _vp, _i32, _i32, _i32, _i32, _i32,
                            _i32, _i64, _i32, _i32, _i32, _vp, _sz, _vp]),
    "pa_attention_noalloc": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _f32, _vp, _i32, _i32, _i32, _i32, _i32,
                                    _i32, _i64, _i32, _i32, _i32, _vp]),
    "pa_attention_flags": (_i32, [_vp, _pi32, _i32, _vp]),
    "pa_validate_metadata": (_i32, [_pi32, _pi32, _pi32, _pi32, _pi32, _i32, _i32, _i32, _i64, _i32]),
    "pa_last_error": (C.c_char_p, []),
    "pa_set_option": (_i32, [_i32, _i64]),
    "pa_get_option": (_i64, [_i32]),
    "pa_profile_enable": (_i32, [_i32]),
    "pa_profile_read": (_i32, [C.POINTER(C.c_int64), C.POINTER(C.c_double)]),
    "pa_measure_copy": (_i32, [_vp, _vp, _sz, _vp]),
    "pa_measure_read": (_i32, [_vp, _sz, _vp, _vp]),
    "pa_measure_gather": (_i32, [_vp, _i64, _vp, _i64, _i32, _vp, _vp]),
    "pa_measure_mfma": (_i32, [_i32, _vp, C.POINTER(C.c_int64), _vp]),
    "pa_measure_mfma_random": (_i32, [_i32, _vp, C.POINTER(C.c_int64), _vp]),
    "pa_pool_create": (_vp, [_i64, _i32, _pi32]),
    "pa_pool_destroy": (None, [_vp]),
    "pa_allocate_slots": (_i32, [_vp, _i64, _i64, _i64, _pi32, _i32, _pi32]),
    "pa_share_prefix": (_i32, [_vp, _i64, _pi32, _i32]),
    "pa_free": (_i32, [_vp, _i64]),
    "pa_num_free": (_i64, [_vp]),
    "pa_prefix_match": (_i32, [_vp, _i64, _pu64, _i32, _pi32]),
    "pa_prefix_register": (_i32, [_vp, _i64, _pu64, _i32]),
    "pa_prefix_cached": (_i64, [_vp]),
    "pa_num_req_blocks": (_i32, [_vp, _i64]),
    "pa_refcount": (_i32, [_vp, _i32]),
    "pa_block_table_row": (_i32, [_vp, _i64, _pi32, _i32, _i32]),
    "pa_slot_mapping": (_i32, [_vp, _i64, _i64, _i32, _pi32]),
}

_lib: Optional[C.CDLL] = None


class PAError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libpa error {code}: {msg}")
        self.code = code


def lib() -> C.CDLL:
    """Load libpa.so from the package directory (built by build())."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m paged_kv_varlen_reshape_amd.build` (no fallback path exists)")
        l = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


def last_error() -> str:
    return lib().pa_last_error().decode()


def _check(rc: int) -> int:
    if rc < 0:
        raise PAError(rc, last_error())
    return rc


def _np_i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _ptr32(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(_pi32)


# ----------------------------------------------------------------- device calls
def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.bfloat16:
        return PA_BF16
    if t.dtype == torch.float32:
        return PA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream_handle(device) -> int:
    import torch

    return torch.cuda.current_stream(device).cuda_stream


def _dev_ptr(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def pa_reshape_and_cache(k, v, slot_mapping, k_cache, v_cache) -> None:
    """Scatter k, v [T, Hkv, D] into k_cache, v_cache [NB, Hkv, 16, D] at slot_mapping [T] (int32)."""
    T, hkv, d = k.shape
    nb, hkv2, bs, d2 = k_cache.shape
    if v.shape != k.shape or v_cache.shape != k_cache.shape or (hkv2, d2) != (hkv, d):
        raise ValueError("shape mismatch")
    if k.dtype != k_cache.dtype or v.dtype != k.dtype or v_cache.dtype != k.dtype:
        raise ValueError("dtype mismatch")
    if slot_mapping.dtype != __import__("torch").int32 or slot_mapping.numel() != T:
        raise ValueError("slot_mapping must be int32 [T]")
    _check(lib().pa_reshape_and_cache(_dev_ptr(k, "k"), _dev_ptr(v, "v"), _dev_ptr(slot_mapping, "slot_mapping"),
                                      _dev_ptr(k_cache, "k_cache"), _dev_ptr(v_cache, "v_cache"), T, hkv, d, bs,
                                      nb, _dtype_code(k), _stream_handle(k.device)))


def pa_attention_workspace_size(num_seqs: int, num_tokens: int, num_q_heads: int, num_kv_heads: int,
                                head_dim: int, max_blocks_per_seq: int) -> int:
    n = lib().pa_attention_workspace_size(num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim,
                                          max_blocks_per_seq)
    if n == 0:
        raise PAError(PA_ERR_INVALID, "invalid shape for workspace sizing")
    return int(n)


def pa_attention(q, k_cache, v_cache, block_tables, seq_lens, query_start_loc, context_lens, scale: float,
                 out=None, workspace=None, max_query_len=None):
    """Attention of the step's query rows q [T, Hq, D] over the paged caches; returns out [T, Hq, D] fp32.

    max_query_len: the step's longest query as the caller knows it (host int); None passes T (unknown)."""
    import torch

    # the library sees only pointers and sizes: every size it derives from
    # these tensors is checked here, before any kernel could read past one
    if q.dim() != 3 or k_cache.dim() != 4:
        raise ValueError("q must be [T, Hq, D] and k_cache [NB, Hkv, 16, D]")
    T, hq, d = q.shape
    nb, hkv, bs, d2 = k_cache.shape
    if v_cache.shape != k_cache.shape:
        raise ValueError("v_cache must have k_cache's shape")
    if d2 != d:
        raise ValueError(f"q has head_dim {d}, the caches {d2}")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("q and the caches must share one dtype")
    S = seq_lens.numel()
    if block_tables.dim() != 2 or (S > 0 and block_tables.shape[0] != S):
        raise ValueError("block_tables must be [num_seqs, max_blocks_per_seq]")
    mbps = block_tables.shape[1]
    if context_lens.numel() != S or query_start_loc.numel() != S + 1:
        raise ValueError("seq_lens and context_lens need num_seqs entries, query_start_loc num_seqs + 1")
    for t, n in ((block_tables, "block_tables"), (seq_lens, "seq_lens"), (query_start_loc, "query_start_loc"),
                 (context_lens, "context_lens")):
        if t.dtype != torch.int32:
            raise ValueError(f"{n} must be int32")
    devices = {t.device for t in (q, k_cache, v_cache, block_tables, seq_lens, query_start_loc, context_lens)}
    if out is not None:
        if tuple(out.shape) != (T, hq, d) or out.dtype != torch.float32:
            raise ValueError("out must be float32 [T, Hq, D]")
        devices.add(out.device)
    if workspace is not None:
        devices.add(workspace.device)
    if len(devices) != 1:
        raise ValueError("all tensors must be on one device")
    if out is None:
        out = torch.empty((T, hq, d), dtype=torch.float32, device=q.device)
    need = pa_attention_workspace_size(S, T, hq, hkv, d, mbps)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _check(lib().pa_attention(_dev_ptr(q, "q"), _dev_ptr(k_cache, "k_cache"), _dev_ptr(v_cache, "v_cache"),
                              _dev_ptr(block_tables, "block_tables"), _dev_ptr(seq_lens, "seq_lens"),
                              _dev_ptr(query_start_loc, "query_start_loc"), _dev_ptr(context_lens, "context_lens"),
                              float(scale), _dev_ptr(out, "out"), S, T, hq, hkv, d, bs, nb, mbps,
                              T if max_query_len is None else int(max_query_len), _dtype_code(q),
                              _dev_ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
                              _stream_handle(q.device)))
    return out


def pa_attention_noalloc(q, k_cache, v_cache, block_tables, seq_lens, query_start_loc, context_lens, scale: float,
                         out, max_query_len=None):
    """pa_attention with the library's static per-GPU workspace instead of a caller buffer
    (nothing is allocated: `out` must be given).  Calls that overlap on one GPU race."""
    import torch

    if q.dim() != 3 or k_cache.dim() != 4:
        raise ValueError("q must be [T, Hq, D] and k_cache [NB, Hkv, 16, D]")
    T, hq, d = q.shape
    nb, hkv, bs, d2 = k_cache.shape
    if v_cache.shape != k_cache.shape or d2 != d or k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("q and the caches disagree in shape or dtype")
    S = seq_lens.numel()
    if block_tables.dim() != 2 or (S > 0 and block_tables.shape[0] != S):
        raise ValueError("block_tables must be [num_seqs, max_blocks_per_seq]")
    if context_lens.numel() != S or query_start_loc.numel() != S + 1:
        raise ValueError("seq_lens and context_lens need num_seqs entries, query_start_loc num_seqs + 1")
    for t in (block_tables, seq_lens, query_start_loc, context_lens):
        if t.dtype != torch.int32:
            raise ValueError("index arrays must be int32")
    if tuple(out.shape) != (T, hq, d) or out.dtype != torch.float32:
        raise ValueError("out must be float32 [T, Hq, D]")
    if len({t.device for t in (q, k_cache, v_cache, block_tables, seq_lens, query_start_loc, context_lens,
                               out)}) != 1:
        raise ValueError("all tensors must be on one device")
    _check(lib().pa_attention_noalloc(_dev_ptr(q, "q"), _dev_ptr(k_cache, "k_cache"), _dev_ptr(v_cache, "v_cache"),
                                      _dev_ptr(block_tables, "block_tables"), _dev_ptr(seq_lens, "seq_lens"),
                                      _dev_ptr(query_start_loc, "query_start_loc"),
                                      _dev_ptr(context_lens, "context_lens"), float(scale), _dev_ptr(out, "out"),
                                      S, T, hq, hkv, d, bs, nb, block_tables.shape[1],
                                      T if max_query_len is None else int(max_query_len), _dtype_code(q),
                                      _stream_handle(q.device)))
    return out


def pa_attention_flags(workspace=None, clear: bool = False, device=None) -> int:
    """Sticky PA_FLAG_* bits of metadata the kernels clamped, from a pa_attention
    workspace (None: this device's pa_attention_noalloc workspace); waits for the
    current stream.  clear=True zeroes the word afterwards."""
    import torch

    dev = workspace.device if workspace is not None else (device or torch.device("cuda", torch.cuda.current_device()))
    out = C.c_int32(0)
    ptr = _dev_ptr(workspace, "workspace") if workspace is not None else None
    _check(lib().pa_attention_flags(ptr, C.byref(out), 1 if clear else 0, _stream_handle(dev)))
    return int(out.value)


def pa_measure_copy(dst, src) -> None:
    """Streaming copy of src into dst (device tensors of the same byte size)."""
    nb = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nb:
        raise ValueError("size mismatch")
    _check(lib().pa_measure_copy(_dev_ptr(dst, "dst"), _dev_ptr(src, "src"), nb, _stream_handle(src.device)))


def pa_measure_read(src, out) -> None:
    """Read-only pass over src; out is an int32 device tensor of >= 65536 entries."""
    if out.numel() < 65536 or out.dtype.itemsize != 4:
        raise ValueError("out must hold 65536 32-bit entries")
    _check(lib().pa_measure_read(_dev_ptr(src, "src"), src.numel() * src.element_size(), _dev_ptr(out, "out"),
                                 _stream_handle(src.device)))


def pa_measure_gather(src, pages, page_bytes: int, out) -> None:
    """Reads the page_bytes pages of src named by the int32 device tensor pages, in
    order; out is an int32 device tensor of >= 65536 entries."""
    import torch
    if out.numel() < 65536 or out.dtype.itemsize != 4:
        raise ValueError("out must hold 65536 32-bit entries")
    if pages.dtype != torch.int32:
        raise ValueError("pages must be int32")
    nb = src.numel() * src.element_size()
    _check(lib().pa_measure_gather(_dev_ptr(src, "src"), nb // page_bytes, _dev_ptr(pages, "pages"), pages.numel(),
                                   page_bytes, _dev_ptr(out, "out"), _stream_handle(src.device)))


def pa_measure_mfma(iters: int, out) -> int:
    """bf16 matrix-core loop; out is a float32 device tensor of >= 65536 entries.
    Returns the launch's flop count."""
    if out.numel() < 65536 or out.dtype.itemsize != 4:
        raise ValueError("out must hold 65536 32-bit entries")
    flops = C.c_int64(0)
    _check(lib().pa_measure_mfma(int(iters), _dev_ptr(out, "out"), C.byref(flops), _stream_handle(out.device)))
    return flops.value


def pa_measure_mfma_random(iters: int, out) -> int:
    """bf16 matrix-core loop on N(0,1)-like operands that change with every product;
    out as for pa_measure_mfma.  Returns the launch's flop count."""
    if out.numel() < 65536 or out.dtype.itemsize != 4:
        raise ValueError("out must hold 65536 32-bit entries")
    flops = C.c_int64(0)
    _check(lib().pa_measure_mfma_random(int(iters), _dev_ptr(out, "out"), C.byref(flops),
                                        _stream_handle(out.device)))
    return flops.value


# ----------------------------------------------------------------- host calls
def pa_validate_metadata(block_tables, seq_lens, query_start_loc, context_lens, slot_mapping,
                         num_blocks: int, block_size: int = 16) -> None:
    bt = _np_i32(block_tables)
    sl, qsl, cl = _np_i32(seq_lens), _np_i32(query_start_loc), _np_i32(context_lens)
    sm = None if slot_mapping is None else _np_i32(slot_mapping)
    S = sl.size
    mbps = bt.shape[1] if bt.ndim == 2 else 0
    T = int(qsl[-1]) if qsl.size else 0
    if sm is not None:
        T = sm.size
    _check(lib().pa_validate_metadata(_ptr32(bt), _ptr32(sl), _ptr32(qsl), _ptr32(cl), _ptr32(sm), S, T, mbps,
                                      num_blocks, block_size))


def pa_set_option(option: int, value: int) -> None:
    _check(lib().pa_set_option(option, value))


def pa_get_option(option: int) -> int:
    return int(lib().pa_get_option(option))


def pa_profile_enable(mask: int) -> None:
    _check(lib().pa_profile_enable(mask))


def pa_profile_read():
    """{kernel name: (timed launches, summed ms)} since the last read; clears the record."""
    counts = (C.c_int64 * PA_K_COUNT)()
    ms = (C.c_double * PA_K_COUNT)()
    _check(lib().pa_profile_read(counts, ms))
    return {KERNEL_NAMES[k]: (int(counts[k]), float(ms[k])) for k in range(PA_K_COUNT)}


class BlockPool:
    """The C++ block allocator (pa_pool_*), same interface as the oracle's reference pool."""

    def __init__(self, num_blocks: int, block_size: int = 16, initial_order=None):
        order = None if initial_order is None else _np_i32(initial_order)
        self._order = order
        h = lib().pa_pool_create(num_blocks, block_size, _ptr32(order))
        if not h:
            raise PAError(PA_ERR_INVALID, last_error())
        self._h = C.c_void_p(h)
        self.num_blocks = num_blocks
        self.block_size = block_size

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and _lib is not None:
            _lib.pa_pool_destroy(h)
            self._h = None

    def allocate_slots(self, req: int, num_computed: int, num_new: int) -> Optional[List[int]]:
        cap = max(1, (num_computed + num_new) // self.block_size + 2)
        buf = np.empty(cap, dtype=np.int32)
        n = C.c_int32(0)
        rc = lib().pa_allocate_slots(self._h, req, num_computed, num_new, _ptr32(buf), cap, C.byref(n))
        if rc == PA_ERR_NO_BLOCKS:
            return None
        _check(rc)
        return buf[: n.value].tolist()

    def share_prefix(self, req: int, ids) -> None:
        a = _np_i32(ids)
        _check(lib().pa_share_prefix(self._h, req, _ptr32(a), a.size))

    def free(self, req: int) -> None:
        _check(lib().pa_free(self._h, req))

    def prefix_match(self, req: int, keys) -> int:
        """Reuse the cached blocks of the leading keys (up to the first miss); returns how many."""
        k = np.ascontiguousarray(keys, dtype=np.uint64)
        n = C.c_int32(0)
        _check(lib().pa_prefix_match(self._h, req, k.ctypes.data_as(_pu64), k.size, C.byref(n)))
        return int(n.value)

    def prefix_register(self, req: int, keys) -> None:
        """Register the request's first len(keys) blocks under these keys."""
        k = np.ascontiguousarray(keys, dtype=np.uint64)
        _check(lib().pa_prefix_register(self._h, req, k.ctypes.data_as(_pu64), k.size))

    @property
    def num_cached(self) -> int:
        return int(lib().pa_prefix_cached(self._h))

    @property
    def num_free(self) -> int:
        return int(lib().pa_num_free(self._h))

    def refcount(self, block: int) -> int:
        return int(lib().pa_refcount(self._h, block))

    def blocks(self, req: int) -> List[int]:
        n = lib().pa_num_req_blocks(self._h, req)
        return self.block_table_row(req, n, -1).tolist()

    def block_table_row(self, req: int, width: int, pad_value: int = -1) -> np.ndarray:
        out = np.empty(width, dtype=np.int32)
        _check(lib().pa_block_table_row(self._h, req, _ptr32(out), width, pad_value))
        return out

    def slot_mapping(self, req: int, start_pos: int, n: int) -> np.ndarray:
        out = np.empty(n, dtype=np.int32)
        _check(lib().pa_slot_mapping(self._h, req, start_pos, n, _ptr32(out)))
        return out
