"""The C-ABI library loads on the host, exports every entry point include/pa.h
declares, and rejects bad arguments before touching the GPU (CPU only)."""
import ctypes
import os
import re

import numpy as np
import pytest

import paged_kv_varlen_reshape_amd as pk
from paged_kv_varlen_reshape_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    names = set()
    inc = os.path.join(ROOT, "include")
    for h in sorted(os.listdir(inc)):
        if h.endswith(".h"):
            src = re.sub(r"/\*.*?\*/", "", open(os.path.join(inc, h)).read(), flags=re.S)
            names.update(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", src))
    return sorted(names)


def test_library_exports_every_declared_function():
    lib = pk.lib()
    names = header_functions()
    assert len(names) >= 17
    for n in names:
        assert hasattr(lib, n), n
        assert ctypes.cast(getattr(lib, n), ctypes.c_void_p).value


def test_binding_covers_header():
    assert set(header_functions()) == set(B.SIGNATURES)


def test_measure_rejects_bad_arguments():
    lib = pk.lib()
    assert lib.pa_measure_copy(16, 4096, 100, None) == pk.PA_ERR_INVALID  # not a multiple of 16
    assert lib.pa_measure_copy(16, 32, 64, None) == pk.PA_ERR_INVALID  # overlap
    assert lib.pa_measure_copy(None, 32, 64, None) == pk.PA_ERR_INVALID
    assert lib.pa_measure_read(8, 64, 4096, None) == pk.PA_ERR_INVALID  # misaligned
    assert lib.pa_measure_read(16, 0, 4096, None) == pk.PA_ERR_INVALID
    assert lib.pa_measure_gather(16, 4, 32, 4, 1000, 4096, None) == pk.PA_ERR_INVALID  # page not 1 KiB-aligned
    assert lib.pa_measure_gather(16, 4, None, 4, 4096, 4096, None) == pk.PA_ERR_INVALID
    assert lib.pa_measure_gather(16, 0, 32, 4, 4096, 4096, None) == pk.PA_ERR_INVALID
    flops = ctypes.c_int64(0)
    assert lib.pa_measure_mfma(0, 4096, ctypes.byref(flops), None) == pk.PA_ERR_INVALID
    assert lib.pa_measure_mfma(10, None, ctypes.byref(flops), None) == pk.PA_ERR_INVALID
    assert lib.pa_measure_mfma_random(0, 4096, ctypes.byref(flops), None) == pk.PA_ERR_INVALID
    assert lib.pa_measure_mfma_random(6, 4096, ctypes.byref(flops), None) == pk.PA_ERR_INVALID  # not a multiple of 4
    assert lib.pa_measure_mfma_random(8, None, ctypes.byref(flops), None) == pk.PA_ERR_INVALID


def test_reshape_rejects_bad_arguments():
    lib = pk.lib()
    ok = dict(num_tokens=4, hkv=2, d=64, bs=16, nb=8, dtype=pk.PA_F32)

    def call(num_tokens=4, hkv=2, d=64, bs=16, nb=8, dtype=pk.PA_F32, ptr=1):
        p = ptr
        return lib.pa_reshape_and_cache(p, p, p, p, p, num_tokens, hkv, d, bs, nb, dtype, None)

    assert call(d=96) == pk.PA_ERR_UNSUPPORTED
    assert call(bs=32) == pk.PA_ERR_UNSUPPORTED
    assert call(dtype=7) == pk.PA_ERR_UNSUPPORTED
    assert call(hkv=0) == pk.PA_ERR_INVALID
    assert call(nb=0) == pk.PA_ERR_INVALID
    assert call(nb=1 << 27) == pk.PA_ERR_INVALID  # slots would not fit in int32
    assert call(num_tokens=-1) == pk.PA_ERR_INVALID
    assert call(ptr=None) == pk.PA_ERR_INVALID
    assert "null" in pk.last_error()
    assert call(num_tokens=0, ptr=None) == pk.PA_OK  # nothing to do, nothing launched
    del ok


def test_attention_rejects_bad_arguments():
    lib = pk.lib()

    def call(hq=8, hkv=2, d=128, bs=16, nb=64, mbps=4, S=2, T=3, dtype=pk.PA_BF16, ws=256, ws_bytes=None,
             ptr=1, scale=0.1):
        need = lib.pa_attention_workspace_size(S, T, hq, hkv, d, mbps)
        wsb = need if ws_bytes is None else ws_bytes
        p = ptr
        return lib.pa_attention(p, p, p, p, p, p, p, scale, p, S, T, hq, hkv, d, bs, nb, mbps, T, dtype, ws, wsb,
                                None)

    assert call(hq=6, hkv=4) == pk.PA_ERR_INVALID
    assert call(hq=32, hkv=2) == pk.PA_ERR_UNSUPPORTED  # group 16 is not built
    assert call(d=80) == pk.PA_ERR_UNSUPPORTED
    assert call(bs=8) == pk.PA_ERR_UNSUPPORTED
    assert call(ws_bytes=16) == pk.PA_ERR_WORKSPACE
    assert call(ws=0) == pk.PA_ERR_WORKSPACE
    assert call(ws=257) == pk.PA_ERR_WORKSPACE  # misaligned
    assert call(ptr=None) == pk.PA_ERR_INVALID
    assert call(scale=float("nan")) == pk.PA_ERR_INVALID
    assert call(S=-1) == pk.PA_ERR_INVALID
    assert call(T=0, ptr=None) == pk.PA_OK
    assert call(mbps=0) == pk.PA_ERR_INVALID


def test_workspace_size_is_deterministic_and_grows():
    a = pk.pa_attention_workspace_size(64, 64, 32, 8, 128, 129)
    b = pk.pa_attention_workspace_size(64, 64, 32, 8, 128, 129)
    c = pk.pa_attention_workspace_size(6148, 8192, 32, 8, 128, 513)
    assert a == b > 0 and c > a and a % 256 == 0
    with pytest.raises(pk.PAError):
        pk.pa_attention_workspace_size(1, 1, 0, 1, 64, 1)


def test_options_roundtrip_and_errors():
    for opt, val in ((pk.PA_OPT_FORCE_ROWWISE, 1), (pk.PA_OPT_SPLIT_TOKENS, 64), (pk.PA_OPT_TARGET_ITEMS, 100),
                     (pk.PA_OPT_DECODE_BUFFERS, 2), (pk.PA_OPT_DECODE_KERNEL, 1), (pk.PA_OPT_VERIFY_ROWS, 3),
                     (pk.PA_OPT_CHUNK_KERNEL, 2)):
        old = pk.pa_get_option(opt)
        pk.pa_set_option(opt, val)
        assert pk.pa_get_option(opt) == val
        pk.pa_set_option(opt, old)
    with pytest.raises(pk.PAError):
        pk.pa_set_option(pk.PA_OPT_SPLIT_TOKENS, 17)
    with pytest.raises(pk.PAError):
        pk.pa_set_option(pk.PA_OPT_FORCE_ROWWISE, 2)
    with pytest.raises(pk.PAError):
        pk.pa_set_option(pk.PA_OPT_DECODE_BUFFERS, 5)
    with pytest.raises(pk.PAError):
        pk.pa_set_option(pk.PA_OPT_DECODE_KERNEL, -1)
    with pytest.raises(pk.PAError):
        pk.pa_set_option(pk.PA_OPT_VERIFY_ROWS, 17)
    with pytest.raises(pk.PAError):
        pk.pa_set_option(99, 0)


def test_noalloc_attention_rejects_bad_arguments_and_oversized_steps():
    """pa_attention_noalloc: pa_attention's argument checks, and a step whose workspace
    exceeds the static per-GPU array is refused before anything is launched."""
    lib = pk.lib()

    def call(hq=8, hkv=2, d=128, bs=16, nb=64, mbps=4, S=2, T=3, dtype=pk.PA_BF16, ptr=1, scale=0.1):
        p = ptr
        return lib.pa_attention_noalloc(p, p, p, p, p, p, p, scale, p, S, T, hq, hkv, d, bs, nb, mbps, T, dtype,
                                        None)

    assert call(hq=6, hkv=4) == pk.PA_ERR_INVALID
    assert call(d=80) == pk.PA_ERR_UNSUPPORTED
    assert call(ptr=None) == pk.PA_ERR_INVALID
    assert call(scale=float("inf")) == pk.PA_ERR_INVALID
    assert call(T=0, ptr=None) == pk.PA_OK
    big_T = 4 << 20
    assert pk.pa_attention_workspace_size(1, big_T, 8, 1, 128, 8) > (96 << 20)
    assert call(hq=8, hkv=1, S=1, T=big_T, mbps=8) == pk.PA_ERR_WORKSPACE
    assert "static scratch" in pk.last_error()


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without libpa.so the binding raises at the first call: there is no CPU
    or PyTorch fallback for any step of the path."""
    from paged_kv_varlen_reshape_amd import _binding
    monkeypatch.setattr(_binding, "LIB_PATH", str(tmp_path / "libpa.so"))
    monkeypatch.setattr(_binding, "_lib", None)
    with pytest.raises(ImportError, match="no fallback"):
        _binding.lib()
    with pytest.raises(ImportError):
        _binding.pa_attention_workspace_size(64, 64, 32, 8, 128, 129)
