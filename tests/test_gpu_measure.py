"""The ceiling kernels behind bench.py's roofline fractions do the work they are
credited with (GPU): the copy copies, the read and the page gather fold every
32-bit word they are said to read exactly once (XOR), and the matrix-core loop
reports the flops of its launch."""
import numpy as np
import pytest
import torch

import paged_kv_varlen_reshape_amd as pk

pytestmark = pytest.mark.gpu


def _words(t):
    return t.view(torch.int32).cpu().numpy().view(np.uint32)


def _xor_all(a):
    return int(np.bitwise_xor.reduce(a.ravel())) if a.size else 0


def _src(nbytes, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=g)


def test_copy_copies():
    src = _src(64 << 20, 1)
    dst = torch.zeros_like(src)
    pk.pa_measure_copy(dst, src)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)


def test_read_folds_every_word_once():
    src = _src((48 << 20) + 4096, 2)  # not a multiple of the grid's stride
    out = torch.zeros(65536, dtype=torch.int32, device="cuda")
    pk.pa_measure_read(src, out)
    torch.cuda.synchronize()
    assert _xor_all(_words(out)) == _xor_all(_words(src))


@pytest.mark.parametrize("page", [1024, 4096])
def test_gather_reads_the_pages_named(page):
    src = _src(32 << 20, 3)
    n = src.numel() // page
    out = torch.zeros(65536, dtype=torch.int32, device="cuda")
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(4)).to(torch.int32).cuda()
    pk.pa_measure_gather(src, perm, page, out)
    torch.cuda.synchronize()
    assert _xor_all(_words(out)) == _xor_all(_words(src))  # every page once, any order
    # a page named twice cancels; numbers past the buffer are clamped to its last page
    pages = torch.tensor([5, 5, 7, n + 100, -3], dtype=torch.int32, device="cuda")
    out.zero_()
    pk.pa_measure_gather(src, pages, page, out)
    torch.cuda.synchronize()
    w = _words(src).reshape(n, page // 4)
    want = _xor_all(w[7]) ^ _xor_all(w[n - 1]) ^ _xor_all(w[0])
    assert _xor_all(_words(out)) == want


def test_mfma_loop_reports_its_flops():
    out = torch.zeros(65536, dtype=torch.float32, device="cuda")
    iters = 100
    flops = pk.pa_measure_mfma(iters, out)
    torch.cuda.synchronize()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert flops == cus * 2 * 4 * iters * 4 * 2 * 32 * 32 * 16
    got = out[: cus * 2 * 4].cpu().numpy()
    assert np.isfinite(got).all() and (got != 0).all()


def test_mfma_random_loop_reports_its_flops():
    out = torch.zeros(65536, dtype=torch.float32, device="cuda")
    iters = 100
    flops = pk.pa_measure_mfma_random(iters, out)
    torch.cuda.synchronize()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert flops == cus * 2 * 4 * iters * 4 * 2 * 32 * 32 * 16
    got = out[: cus * 2 * 4].cpu().numpy()
    assert np.isfinite(got).all() and (got != 0).all()
    # different lanes multiply different data
    assert len(np.unique(got)) > len(got) // 2
