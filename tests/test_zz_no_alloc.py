"""cdma_compress_noalloc (the compress entry point whose workspace is the
library's per-GPU static array) against cdma_compress with a caller
workspace: two calls in a row, the second on a smaller input, must each give
the same stream and size as the workspace entry point, and as the oracle."""


import numpy as np
import pytest

import oracle

from gpu_util import device, random_patterns, to_device

pytestmark = pytest.mark.gpu

ALGO = {"zvc": 0, "rle": 1, "zvci": 2}
ORACLE = {"zvc": oracle.zvc_compress, "rle": oracle.rle_compress, "zvci": oracle.zvci_compress}


def _noalloc(cdma, torch, xd, algo, esz):
    a = ALGO[algo]
    n = xd.numel()
    cap = cdma.cdma_max_compressed_bytes(a, esz, n)
    dst = torch.zeros(max(16, cap), dtype=torch.uint8, device=xd.device)
    sz = torch.full((1,), -1, dtype=torch.int64, device=xd.device)
    rc = cdma.cdma_compress_noalloc(a, esz, xd.data_ptr(), n, dst.data_ptr(), dst.numel(), sz.data_ptr(),
                                    torch.cuda.current_stream().cuda_stream)
    assert rc == 0, cdma.cdma_status_string(rc)
    torch.cuda.synchronize()
    size = int(sz.item())
    return dst[:size].cpu().numpy(), size


@pytest.mark.parametrize("algo", ["zvc", "rle", "zvci"])
@pytest.mark.parametrize("esz", [4, 2])
def test_noalloc_equals_workspace_entry_point_twice(algo, esz):
    import torch
    import sparse_activation_compression_amd as cdma
    device()
    # the first call leaves its aggregates in the shared array; the second,
    # smaller one must clear what it needs and give its own exact stream
    for n, dens, seed in ((4_000_037, 0.4, 3), (1_000_003, 0.7, 4)):
        bits = random_patterns(n, esz, dens, seed=seed + esz)
        xd = to_device(bits)
        ref, nb = cdma.compress(xd, algo)
        torch.cuda.synchronize()
        ref_size = int(nb.item())
        got, size = _noalloc(cdma, torch, xd, algo, esz)
        assert size == ref_size, (n, size, ref_size)
        assert np.array_equal(got, ref[:ref_size].cpu().numpy()), f"stream differs at n={n}"
        assert np.array_equal(got, ORACLE[algo](bits)), f"stream differs from the oracle at n={n}"


def test_noalloc_empty_input_and_host_checks():
    import torch
    import sparse_activation_compression_amd as cdma
    dev = device()
    sz = torch.full((1,), -1, dtype=torch.int64, device=dev)
    dst = torch.zeros(16, dtype=torch.uint8, device=dev)
    s = torch.cuda.current_stream().cuda_stream
    for algo, want in (("zvc", 0), ("rle", 8), ("zvci", 4)):
        sz.fill_(-1)
        assert cdma.cdma_compress_noalloc(ALGO[algo], 4, None, 0, dst.data_ptr(), 16, sz.data_ptr(), s) == 0
        torch.cuda.synchronize()
        assert int(sz.item()) == want
    # rejected on the host, nothing enqueued
    assert cdma.cdma_compress_noalloc(0, 4, None, 100, dst.data_ptr(), 10 ** 6, sz.data_ptr(), s) == 1
    assert cdma.cdma_compress_noalloc(0, 4, dst.data_ptr(), 100, dst.data_ptr(), 16, sz.data_ptr(), s) == 2
    assert cdma.cdma_compress_noalloc(1, 4, None, 0, None, 16, sz.data_ptr(), s) == 1
