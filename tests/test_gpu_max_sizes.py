"""The largest inputs each codec accepts (CDMA_ZVC_MAX_N = 2^31 elements for
ZVC and interleaved ZVC, CDMA_RLE_MAX_N = 2^30 for run-length), fp32 bit
patterns of the sweep generator with half the values zero, in the launch
configuration the benchmark times.  At 2^31 the oracle would take minutes, so
the stream is checked by its closed-form size (nonzeros counted by torch),
a bit-exact round trip, the whole interleaved index, and regions at the start,
middle and end compared byte for byte with the oracle's encoding of the same
elements ("Compressing DMA Engine: Leveraging Activation Sparsity for Training
Deep Neural Networks", §V.A; §VII.A for the 4 KB window)."""

import numpy as np
import pytest

import oracle

from gpu_util import device

pytestmark = pytest.mark.gpu


def _round(xd, algo):
    import torch
    import sparse_activation_compression_amd as cdma
    dst, nb = cdma.compress(xd, algo)
    out, err = cdma.decompress(dst, xd.numel(), 4, algo, src_bytes=nb)
    torch.cuda.synchronize()
    same = bool(torch.equal(out, xd))
    del out
    return dst, int(nb.item()), int(err.item()), same


def test_zvc_at_the_largest_n():
    import torch
    from synth import sweep_bits_device
    dev = device()
    n = 1 << 31
    W = n // 32
    xd = sweep_bits_device(n, 0.5, 52, device=dev)
    dst, size, err, same = _round(xd, "zvc")
    per_window = (xd.view(W, 32) != 0).sum(1)
    nnz = int(per_window.sum().item())
    print(f"zvc n=2^31: size {size}, nonzeros {nnz}", flush=True)
    assert err == 0 and same
    assert size == 4 * W + 4 * nnz
    before = torch.cumsum(per_window, 0) - per_window      # nonzeros before each window
    span = 1 << 17                                          # elements per sampled region
    for lo in (0, (n // 2 // span) * span + 12345 * 32, n - span):
        seg = xd[lo:lo + span].cpu().numpy().view(np.uint32)
        want = oracle.zvc_compress(seg)
        g0, wm = lo // 32, span // 32
        assert np.array_equal(dst[4 * g0:4 * (g0 + wm)].cpu().numpy(), want[:4 * wm]), lo
        v0 = 4 * W + 4 * int(before[g0].item())
        nv = want.size - 4 * wm
        assert np.array_equal(dst[v0:v0 + nv].cpu().numpy(), want[4 * wm:]), lo
    del xd, dst, per_window, before
    torch.cuda.empty_cache()


def test_interleaved_at_the_largest_n():
    import torch
    from synth import sweep_bits_device
    dev = device()
    n = 1 << 31
    E = 1024
    Wr = n // E
    xd = sweep_bits_device(n, 0.5, 53, device=dev)
    dst, size, err, same = _round(xd, "zvci")
    per_block = (xd.view(Wr, E) != 0).sum(1)
    index = torch.zeros(Wr + 1, dtype=torch.int64, device=dev)
    index[1:] = torch.cumsum(per_block, 0)
    nnz = int(index[-1].item())
    print(f"zvci n=2^31: size {size}, nonzeros {nnz}", flush=True)
    assert err == 0 and same
    assert size == 4 * (Wr + 1) + 4 * (n // 32) + 4 * nnz
    assert np.array_equal(dst[:4 * (Wr + 1)].cpu().numpy().view("<u4").astype(np.int64), index.cpu().numpy())
    blocks = 128
    for b0 in (0, Wr // 2 + 777, Wr - blocks):
        seg = xd[b0 * E:(b0 + blocks) * E].cpu().numpy().view(np.uint32)
        want = oracle.zvci_compress(seg)[4 * (blocks + 1):]   # the blocks after the slice's own index
        at = 4 * (Wr + 1) + 4 * b0 * (E // 32) + 4 * int(index[b0].item())
        assert np.array_equal(dst[at:at + want.size].cpu().numpy(), want), b0
    del xd, dst, per_block, index
    torch.cuda.empty_cache()


def test_rle_at_the_largest_n():
    import torch
    from synth import sweep_bits_device
    dev = device()
    n = 1 << 30
    xd = sweep_bits_device(n, 0.5, 54, device=dev)
    dst, size, err, same = _round(xd, "rle")
    print(f"rle n=2^30: size {size}", flush=True)
    assert err == 0 and same
    got = dst[:size].cpu().numpy()
    x = xd.cpu().numpy().view(np.uint32)
    del xd, dst
    torch.cuda.empty_cache()
    want = oracle.rle_compress(x)
    assert got.size == want.size
    assert np.array_equal(got, want)
