"""The library on several streams at once and under HIP graph capture.

The compressors run persistent grids that take tiles from a ticket counter and
never assume that all their workgroups are resident, so two of them running
side by side on different streams (each taking part of the GPU) must both
finish with the exact stream.  Every call enqueues only kernels (the workspace
and size word are cleared by a fill kernel, not a memset node), so a captured
compress + decompress must replay correctly, replay after replay, with eager
work in between.  Streams are checked against the CPU oracle."""

import numpy as np
import pytest

import oracle

from gpu_util import device, random_patterns

pytestmark = pytest.mark.gpu

ORACLE = {"zvc": oracle.zvc_compress, "rle": oracle.rle_compress, "zvci": oracle.zvci_compress}


def _bits(n, density, seed):
    return random_patterns(n, 4, density, seed=seed)


def _to_dev(bits):
    import torch
    return torch.from_numpy(bits.view(np.int32).copy()).to(device())


def _buffers(cdma, algo, n):
    import torch
    a = {"zvc": 0, "rle": 1, "zvci": 2}[algo]
    dev = device()
    return (torch.empty(cdma.cdma_max_compressed_bytes(a, 4, n), dtype=torch.uint8, device=dev),
            torch.zeros(1, dtype=torch.int64, device=dev),
            torch.empty(max(256, cdma.cdma_workspace_bytes(a, 4, n)), dtype=torch.uint8, device=dev))


def test_concurrent_compressions_on_four_streams():
    import torch
    import sparse_activation_compression_amd as cdma
    device()
    jobs = [("zvc", (1 << 26) + 17, 0.5, 1), ("zvc", (1 << 26) + 4099, 0.1, 2),
            ("rle", (1 << 25) + 33, 0.5, 3), ("zvci", (1 << 26) + 5, 0.3, 4)]
    streams = [torch.cuda.Stream() for _ in jobs]
    prepared = []
    for algo, n, d, seed in jobs:
        x = _bits(n, d, seed)
        prepared.append((algo, x, _to_dev(x), *_buffers(cdma, algo, n)))
    torch.cuda.synchronize()
    for (algo, _, xd, dst, nb, ws), st in zip(prepared, streams):
        cdma.compress(xd, algo, dst=dst, out_bytes=nb, ws=ws, stream=st)
    torch.cuda.synchronize()
    for algo, x, _, dst, nb, ws in prepared:
        want = ORACLE[algo](x)
        size = int(nb.item())
        hdr = ws[:256].cpu().numpy().view(np.uint32)  # ticket counter, workgroups started, tile mode
        print(f"{algo} n={x.size}: size {size}, header words {hdr[0]} {hdr[16]} {hdr[32]}", flush=True)
        assert size == want.size
        assert np.array_equal(dst[:size].cpu().numpy(), want)


def test_compress_and_decompress_side_by_side():
    """A compression on one stream while two decompressions run on others."""
    import torch
    import sparse_activation_compression_amd as cdma
    device()
    n = (1 << 26) + 123
    xs = [_bits(n, 0.4, 10 + k) for k in range(3)]
    xds = [_to_dev(x) for x in xs]
    st = [torch.cuda.Stream() for _ in range(3)]
    bufs = [_buffers(cdma, "zvc", n) for _ in range(3)]
    # streams for k = 1, 2 prepared up front (on the current stream)
    for k in (1, 2):
        cdma.compress(xds[k], "zvc", dst=bufs[k][0], out_bytes=bufs[k][1], ws=bufs[k][2])
    outs = [torch.empty_like(xds[0]) for _ in range(3)]
    errs = [torch.zeros(1, dtype=torch.int32, device=device()) for _ in range(3)]
    dws = [torch.empty(cdma.cdma_workspace_bytes(0, 4, n), dtype=torch.uint8, device=device()) for _ in range(3)]
    torch.cuda.synchronize()
    cdma.compress(xds[0], "zvc", dst=bufs[0][0], out_bytes=bufs[0][1], ws=bufs[0][2], stream=st[0])
    for k in (1, 2):
        cdma.decompress(bufs[k][0], n, 4, "zvc", src_bytes=bufs[k][1], out=outs[k], error=errs[k], ws=dws[k],
                        stream=st[k])
    torch.cuda.synchronize()
    want = oracle.zvc_compress(xs[0])
    size = int(bufs[0][1].item())
    assert size == want.size and np.array_equal(bufs[0][0][:size].cpu().numpy(), want)
    for k in (1, 2):
        assert int(errs[k].item()) == 0
        assert torch.equal(outs[k], xds[k])


@pytest.mark.parametrize("algo", ["zvc", "rle", "zvci"])
def test_graph_capture_replays(algo):
    import torch
    import sparse_activation_compression_amd as cdma
    dev = device()
    n = 3 * 61440 + 1029  # several compress tiles and a ragged tail
    x0 = _bits(n, 0.5, 20)
    xd = _to_dev(x0)
    dst, nb, ws = _buffers(cdma, algo, n)
    out = torch.empty_like(xd)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    dws = torch.empty(max(256, cdma.cdma_workspace_bytes({"zvc": 0, "rle": 1, "zvci": 2}[algo], 4, n)),
                      dtype=torch.uint8, device=dev)

    def step():
        cdma.compress(xd, algo, dst=dst, out_bytes=nb, ws=ws)
        err.zero_()  # a kernel, not a memset node
        cdma.decompress(dst, n, 4, algo, src_bytes=nb, out=out, error=err, ws=dws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside capture (caches launch attributes)
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for r in range(3):
        x = _bits(n, (0.2, 0.7, 0.95)[r], 21 + r)
        xd.copy_(torch.from_numpy(x.view(np.int32).copy()).to(dev))  # eager work between replays
        out.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = ORACLE[algo](x)
        size = int(nb.item())
        print(f"{algo} replay {r}: size {size}", flush=True)
        assert size == want.size, r
        assert np.array_equal(dst[:size].cpu().numpy(), want), r
        assert int(err.item()) == 0, r
        assert torch.equal(out, xd), r


@pytest.mark.parametrize("algo", ["zvc", "rle", "zvci"])
def test_side_stream_with_buffers_made_by_the_binding(algo):
    """compress/decompress with stream= and no buffers passed in: the binding
    makes and zeroes the workspace, size and error words on that stream, so a
    busy current stream cannot clear the error bits after the decoder set them,
    and the round trip and the bits equal the oracle's."""
    import torch
    import sparse_activation_compression_amd as cdma
    n = 300_000
    bits = _bits(n, 0.4, seed=31)
    xd = _to_dev(bits)
    s = torch.cuda.Stream(device=device())
    torch.cuda.synchronize()
    torch.cuda._sleep(50_000_000)  # the current stream stays busy for tens of ms
    dst, nbytes = cdma.compress(xd, algo, stream=s)
    out, err = cdma.decompress(dst, n, 4, algo, src_bytes=nbytes, stream=s)
    s.synchronize()
    size = int(nbytes.item())
    expect = ORACLE[algo](bits)
    assert size == expect.size and np.array_equal(dst[:size].cpu().numpy(), expect)
    assert int(err.item()) == 0 and np.array_equal(out.cpu().numpy().view(np.uint32), bits)
    # a stream one value short: the decoder's error bits must survive
    bad = torch.from_numpy(expect[:-4].copy()).to(device())
    bad_size = torch.tensor([expect.size - 4], dtype=torch.int64, device=device())
    _, want = {"zvc": oracle.zvc_decompress, "rle": oracle.rle_decompress,
               "zvci": oracle.zvci_decompress}[algo](expect[:-4], n, 4)
    assert want != 0
    torch.cuda.synchronize()
    torch.cuda._sleep(50_000_000)
    _, err2 = cdma.decompress(bad, n, 4, algo, src_bytes=bad_size, stream=s)
    s.synchronize()
    got = int(err2.item())
    torch.cuda.synchronize()
    assert got == want, (got, want)
