"""Parity on the five workloads at their full sizes: every byte of the GPU
stream equals the CPU oracle's, and decompressing it on the GPU gives back
the input bit for bit.  The workloads stand in for the activation maps of
the ImageNet CNNs studied in "Compressing DMA Engine: Leveraging Activation
Sparsity for Training Deep Neural Networks" (§IV sparsity, §V.A codecs,
§VII.A 4 KB window); see synth/activations.py for the recipes."""

import numpy as np
import pytest

import oracle

from gpu_util import bits_of, device, to_device

pytestmark = pytest.mark.gpu

NAMED = ["single_map_fp32_1x64x56x56_s0.5", "alexnet_conv1_fp32_128x96x55x55",
         "vgg16_layer1_fp32_32x64x224x224", "vgg16_layer2_fp32_32x128x112x112",
         "vgg16_layer3_fp32_32x256x56x56", "vgg16_layer4_fp32_32x512x28x28",
         "vgg16_layer5_fp32_32x512x14x14", "fp16_256x256x56x56_s0.6_specials"]


def _gpu_round(xd, esz, algo):
    import torch
    import sparse_activation_compression_amd as cdma
    dst, nb = cdma.compress(xd, algo)
    out, err = cdma.decompress(dst, xd.numel(), esz, algo, src_bytes=nb)
    torch.cuda.synchronize()
    size = int(nb.item())
    return dst[:size].cpu().numpy(), int(err.item()), bool(torch.equal(out, xd))


@pytest.mark.parametrize("name", NAMED)
@pytest.mark.parametrize("algo", ["zvc", "rle"])
def test_named_workload(name, algo):
    from synth import workload
    device()
    x = bits_of(workload(name))
    print(f"{name} {algo}: n={x.size}", flush=True)
    xd = to_device(x)
    got, err, same = _gpu_round(xd, x.dtype.itemsize, algo)
    want = oracle.zvc_compress(x) if algo == "zvc" else oracle.rle_compress(x)
    assert got.size == want.size
    assert np.array_equal(got, want)
    assert err == 0 and same


def test_fp16_workload_has_the_patterns_it_must_keep():
    from synth import workload
    x = bits_of(workload("fp16_256x256x56x56_s0.6_specials", scale_n=1 << 22))
    assert (x == 0x8000).any() and ((x > 0) & (x < 0x0400)).any()


SWEEP = [(0.0, 50), (0.25, 51), (0.5, 52), (0.75, 53), (0.9, 54), (0.99, 55), (1.0, 56)]


@pytest.mark.parametrize("s,seed", SWEEP, ids=[f"s{s}" for s, _ in SWEEP])
def test_sweep_4GiB(s, seed):
    """The 4 GiB buffer: the GPU generator is checked against the host one on
    a sample, then the whole GPU stream is compared with the oracle's."""
    import torch
    from synth import sweep_bits_device, sweep_bits_host
    dev = device()
    n = 1 << 30
    xd = sweep_bits_device(n, s, seed, device=dev)
    for lo in (0, 123456789, n - 4096):
        assert np.array_equal(xd[lo:lo + 4096].cpu().numpy().view(np.uint32), sweep_bits_host(lo, 4096, s, seed))
    got, err, same = _gpu_round(xd, 4, "zvc")
    assert err == 0 and same
    x = xd.cpu().numpy().view(np.uint32)
    del xd
    torch.cuda.empty_cache()
    want = oracle.zvc_compress(x)
    assert got.size == want.size
    assert np.array_equal(got, want)


@pytest.mark.parametrize("s,seed", [(0.5, 52), (0.99, 55)])
def test_sweep_4GiB_offload(s, seed):
    import torch
    import sparse_activation_compression_amd as cdma
    from synth import sweep_bits_device
    dev = device()
    n, chunk = 1 << 30, 1 << 24
    xd = sweep_bits_device(n, s, seed, device=dev)
    host = torch.empty(cdma.cdma_max_compressed_bytes(0, 4, n) + (n // chunk) * 256, dtype=torch.uint8,
                       pin_memory=True)
    rc, total, sizes = cdma.offload(xd, host, chunk, "zvc", 3).wait()
    assert rc == 0 and len(sizes) == n // chunk and sum(sizes) == total
    x = xd.cpu().numpy().view(np.uint32)
    del xd
    img = host.numpy()
    lo = 0
    for k, sz in enumerate(sizes):
        want = oracle.zvc_compress(x[k * chunk:(k + 1) * chunk])
        assert sz == want.size, k
        assert np.array_equal(img[lo:lo + sz], want), k
        lo += sz
