"""Helpers shared by the GPU parity tests: move seeded host inputs to the
device, run the library through its binding and bring results back."""

import numpy as np
import pytest


def device():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    return torch.device("cuda:0")


def bits_of(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x).reshape(-1)
    return x.view(np.uint32 if x.dtype.itemsize == 4 else np.uint16)


def to_device(bits: np.ndarray):
    import torch
    sig = bits.view(np.int32 if bits.dtype.itemsize == 4 else np.int16)
    return torch.from_numpy(sig.copy()).to(device())


def random_patterns(n: int, esz: int, density: float, seed: int) -> np.ndarray:
    """Random nonzero bit patterns at the given density, with some -0.0,
    denormal and NaN patterns mixed in."""
    rng = np.random.default_rng(seed)
    dt = np.uint32 if esz == 4 else np.uint16
    x = rng.integers(1, 2 ** (8 * esz), size=n, dtype=np.uint64).astype(dt)
    x[rng.random(n) >= density] = 0
    if n:
        sp = np.array([0x80000000, 1, 0x7FC00001] if esz == 4 else [0x8000, 1, 0x7E01], dtype=dt)
        pos = rng.integers(0, n, size=max(1, n // 200))
        keep = x[pos] != 0  # specials only replace nonzeros so the density holds
        x[pos[keep]] = sp[rng.integers(0, 3, size=int(keep.sum()))]
    return x


def gpu_compress(bits: np.ndarray, algo: str = "zvc"):
    """(stream uint8 array, size) from the HIP library."""
    import torch
    import sparse_activation_compression_amd as cdma
    xd = to_device(bits)
    dst, nbytes = cdma.compress(xd, algo)
    torch.cuda.synchronize()
    size = int(nbytes.item())
    return dst[:size].cpu().numpy(), size


def gpu_decompress(stream: np.ndarray, n: int, esz: int, algo: str = "zvc", exact_size: bool = True,
                   capacity_pad: int = 0):
    """(patterns, error bits) from the HIP library for a host stream."""
    import torch
    import sparse_activation_compression_amd as cdma
    dev = device()
    buf = np.zeros(stream.size + capacity_pad, dtype=np.uint8)
    buf[:stream.size] = stream
    src = torch.from_numpy(buf).to(dev)
    sb = torch.tensor([stream.size], dtype=torch.int64, device=dev) if exact_size else None
    out, err = cdma.decompress(src, n, esz, algo, src_bytes=sb)
    torch.cuda.synchronize()
    o = out.cpu().numpy().view(np.uint32 if esz == 4 else np.uint16)
    return o, int(err.item())
