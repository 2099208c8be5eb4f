"""Seeded random corruptions of valid streams, every codec and element size:
the GPU decoder must report exactly the oracle's error bits, and where
neither finds an error (a corruption that leaves a valid stream, such as a
changed value) the same output.  Index entries, run lengths, masks and values
are hit, and streams are cut short or extended ("Compressing DMA Engine:
Leveraging Activation Sparsity for Training Deep Neural Networks", §V.A; the
error bits are this library's, documented with cdma_decompress)."""

import numpy as np
import pytest

import oracle

from gpu_util import device, gpu_decompress, random_patterns

pytestmark = pytest.mark.gpu

CODEC = {"zvc": (oracle.zvc_compress, oracle.zvc_decompress),
         "rle": (oracle.rle_compress, oracle.rle_decompress),
         "zvci": (oracle.zvci_compress, oracle.zvci_decompress)}


def _input(rng, esz):
    n = int(rng.integers(1, 12000))
    x = random_patterns(n, esz, float(rng.choice([0.0, 0.05, 0.5, 0.95, 1.0])), seed=int(rng.integers(1 << 30)))
    if rng.random() < 0.5:  # zeros in runs as well
        a = int(rng.integers(0, n))
        x[a:a + int(rng.integers(1, 3000))] = 0
    return x


def _corrupt(rng, s):
    s = s.copy()
    kind = int(rng.integers(0, 6))
    if s.size == 0 or kind == 4:
        return np.concatenate([s, rng.integers(0, 256, size=int(rng.integers(1, 40)), dtype=np.uint8)])
    if kind == 5:
        return s[:int(rng.integers(0, s.size))]
    if kind == 0:      # one byte anywhere
        s[int(rng.integers(0, s.size))] ^= np.uint8(1 << int(rng.integers(0, 8)))
    elif kind == 1:    # a byte near the start (index, first masks or run lengths)
        s[int(rng.integers(0, min(s.size, 64)))] ^= np.uint8(int(rng.integers(1, 256)))
    elif kind == 2:    # several bytes
        for _ in range(int(rng.integers(2, 6))):
            s[int(rng.integers(0, s.size))] = np.uint8(int(rng.integers(0, 256)))
    else:              # a 16-bit field set to 0 or to all ones
        i = int(rng.integers(0, max(1, s.size - 1)))
        s[i:i + 2] = 0 if rng.random() < 0.5 else 255
    return s


@pytest.mark.parametrize("esz", [4, 2])
@pytest.mark.parametrize("algo", ["zvc", "rle", "zvci"])
def test_corrupted_streams_match_the_oracle(algo, esz):
    device()
    comp, dec = CODEC[algo]
    rng = np.random.default_rng({"zvc": 11, "rle": 22, "zvci": 33}[algo] + esz)
    clean = 0
    for k in range(60):
        x = _input(rng, esz)
        s = _corrupt(rng, comp(x))
        want, werr = dec(s, x.size, esz)
        got, gerr = gpu_decompress(s, x.size, esz, algo)
        assert gerr == werr, (k, x.size, s.size, gerr, werr)
        if werr == 0:
            clean += 1
            assert np.array_equal(got, want), (k, x.size)
    print(f"{algo} esz={esz}: {60 - clean} corrupt, {clean} still valid", flush=True)
