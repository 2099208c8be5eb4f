"""Seeded random cases for every codec: lengths anywhere from one element to
several compress tiles (so ragged windows, blocks and tiles), both element
sizes, densities from empty to full, zeros either scattered or in runs.  The
GPU stream must equal the CPU oracle's byte for byte and the GPU must decode
the oracle's stream back to the input bit for bit."""

import numpy as np
import pytest

import oracle

from gpu_util import device, gpu_compress, gpu_decompress

pytestmark = pytest.mark.gpu

ORACLE = {"zvc": oracle.zvc_compress, "rle": oracle.rle_compress, "zvci": oracle.zvci_compress}


def _case(rng):
    esz = int(rng.choice([2, 4]))
    n = int(rng.choice([rng.integers(1, 300), rng.integers(300, 70000), rng.integers(70000, 400000)]))
    density = float(rng.choice([0.0, 1.0, rng.random(), rng.random() ** 4]))
    dt = np.uint32 if esz == 4 else np.uint16
    x = rng.integers(1, 2 ** (8 * esz), size=n, dtype=np.uint64).astype(dt)
    if rng.random() < 0.5:
        x[rng.random(n) >= density] = 0              # scattered zeros
    else:
        # zeros in runs: alternate run lengths drawn around a random mean
        mean = int(rng.integers(1, 3000))
        pos, keep = 0, rng.random() < density
        while pos < n:
            ln = int(rng.integers(1, 2 * mean + 1))
            if not keep:
                x[pos:pos + ln] = 0
            keep = not keep
            pos += ln
    return esz, x


@pytest.mark.parametrize("algo", ["zvc", "rle", "zvci"])
def test_random_cases(algo):
    device()
    rng = np.random.default_rng({"zvc": 101, "rle": 202, "zvci": 303}[algo])
    for k in range(40):
        esz, x = _case(rng)
        want = ORACLE[algo](x)
        got, size = gpu_compress(x, algo)
        assert size == want.size, (k, esz, x.size)
        assert np.array_equal(got, want), (k, esz, x.size)
        out, err = gpu_decompress(want, x.size, esz, algo)
        assert err == 0, (k, esz, x.size, err)
        assert np.array_equal(out, x), (k, esz, x.size)
