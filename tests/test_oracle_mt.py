"""The oracle's multi-threaded forms against its single-threaded functions.

The threaded forms exist only to time the oracle on all host cores beside the
GPU; they must compute exactly what the single-threaded loops compute (which
the pins in test_oracle_pins.py tie to the page's definitions): the same
stream bytes, the same decoded patterns and the same error bits, for any
number of threads, including more threads than windows and corrupt streams.
"""

import numpy as np
import pytest

import oracle

THREADS = [1, 2, 3, 7, 16, 300]


def _patterns(n, esz, density, seed, clustered=False):
    rng = np.random.default_rng(seed)
    dt = np.uint32 if esz == 4 else np.uint16
    x = rng.integers(1, 2 ** (8 * esz), size=n, dtype=np.uint64).astype(dt)
    if clustered:
        keep = np.repeat(rng.random(n // 37 + 1) < density, 37)[:n]
    else:
        keep = rng.random(n) < density
    x[~keep] = 0
    return x


CASES = [(n, esz, d, c) for esz in (4, 2)
         for n in (0, 1, 31, 32, 33, 1023, 1024, 1025, 2049, 40000, 123457)
         for d, c in ((0.0, False), (0.5, False), (1.0, False), (0.3, True))]


@pytest.mark.parametrize("n,esz,dens,clustered", CASES)
def test_zvc_mt_equals_single_thread(n, esz, dens, clustered):
    x = _patterns(n, esz, dens, seed=n + esz, clustered=clustered)
    ref = oracle.zvc_compress(x)
    out_ref, e_ref = oracle.zvc_decompress(ref, n, esz)
    for t in THREADS:
        s = oracle.zvc_compress_mt(x, t)
        assert s.size == ref.size and np.array_equal(s, ref), t
        out, e = oracle.zvc_decompress_mt(ref, n, esz, t)
        assert e == e_ref == 0 and np.array_equal(out, out_ref) and np.array_equal(out, x), t


@pytest.mark.parametrize("n,esz,dens,clustered", CASES)
def test_rle_mt_equals_single_thread(n, esz, dens, clustered):
    x = _patterns(n, esz, dens, seed=3 * n + esz, clustered=clustered)
    ref = oracle.rle_compress(x)
    out_ref, e_ref = oracle.rle_decompress(ref, n, esz)
    for t in THREADS:
        s = oracle.rle_compress_mt(x, t)
        assert s.size == ref.size and np.array_equal(s, ref), t
        out, e = oracle.rle_decompress_mt(ref, n, esz, t)
        assert e == e_ref == 0 and np.array_equal(out, out_ref) and np.array_equal(out, x), t


def _corruptions(stream, rng, k=40):
    """Seeded corruptions: flipped bytes, cuts and extensions."""
    out = []
    for _ in range(k):
        s = stream.copy()
        kind = rng.integers(0, 3)
        if kind == 0 and s.size:
            i = rng.integers(0, s.size)
            s[i] ^= np.uint8(1 << rng.integers(0, 8))
        elif kind == 1 and s.size:
            s = s[: rng.integers(0, s.size)]
        else:
            s = np.concatenate([s, rng.integers(0, 256, size=rng.integers(1, 9), dtype=np.uint8)])
        out.append(s)
    return out


@pytest.mark.parametrize("algo", ["zvc", "rle"])
@pytest.mark.parametrize("esz", [4, 2])
def test_mt_decoders_report_the_same_errors(algo, esz):
    n = 5000 if esz == 4 else 9000
    x = _patterns(n, esz, 0.4, seed=7 + esz, clustered=True)
    comp = oracle.zvc_compress if algo == "zvc" else oracle.rle_compress
    dec = oracle.zvc_decompress if algo == "zvc" else oracle.rle_decompress
    dec_mt = oracle.zvc_decompress_mt if algo == "zvc" else oracle.rle_decompress_mt
    rng = np.random.default_rng(11 + esz)
    seen = 0
    for bad in _corruptions(comp(x), rng):
        out_ref, e_ref = dec(bad, n, esz)
        seen |= e_ref
        for t in (2, 5, 16):
            out, e = dec_mt(bad, n, esz, t)
            assert e == e_ref, (t, e, e_ref)
            assert np.array_equal(out, out_ref), t
    assert seen  # the corruptions did exercise the error paths
