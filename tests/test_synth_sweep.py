"""The 4 GiB sweep generator: zero fractions, forced windows and magnitudes.

The sweep stands in for the page's measured sparsities; these checks tie what
it generates to the zero fraction each configuration names.
"""

import numpy as np
import pytest

from synth import SWEEP_SEEDS, SWEEP_ZERO_FRACTIONS, sweep_bits_host

N = 1 << 21  # 65536 windows of 32


@pytest.mark.parametrize("s,seed", list(zip(SWEEP_ZERO_FRACTIONS, SWEEP_SEEDS)))
def test_zero_fraction_and_forced_windows(s, seed):
    x = sweep_bits_host(0, N, s, seed)
    zero = x == 0
    g = np.arange(N) >> 5
    if s in (0.0, 1.0):
        assert zero.mean() == s  # no forcing at the ends
        return
    forced_zero = g % 97 == 0
    forced_dense = (g % 89 == 1) & ~forced_zero
    assert zero[forced_zero].all()
    assert not zero[forced_dense].any()
    free = ~(forced_zero | forced_dense)
    # binomial: 2^21 draws, so 5 standard deviations are well under 0.002
    sd = np.sqrt(s * (1 - s) / free.sum())
    assert abs(zero[free].mean() - s) < 5 * sd + 1e-9


def test_magnitudes_are_exact_positive_floats():
    x = sweep_bits_host(12345, 1 << 16, 0.5, 52)
    v = x[x != 0].view(np.float32)
    assert (v > 0).all() and np.isfinite(v).all()
    m = v * 256.0  # (2|S - 510| + 1) with S a byte sum: odd integers up to 1021
    assert np.array_equal(m, np.round(m)) and (m % 2 == 1).all() and m.max() <= 1021


def test_windows_regenerate_anywhere():
    a = sweep_bits_host(0, 1 << 16, 0.75, 53)
    b = sweep_bits_host(40000, 1000, 0.75, 53)
    assert np.array_equal(a[40000:41000], b)
