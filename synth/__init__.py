"""Seeded synthetic activation maps shared by the tests, the benchmark and smoke().

This package only draws inputs.  It holds none of the codec's arithmetic
(no masks, counts, runs or offsets) and imports neither the oracle nor the
HIP library, so both sides of every parity check read the same bytes without
sharing any code that computes a result.
"""

from .activations import (  # noqa: F401
    iid_relu,
    clustered_relu,
    inject_specials,
    sweep_bits_host,
    sweep_bits_device,
    SWEEP_ZERO_FRACTIONS,
    SWEEP_SEEDS,
    WORKLOADS,
    LAYOUTS,
    to_layout,
    workload,
)
