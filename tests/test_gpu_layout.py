"""The layout study on the GPU ("Compressing DMA Engine: Leveraging Activation
Sparsity for Training Deep Neural Networks", §VII.A: ZVC's ratio does not
depend on how the activations are arranged, run-length coding's does).  The
same clustered post-ReLU map is laid out as NCHW, NHWC and CHWN; for each
layout the GPU streams must equal the oracle's byte for byte, the ZVC sizes
must be equal across layouts and the RLE sizes must not."""

import numpy as np
import pytest

import oracle

from gpu_util import bits_of, device, gpu_compress

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["alexnet_conv1_fp32_128x96x55x55", "fp16_256x256x56x56_s0.6_specials"])
def test_layouts_match_oracle_and_zvc_is_layout_invariant(name):
    from synth import LAYOUTS, to_layout, workload
    device()
    x = workload(name, scale_n=1 << 22)
    zsizes, rsizes = {}, {}
    for layout in LAYOUTS:
        b = bits_of(to_layout(x, layout))
        print(f"{name} {layout}: n={b.size}", flush=True)
        for algo, comp, sizes in (("zvc", oracle.zvc_compress, zsizes), ("rle", oracle.rle_compress, rsizes)):
            want = comp(b)
            got, size = gpu_compress(b, algo)
            assert size == want.size, (layout, algo)
            assert np.array_equal(got, want), (layout, algo)
            sizes[layout] = size
    assert len(set(zsizes.values())) == 1, zsizes
    assert len(set(rsizes.values())) == len(rsizes), rsizes
