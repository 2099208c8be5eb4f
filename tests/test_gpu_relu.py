"""Fused ReLU + compression on the GPU: the stream must be byte for byte the
oracle's stream of ReLU(x), and the dense output the oracle's ReLU(x)
("Compressing DMA Engine: Leveraging Activation Sparsity for Training Deep
Neural Networks", §I and §V.B: activation maps are compressed while they
are being moved out of GPU memory; §V.A: ZVC and run-length coding)."""

import numpy as np
import pytest

import oracle

from gpu_util import device

pytestmark = pytest.mark.gpu

FMTS = {"f32": (oracle.FMT_F32, np.uint32), "f16": (oracle.FMT_F16, np.uint16),
        "bf16": (oracle.FMT_BF16, np.uint16)}

# special patterns per format: -0.0, +-denormal, +-inf, +-NaN, -1.0, +1.0
SPECIALS = {
    "f32": [0x80000000, 0x00000001, 0x80000001, 0x7F800000, 0xFF800000, 0x7FC00000, 0xFFC00001, 0xBF800000,
            0x3F800000],
    "f16": [0x8000, 0x0001, 0x8001, 0x7C00, 0xFC00, 0x7E00, 0xFE01, 0xBC00, 0x3C00],
    "bf16": [0x8000, 0x0001, 0x8001, 0x7F80, 0xFF80, 0x7FC0, 0xFFC1, 0xBF80, 0x3F80],
}


def pre_activations(n, fmt_name, seed, zero_frac=0.5):
    """Random patterns, about zero_frac of them negative (and a few exact
    zeros), with the format's special patterns sprinkled in."""
    _, dt = FMTS[fmt_name]
    esz = np.dtype(dt).itemsize
    rng = np.random.default_rng(seed)
    x = rng.integers(0, 2 ** (8 * esz - 1), size=n, dtype=np.uint64).astype(dt)  # positive patterns
    neg = rng.random(n) < zero_frac
    x[neg] |= dt(1 << (8 * esz - 1))
    x[rng.random(n) < 0.02] = 0
    if n:
        pos = rng.integers(0, n, size=max(1, n // 100))
        x[pos] = np.array(SPECIALS[fmt_name], dtype=dt)[rng.integers(0, len(SPECIALS[fmt_name]), size=pos.size)]
    return x


def _torch_dtype(fmt_name):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[fmt_name]


def _gpu_relu_compress(x, fmt_name, algo, with_act=True):
    import torch
    import sparse_activation_compression_amd as cdma
    dev = device()
    sig = x.view(np.int32 if x.dtype.itemsize == 4 else np.int16)
    xd = torch.from_numpy(sig.copy()).to(dev).view(_torch_dtype(fmt_name))
    dst, nb, act = cdma.relu_compress(xd, algo, act=True if with_act else None)
    torch.cuda.synchronize()
    size = int(nb.item())
    a = act.view(torch.int32 if x.dtype.itemsize == 4 else torch.int16).cpu().numpy().view(x.dtype) if with_act \
        else None
    return dst[:size].cpu().numpy(), a, dst, nb


def _sizes(algo, esz):
    te = {("zvc", 4): 15360, ("zvc", 2): 30720, ("rle", 4): 15360, ("rle", 2): 14336}[(algo, esz)]
    return [1, 33, 1000, te - 1, te, te + 1, 3 * te + 17, 200_003]


@pytest.mark.parametrize("algo", ["zvc", "rle"])
@pytest.mark.parametrize("fmt_name", ["f32", "f16", "bf16"])
def test_stream_and_dense_output_match_oracle(fmt_name, algo):
    fmt, dt = FMTS[fmt_name]
    comp = oracle.zvc_compress if algo == "zvc" else oracle.rle_compress
    for n in _sizes(algo, np.dtype(dt).itemsize):
        x = pre_activations(n, fmt_name, seed=n)
        y = oracle.relu(x, fmt)
        want = comp(y)
        got, act, _, _ = _gpu_relu_compress(x, fmt_name, algo)
        assert got.size == want.size, (n, got.size, want.size)
        assert np.array_equal(got, want), f"stream differs at n={n}"
        assert np.array_equal(act, y), f"dense ReLU output differs at n={n}"


@pytest.mark.parametrize("fmt_name", ["f32", "bf16"])
def test_without_dense_output_and_round_trip(fmt_name):
    import torch
    import sparse_activation_compression_amd as cdma
    fmt, dt = FMTS[fmt_name]
    n = 5 * 15360 + 999
    x = pre_activations(n, fmt_name, seed=3, zero_frac=0.7)
    y = oracle.relu(x, fmt)
    got, _, dst, nb = _gpu_relu_compress(x, fmt_name, "zvc", with_act=False)
    assert np.array_equal(got, oracle.zvc_compress(y))
    out, err = cdma.decompress(dst, n, x.dtype.itemsize, "zvc", src_bytes=nb)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert np.array_equal(out.cpu().numpy().view(dt), y)


def test_every_16bit_pattern_fp16_and_bf16():
    """All 65536 patterns of each 16-bit format pass through the fused
    kernel's ReLU exactly as through the oracle's."""
    for fmt_name in ("f16", "bf16"):
        fmt, _ = FMTS[fmt_name]
        x = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
        got, act, _, _ = _gpu_relu_compress(x, fmt_name, "zvc")
        y = oracle.relu(x, fmt)
        assert np.array_equal(act, y), fmt_name
        assert np.array_equal(got, oracle.zvc_compress(y)), fmt_name


def test_sweep_4GiB_fused_equals_plain_compress():
    """At the 4 GiB size: negative pre-activations put where the map has its
    zeros make ReLU(x) the map itself, so the fused stream must equal the
    plain compressor's stream of the map, and the dense output the map."""
    import torch
    import sparse_activation_compression_amd as cdma
    from synth import sweep_bits_device
    dev = device()
    n = 1 << 30
    xm = sweep_bits_device(n, 0.5, 52, device=dev)
    minus_one = torch.tensor(-0x40800000, dtype=torch.int32, device=dev)  # the pattern of -1.0f
    pre = torch.where(xm == 0, minus_one, xm)
    ref, rnb = cdma.compress(xm, "zvc")
    dst, nb, act = cdma.relu_compress(pre.view(torch.float32), "zvc", act=True)
    torch.cuda.synchronize()
    size = int(nb.item())
    assert size == int(rnb.item())
    assert torch.equal(dst[:size], ref[:size])
    assert torch.equal(act.view(torch.int32), xm)
