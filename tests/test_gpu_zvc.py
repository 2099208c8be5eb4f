"""ZVC on the GPU against the CPU oracle: byte-exact streams, bitwise round
trips and identical error reports ("Compressing DMA Engine: Leveraging
Activation Sparsity for Training Deep Neural Networks", §V.A)."""

import numpy as np
import pytest

import oracle

from gpu_util import bits_of, device, gpu_compress, gpu_decompress, random_patterns, to_device

pytestmark = pytest.mark.gpu

TE = {4: 4096, 2: 8192}    # elements per decompress tile (one 256-thread workgroup, 16 KB)
TC = {4: 15360, 2: 30720}  # elements per compress tile (15 data wavefronts x 64 lanes x 64 bytes)


def _sizes(esz):
    t, c = TE[esz], TC[esz]
    return [1, 3, 4, 5, 8, 9, 31, 32, 33, 63, 64, 65, 255, 256, 257, 1023, 1024, 1025,
            t - 1, t, t + 1, 2 * t + 17, 5 * t + 3, 64 * t + 100,
            # compress tiles: a bounded last tile, none (exact multiples), and
            # more tiles than a grid of one workgroup per CU takes in one round;
            # 255-256 tiles take the single-pass kernel (one workgroup per tile,
            # up to one per resident workgroup: 256 on a 256-CU GPU), 257 and
            # more the persistent one
            c - 1, c, c + 1, 2 * c, 3 * c - 1, 3 * c + 1, 255 * c + 7, 256 * c, 257 * c, 257 * c + 1,
            513 * c - 1]


@pytest.mark.parametrize("esz", [4, 2])
@pytest.mark.parametrize("density", [0.0, 0.5, 1.0])
def test_edge_sizes_stream_and_round_trip(esz, density):
    device()
    for n in _sizes(esz):
        x = random_patterns(n, esz, density, seed=n * 3 + esz)
        expect = oracle.zvc_compress(x)
        got, size = gpu_compress(x)
        assert size == expect.size, (n, size, expect.size)
        assert np.array_equal(got, expect), f"stream differs at n={n}"
        out, err = gpu_decompress(expect, n, esz)
        assert err == 0, (n, err)
        assert np.array_equal(out, x), f"round trip differs at n={n}"


@pytest.mark.parametrize("esz", [4, 2])
def test_many_tiles_mixed_density(esz):
    device()
    n = 3_000_017
    rng = np.random.default_rng(7)
    x = random_patterns(n, esz, 0.5, seed=11)
    # whole tiles empty or dense, to exercise zero and full tile aggregates
    t = TE[esz]
    for k in range(0, n // t, 7):
        x[k * t:(k + 1) * t] = 0
    for k in range(3, n // t, 11):
        x[k * t:(k + 1) * t] = rng.integers(1, 2 ** 15, size=t).astype(x.dtype)
    expect = oracle.zvc_compress(x)
    got, size = gpu_compress(x)
    assert size == expect.size
    assert np.array_equal(got, expect)
    out, err = gpu_decompress(expect, n, esz)
    assert err == 0 and np.array_equal(out, x)


def test_single_map_workload():
    device()
    from synth import workload
    x = bits_of(workload("single_map_fp32_1x64x56x56_s0.5"))
    expect = oracle.zvc_compress(x)
    got, size = gpu_compress(x)
    assert np.array_equal(got, expect)
    out, err = gpu_decompress(got, x.size, 4)
    assert err == 0 and np.array_equal(out, x)


def test_specials_survive():
    device()
    x = np.array([0, 0x80000000, 1, 0x007FFFFF, 0x7FC00000, 0x7F800001, 0xFF800000, 0] * 1000,
                 dtype=np.uint32)
    got, _ = gpu_compress(x)
    assert np.array_equal(got, oracle.zvc_compress(x))
    out, err = gpu_decompress(got, x.size, 4)
    assert err == 0 and np.array_equal(out, x)


def test_repeated_runs_are_identical():
    """The order in which workgroups publish their tile aggregates changes
    from run to run; the stream must not."""
    import torch
    import sparse_activation_compression_amd as cdma
    device()
    x = random_patterns(1_000_003, 4, 0.4, seed=21)
    xd = to_device(x)
    first = None
    for _ in range(50):
        dst, nb = cdma.compress(xd)
        torch.cuda.synchronize()
        s = dst[:int(nb.item())].cpu().numpy()
        if first is None:
            first = s
            assert np.array_equal(first, oracle.zvc_compress(x))
        else:
            assert np.array_equal(s, first)


def test_zero_length():
    import torch
    import sparse_activation_compression_amd as cdma
    dev = device()
    x = torch.empty(0, dtype=torch.int32, device=dev)
    dst, nb = cdma.compress(x)
    torch.cuda.synchronize()
    assert int(nb.item()) == 0


def test_decompress_without_size_word():
    device()
    x = random_patterns(100_000, 4, 0.3, seed=5)
    s = oracle.zvc_compress(x)
    out, err = gpu_decompress(s, x.size, 4, exact_size=False, capacity_pad=64)
    assert err == 0 and np.array_equal(out, x)


@pytest.mark.parametrize("esz", [4, 2])
def test_corrupt_streams_report_like_the_oracle(esz):
    device()
    n = 10_007
    x = random_patterns(n, esz, 0.5, seed=99)
    s = oracle.zvc_compress(x)
    W = (n + 31) // 32
    cases = {}
    bad = s.copy()
    bad[4 * (W - 1) + 3] |= 0x80  # mask bit 31 of the last (partial) window
    cases["bit_past_n"] = bad
    cases["truncated"] = s[:-esz]
    cases["too_long"] = np.concatenate([s, np.zeros(16, np.uint8)])
    bad = s.copy()
    bad[0] ^= 0x01  # one value more or fewer than the stream holds
    cases["flipped_mask_bit"] = bad
    cases["masks_only_partly_present"] = s[:4 * W - 6]
    for name, c in cases.items():
        _, want = oracle.zvc_decompress(c, n, esz)
        _, got = gpu_decompress(c, n, esz)
        assert want != 0, name
        assert got == want, (name, got, want)


@pytest.mark.parametrize("algo", ["zvc", "rle", "zvci"])
def test_size_word_beyond_capacity(algo):
    """A valid stream whose size word is right but whose readable buffer is 4
    bytes short of it: the decoder reads nothing past the buffer and reports
    CDMA_E_SIZE (the oracle has no capacity; the size word alone agrees with
    the stream, so this bit comes from the capacity check)."""
    import torch
    import sparse_activation_compression_amd as cdma
    dev = device()
    x = random_patterns(5000, 4, 0.5, seed=123)
    s = {"zvc": oracle.zvc_compress, "rle": oracle.rle_compress, "zvci": oracle.zvci_compress}[algo](x)
    src = torch.from_numpy(s[:-4].copy()).to(dev)
    size = torch.tensor([s.size], dtype=torch.int64, device=dev)
    _, err = cdma.decompress(src, x.size, 4, algo, src_bytes=size)
    torch.cuda.synchronize()
    assert int(err.item()) & oracle.E_SIZE
    _, err = cdma.decompress(torch.from_numpy(s.copy()).to(dev), x.size, 4, algo, src_bytes=size)
    torch.cuda.synchronize()
    assert int(err.item()) == 0


READ_AHEAD = [(4, (1 << 30) + 4097, 0.9, 54), (4, (1 << 30) + 4097, 0.99, 55), (2, (1 << 30) + 8191, 0.95, 57)]


@pytest.mark.parametrize("esz,n,s,seed", READ_AHEAD, ids=[f"esz{e}_s{s}" for e, _, s, _ in READ_AHEAD])
def test_read_ahead_chunks_round_trip(esz, n, s, seed):
    """Outputs over 1 GiB whose stream exceeds what the count pass leaves in
    the memory-side cache but is a small share of the output: the expand
    pass reads each 1 GiB chunk ahead (a ragged last chunk of one or two
    tiles here).  The round trip is bit-exact with and without a size word,
    the size matches the closed form, and a size word one value short is
    reported as CDMA_E_SIZE."""
    import torch
    import sparse_activation_compression_amd as cdma
    from synth import sweep_bits_device
    dev = device()
    print(f"read-ahead esz={esz} n={n} s={s}", flush=True)
    x = sweep_bits_device(n, s, seed, device=dev)
    if esz == 2:
        x = (x >> 16).to(torch.int16)
    nnz = int(torch.count_nonzero(x).item())
    assert 0 < nnz < n // 5
    dst, nb = cdma.compress(x, "zvc")
    size = int(nb.item())
    assert size == 4 * ((n + 31) // 32) + esz * nnz
    out, err = cdma.decompress(dst, n, esz, "zvc", src_bytes=nb)
    torch.cuda.synchronize()
    assert int(err.item()) == 0 and torch.equal(out, x)
    out.fill_(0)
    out2, err2 = cdma.decompress(dst[:size], n, esz, "zvc", out=out)
    torch.cuda.synchronize()
    assert int(err2.item()) == 0 and torch.equal(out2, x)
    short = torch.tensor([size - esz], dtype=torch.int64, device=dev)
    _, err3 = cdma.decompress(dst, n, esz, "zvc", src_bytes=short, out=out)
    torch.cuda.synchronize()
    assert int(err3.item()) & cdma.CDMA_E_SIZE
