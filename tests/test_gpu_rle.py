"""Run-length variant on the GPU against the CPU oracle: byte-exact streams,
bitwise round trips, identical error reports ("Compressing DMA Engine:
Leveraging Activation Sparsity for Training Deep Neural Networks", §V.A
run-length coding, §VII.A 4 KB window)."""

import numpy as np
import pytest

import oracle

from gpu_util import bits_of, device, gpu_compress, gpu_decompress, random_patterns, to_device

pytestmark = pytest.mark.gpu

E = {4: 1024, 2: 2048}  # RLE window in elements (4 KB)
CW = {4: 15, 2: 12}     # windows per compressor tile (one per data wave)


def _sizes(esz):
    e, t, c = E[esz], 4 * E[esz], CW[esz] * E[esz]
    return [1, 2, 3, 31, 32, 33, 100, e - 1, e, e + 1, 2 * e + 5, t - 1, t, t + 1, 3 * t + 17,
            c - 1, c, c + 1, 2 * c + e // 2, 40 * t + 100]


def _markov(n, esz, p_flip, seed):
    rng = np.random.default_rng(seed)
    flips = rng.random(n) < p_flip
    state = np.cumsum(flips) % 2 == 1
    dt = np.uint32 if esz == 4 else np.uint16
    vals = rng.integers(1, 2 ** (8 * esz), size=n, dtype=np.uint64).astype(dt)
    return np.where(state, vals, 0).astype(dt)


def _check(x, esz):
    expect = oracle.rle_compress(x)
    got, size = gpu_compress(x, "rle")
    assert size == expect.size, (x.size, size, expect.size)
    assert np.array_equal(got, expect), f"stream differs at n={x.size}"
    out, err = gpu_decompress(expect, x.size, esz, "rle")
    assert err == 0, (x.size, err)
    assert np.array_equal(out, x), f"round trip differs at n={x.size}"


@pytest.mark.parametrize("esz", [4, 2])
@pytest.mark.parametrize("kind", ["zero", "dense", "iid", "clustered", "alternating"])
def test_edge_sizes(esz, kind):
    device()
    for n in _sizes(esz):
        if kind == "zero":
            x = np.zeros(n, dtype=np.uint32 if esz == 4 else np.uint16)
        elif kind == "dense":
            x = random_patterns(n, esz, 1.0, seed=n)
        elif kind == "iid":
            x = random_patterns(n, esz, 0.5, seed=n + 1)
        elif kind == "clustered":
            x = _markov(n, esz, 0.02, seed=n + 2)
        else:
            x = np.zeros(n, dtype=np.uint32 if esz == 4 else np.uint16)
            x[::2] = 0x3C00 if esz == 2 else 0x3F800000
            x[1::4] = 0x8000 if esz == 2 else 0x80000000
        _check(x, esz)


@pytest.mark.parametrize("esz", [4, 2])
def test_many_tiles(esz):
    device()
    x = _markov(2_500_001, esz, 0.01, seed=3)
    x[E[esz] * 7: E[esz] * 9] = 0
    _check(x, esz)


def test_clustered_activation_map():
    device()
    from synth import clustered_relu
    x = bits_of(clustered_relu((4, 32, 56, 56), 0.6, 2.0, seed=12))
    _check(x, 4)


def test_fp16_clustered_with_specials():
    device()
    from synth import clustered_relu, inject_specials
    x = clustered_relu((2, 64, 56, 56), 0.6, 2.0, seed=13, dtype=np.float16)
    inject_specials(x, 1e-3, seed=14)
    _check(bits_of(x), 2)


def test_repeated_runs_are_identical():
    import torch
    import sparse_activation_compression_amd as cdma
    device()
    x = _markov(1_000_003, 4, 0.05, seed=31)
    xd = to_device(x)
    want = oracle.rle_compress(x)
    for _ in range(30):
        dst, nb = cdma.compress(xd, "rle")
        torch.cuda.synchronize()
        assert np.array_equal(dst[:int(nb.item())].cpu().numpy(), want)


def test_zero_length():
    import torch
    import sparse_activation_compression_amd as cdma
    dev = device()
    x = torch.empty(0, dtype=torch.int32, device=dev)
    dst, nb = cdma.compress(x, "rle")
    torch.cuda.synchronize()
    assert int(nb.item()) == 8 and not dst[:8].cpu().numpy().any()


@pytest.mark.parametrize("esz", [4, 2])
def test_corrupt_streams_report_like_the_oracle(esz):
    device()
    e = E[esz]
    n = 3 * e + 10
    x = _markov(n, esz, 0.03, seed=77)
    s = oracle.rle_compress(x)
    wr = (n + e - 1) // e
    H = 8 * (wr + 1)
    idx = s[:H].view("<u4")
    blk1 = H + 2 * int(idx[1]) + esz * int(idx[wr + 1 + 1])  # block of window 1
    cases = {}
    bad = s.copy()
    bad[H + 2: H + 4].view("<u2")[0] += 1  # window 0, run 1 one longer
    cases["run_length_changed"] = bad
    cases["truncated"] = s[:-2]
    cases["too_long"] = np.concatenate([s, np.zeros(8, np.uint8)])
    bad = s.copy()
    bad[4:8] = np.frombuffer(np.uint32(idx[2] + 2).tobytes(), np.uint8)  # run_off[1] > run_off[2]
    cases["index_decreasing"] = bad
    bad = s.copy()
    bad[blk1 + 2: blk1 + 4] = 0  # window 1: second run zero-length
    cases["zero_length_run"] = bad
    bad = s.copy()
    bad[4 * (wr + 1) + 4: 4 * (wr + 1) + 8] = np.frombuffer(np.uint32(idx[wr + 2] - 1).tobytes(), np.uint8)
    cases["val_off_off_by_one"] = bad
    for name, c in cases.items():
        _, want = oracle.rle_decompress(c, n, esz)
        _, got = gpu_decompress(c, n, esz, "rle")
        assert want != 0, name
        assert got == want, (name, got, want)


@pytest.mark.parametrize("esz", [4, 2])
def test_largest_blocks(esz):
    """Every other element nonzero: the most run entries a window can have,
    so each block has the largest size a stream can hold (4E + 4 bytes for
    32-bit elements with the pad, 3E + 2 for 16-bit)."""
    device()
    e = E[esz]
    for n in (e, 2 * e, 4 * e + 3, 9 * e):
        for first in (0, 1):
            x = np.zeros(n, dtype=np.uint32 if esz == 4 else np.uint16)
            x[first::2] = random_patterns(x[first::2].size, esz, 1.0, seed=n + first)
            _check(x, esz)


@pytest.mark.parametrize("esz", [4, 2])
def test_largest_blocks_cut_in_their_values(esz):
    """Windows of the most run entries, with the stream cut inside the values
    at their end: 16-bit blocks this long are staged only in part and the rest
    of their values come from memory, where bytes past the readable capacity
    must read and report as they do for staged bytes."""
    device()
    e = E[esz]
    n = 2 * e
    x = np.zeros(n, dtype=np.uint32 if esz == 4 else np.uint16)
    x[1::2] = random_patterns(e, esz, 1.0, seed=41)
    s = oracle.rle_compress(x)
    for exact in (True, False):
        out, err = gpu_decompress(s, n, esz, "rle", exact_size=exact, capacity_pad=0 if exact else 64)
        assert err == 0 and np.array_equal(out, x), exact
    # with or without a size word, a cut stream reports E_SIZE only, and the
    # bytes that are missing read as 0 in both decoders
    for cut in (1, 2, 3, esz + 1, 200, 999):
        c = s[:-cut]
        want_out, want = oracle.rle_decompress(c, n, esz)
        assert want == oracle.E_SIZE, cut
        for exact in (True, False):
            out, got = gpu_decompress(c, n, esz, "rle", exact_size=exact)
            assert got == want, (cut, exact, got, want)
            assert np.array_equal(out, want_out), (cut, exact)


def _one_window_stream(esz, runs, nv, seed):
    """A hand-built one-window RLE stream: index, the given run entries, then
    nv random nonzero values (the index claims nv values)."""
    runs = np.asarray(runs, dtype="<u2")
    idx = np.array([0, runs.size, 0, nv], dtype="<u4")
    vals = random_patterns(nv, esz, 1.0, seed=seed)
    return np.concatenate([idx.view(np.uint8), runs.view(np.uint8), vals.view(np.uint8)])


@pytest.mark.parametrize("esz", [4, 2])
def test_oversized_blocks_report_like_the_oracle(esz):
    """Blocks longer than any window that passes the checks can have: the
    decoder stages at most that many bytes, and its error bits must still be
    the oracle's (the checks read run entries only)."""
    device()
    e = E[esz]
    pad = [0] if esz == 4 else []  # a 0 entry after an odd list of 32-bit runs
    cases = [
        # runs sum to e but only half of the claimed values: E_VAL_COUNT
        (e, [0] + [1] * e + pad, e),
        # one run too many: E_RUN_SUM and E_VAL_COUNT
        (e, [0] + [1] * (e + 1), e),
        # an empty run inside the list as well: E_RUN_FORM too
        (e, [0] + [1] * 500 + [0] + [1] * (e - 500), e),
        # a short (last) window
        (e - 5, [0] + [1] * (e - 5), e - 5),
    ]
    bound = 4 * e + 8 if esz == 4 else 3 * e + 6
    for k, (n, runs, nv) in enumerate(cases):
        assert 2 * len(runs) + esz * nv > bound and len(runs) <= n + 2
        s = _one_window_stream(esz, runs, nv, seed=900 + k)
        _, want = oracle.rle_decompress(s, n, esz)
        _, got = gpu_decompress(s, n, esz, "rle")
        assert want != 0, k
        assert got == want, (k, got, want)


def test_stream_cut_inside_a_run_entry():
    """A 16-bit stream whose size ends one byte into a run entry: the byte that
    is there counts and the missing one reads as 0, as in the oracle (found by
    the corruption fuzz test)."""
    device()
    s = np.frombuffer(bytes.fromhex("00000000090000000000000004000000160001000c000100270001000c0001"),
                      dtype=np.uint8).copy()
    _, want = oracle.rle_decompress(s, 370, 2)
    _, got = gpu_decompress(s, 370, 2, "rle")
    assert want != 0 and got == want, (got, want)
