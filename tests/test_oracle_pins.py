"""Pins for the CPU oracle, each fixed by something other than the oracle.

Sources of truth used here:
* hand-worked streams (tests/golden/), derived by hand from "Compressing DMA
  Engine: Leveraging Activation Sparsity for Training Deep Neural Networks",
  §V.A Compression Algorithm and §VII.A Compression Efficiency;
* the page's own figure for an all-zero window (§V.A: 32x for 32 four-byte
  values, one all-zero mask word -- which also fixes the mask polarity);
* closed forms: ZVC size = 4*ceil(n/32) + esz*nnz, RLE size = 8(Wr+1) +
  2*sum(padded runs) + esz*nnz, with nnz and runs counted by brute force;
* the page's claim that ZVC's ratio does not depend on the layout of the
  activations while run-length coding's does (§VII.A);
* the library-routine form (np.packbits + boolean compaction, np.diff runs);
* exhaustive enumeration of every zero/nonzero pattern for tiny n;
* bitwise round trips over random and special bit patterns.
"""

import itertools

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from oracle import np_forms

import golden_io

CASES = golden_io.all_cases()


# --------------------------------------------------------------------------
# hand-worked streams
# --------------------------------------------------------------------------

C_COMP = {"zvc": oracle.zvc_compress, "rle": oracle.rle_compress, "zvci": oracle.zvci_compress}
C_DEC = {"zvc": oracle.zvc_decompress, "rle": oracle.rle_decompress, "zvci": oracle.zvci_decompress}
NP_COMP = {"zvc": np_forms.zvc_compress, "rle": np_forms.rle_compress, "zvci": np_forms.zvci_compress}


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_golden_stream_c_oracle(case):
    s = C_COMP[case["algo"]](case["x"])
    assert s.size == case["size"]
    assert bytes(s) == bytes(case["stream"])


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_golden_stream_numpy_form(case):
    assert bytes(NP_COMP[case["algo"]](case["x"])) == bytes(case["stream"])


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_golden_decode(case):
    out, err = C_DEC[case["algo"]](case["stream"], case["n"], case["esz"])
    assert err == 0
    assert np.array_equal(out, case["x"])
    if case["algo"] != "zvci":
        ndec = np_forms.zvc_decompress if case["algo"] == "zvc" else np_forms.rle_decompress
        assert np.array_equal(ndec(case["stream"], case["n"], case["esz"]), case["x"])


# --------------------------------------------------------------------------
# the page's all-zero window figure
# --------------------------------------------------------------------------

def test_all_zero_window_is_one_zero_mask_32x():
    x = np.zeros(32, dtype=np.float32)
    s = oracle.zvc_compress(x)
    assert s.size == 4 and not s.any()
    assert x.nbytes / s.size == 32.0


def test_all_zero_many_windows_32x():
    x = np.zeros(32 * 1000, dtype=np.float32)
    assert x.nbytes / oracle.zvc_compress(x).size == 32.0


# --------------------------------------------------------------------------
# closed forms with brute-force counts
# --------------------------------------------------------------------------

def _brute_nnz(b):
    return sum(1 for v in b.tolist() if v != 0)


@pytest.mark.parametrize("esz", [2, 4])
@pytest.mark.parametrize("n", [0, 1, 5, 31, 32, 33, 63, 64, 65, 1000, 4097])
@pytest.mark.parametrize("dens", [0.0, 0.3, 1.0])
def test_zvc_size_closed_form(esz, n, dens):
    rng = np.random.default_rng(n * 7 + esz)
    dt = np.uint32 if esz == 4 else np.uint16
    x = rng.integers(1, 2 ** (8 * esz), size=n, dtype=np.uint64).astype(dt)
    x[rng.random(n) >= dens] = 0
    expect = 4 * ((n + 31) // 32) + esz * _brute_nnz(x)
    assert oracle.zvc_compress(x).size == expect
    assert oracle.zvc_size(x) == expect


def _brute_runs(nzlist):
    """Alternating run count, zero run first, by walking the list."""
    runs, cur, kind = [], 0, False
    for v in nzlist:
        if v == kind:
            cur += 1
        else:
            runs.append(cur)
            kind, cur = v, 1
    runs.append(cur)
    return runs


@pytest.mark.parametrize("esz", [2, 4])
@pytest.mark.parametrize("n", [1, 2, 3, 1023, 1024, 1025, 2047, 2048, 2049, 5000])
def test_rle_size_closed_form(esz, n):
    rng = np.random.default_rng(n * 11 + esz)
    dt = np.uint32 if esz == 4 else np.uint16
    # clustered indicator: a two-state Markov chain
    nz = np.zeros(n, dtype=bool)
    state = False
    for i in range(n):
        if rng.random() < 0.05:
            state = not state
        nz[i] = state
    x = np.where(nz, rng.integers(1, 2 ** (8 * esz), size=n, dtype=np.uint64), 0).astype(dt)
    E = 4096 // esz
    wr = (n + E - 1) // E
    ent = 0
    for w in range(wr):
        r = len(_brute_runs([bool(v) for v in nz[w * E:(w + 1) * E]]))
        ent += r + (r % 2 if esz == 4 else 0)
    expect = 8 * (wr + 1) + 2 * ent + esz * _brute_nnz(x)
    assert oracle.rle_compress(x).size == expect
    assert oracle.rle_size(x) == expect


def test_rle_runs_brute_force_small():
    rng = np.random.default_rng(5)
    for _ in range(200):
        n = int(rng.integers(1, 40))
        x = (rng.random(n) < 0.5).astype(np.uint32) * 0x3F800000
        s = oracle.rle_compress(x)
        p = int(s[4:8].view("<u4")[0])
        runs = s[16:16 + 2 * p].view("<u2").tolist()
        want = _brute_runs([bool(v) for v in x])
        if len(want) % 2:
            want = want + [0]
        assert runs == want


# --------------------------------------------------------------------------
# exhaustive tiny inputs
# --------------------------------------------------------------------------

@pytest.mark.parametrize("esz", [2, 4])
def test_exhaustive_patterns_small_n(esz):
    dt = np.uint32 if esz == 4 else np.uint16
    for n in range(1, 11):
        for pat in itertools.product((0, 1), repeat=n):
            x = np.array([(i + 1) * 0x101 if p else 0 for i, p in enumerate(pat)], dtype=dt)
            for comp, ncomp, dec in ((oracle.zvc_compress, np_forms.zvc_compress, oracle.zvc_decompress),
                                     (oracle.rle_compress, np_forms.rle_compress, oracle.rle_decompress)):
                s = comp(x)
                assert bytes(s) == bytes(ncomp(x))
                out, err = dec(s, n, esz)
                assert err == 0 and np.array_equal(out, x)


# --------------------------------------------------------------------------
# layout invariance (ZVC) vs layout sensitivity (RLE), §VII.A
# --------------------------------------------------------------------------

def test_zvc_size_is_layout_invariant_rle_is_not():
    from synth import clustered_relu
    x = clustered_relu((2, 8, 28, 28), 0.7, 2.0, seed=9)
    nchw = x.reshape(-1)
    nhwc = np.ascontiguousarray(x.transpose(0, 2, 3, 1)).reshape(-1)
    perm = np.random.default_rng(3).permutation(nchw)
    z = {k: oracle.zvc_compress(v).size for k, v in (("nchw", nchw), ("nhwc", nhwc), ("perm", perm))}
    r = {k: oracle.rle_compress(v).size for k, v in (("nchw", nchw), ("nhwc", nhwc), ("perm", perm))}
    assert len(set(z.values())) == 1
    assert len(set(r.values())) == 3
    assert r["nchw"] < r["perm"]


# --------------------------------------------------------------------------
# cross-form invariants
# --------------------------------------------------------------------------

@pytest.mark.parametrize("esz", [2, 4])
def test_rle_and_zvc_carry_the_same_values_and_bitmap(esz):
    from synth import clustered_relu
    dt = np.float32 if esz == 4 else np.float16
    x = clustered_relu((1, 4, 40, 40), 0.6, 2.0, seed=11, dtype=dt).reshape(-1)
    b = x.view(np.uint32 if esz == 4 else np.uint16)
    n = b.size
    z = oracle.zvc_compress(b)
    W = (n + 31) // 32
    zvals = z[4 * W:]
    r = oracle.rle_compress(b)
    E = 4096 // esz
    wr = (n + E - 1) // E
    idx = r[:8 * (wr + 1)].view("<u4")
    run_off, val_off = idx[:wr + 1], idx[wr + 1:]
    rvals, bitmap = [], np.zeros(n, dtype=bool)
    for w in range(wr):
        p, nv = int(run_off[w + 1] - run_off[w]), int(val_off[w + 1] - val_off[w])
        at = 8 * (wr + 1) + 2 * int(run_off[w]) + esz * int(val_off[w])
        runs = r[at:at + 2 * p].view("<u2").astype(int)
        pos = w * E
        for k, ln in enumerate(runs):
            if k % 2:
                bitmap[pos:pos + ln] = True
            pos += ln
        rvals.append(r[at + 2 * p: at + 2 * p + esz * nv])
    assert bytes(np.concatenate(rvals)) == bytes(zvals)
    masks = z[:4 * W].view("<u4")
    unpacked = np.unpackbits(masks.view(np.uint8), bitorder="little")[:n].astype(bool)
    assert np.array_equal(unpacked, bitmap)


@pytest.mark.parametrize("algo", ["zvc", "rle"])
def test_encode_of_decode_is_identity(algo):
    rng = np.random.default_rng(17)
    x = rng.integers(0, 3, size=3001).astype(np.uint32) * 0x40000001
    comp = oracle.zvc_compress if algo == "zvc" else oracle.rle_compress
    dec = oracle.zvc_decompress if algo == "zvc" else oracle.rle_decompress
    s = comp(x)
    out, err = dec(s, x.size, 4)
    assert err == 0
    assert bytes(comp(out)) == bytes(s)


# --------------------------------------------------------------------------
# bitwise round trips, including patterns a float compare would mangle
# --------------------------------------------------------------------------

_special32 = st.sampled_from([0, 0x80000000, 1, 0x007FFFFF, 0x80000001, 0x7FC00000,
                              0x7F800001, 0x7F800000, 0xFF800000, 0x3F800000])
_special16 = st.sampled_from([0, 0x8000, 1, 0x03FF, 0x8001, 0x7E00, 0x7C01, 0x7C00, 0xFC00, 0x3C00])


@settings(max_examples=150, deadline=None)
@given(st.lists(st.one_of(_special32, st.integers(0, 2 ** 32 - 1)), max_size=2500),
       st.sampled_from(["zvc", "rle"]))
def test_round_trip_fp32_patterns(vals, algo):
    x = np.array(vals, dtype=np.uint32)
    comp = oracle.zvc_compress if algo == "zvc" else oracle.rle_compress
    dec = oracle.zvc_decompress if algo == "zvc" else oracle.rle_decompress
    s = comp(x)
    out, err = dec(s, x.size, 4)
    assert err == 0 and np.array_equal(out, x)
    ncomp = np_forms.zvc_compress if algo == "zvc" else np_forms.rle_compress
    assert bytes(ncomp(x)) == bytes(s)


@settings(max_examples=150, deadline=None)
@given(st.lists(st.one_of(_special16, st.integers(0, 2 ** 16 - 1)), max_size=5000),
       st.sampled_from(["zvc", "rle"]))
def test_round_trip_fp16_patterns(vals, algo):
    x = np.array(vals, dtype=np.uint16)
    comp = oracle.zvc_compress if algo == "zvc" else oracle.rle_compress
    dec = oracle.zvc_decompress if algo == "zvc" else oracle.rle_decompress
    s = comp(x)
    out, err = dec(s, x.size, 2)
    assert err == 0 and np.array_equal(out, x)
    ncomp = np_forms.zvc_compress if algo == "zvc" else np_forms.rle_compress
    assert bytes(ncomp(x)) == bytes(s)


def test_negative_zero_is_kept():
    x = np.array([0.0, -0.0, 0.0, 1.0], dtype=np.float32)
    s = oracle.zvc_compress(x)
    assert s.size == 4 + 8
    out, _ = oracle.zvc_decompress(s, 4, 4)
    assert out.tolist() == [0, 0x80000000, 0, 0x3F800000]


# --------------------------------------------------------------------------
# statistics: iid zeros give the expected ratio (a loose check)
# --------------------------------------------------------------------------

def test_iid_ratio_matches_expectation():
    from synth import iid_relu
    x = iid_relu(1 << 20, 0.5, seed=1)
    ratio = x.nbytes / oracle.zvc_compress(x).size
    assert abs(ratio - 4 / (0.125 + 4 * 0.5)) < 0.01


# --------------------------------------------------------------------------
# corrupt streams are reported
# --------------------------------------------------------------------------

def test_zvc_corruptions():
    x = np.array([0, 5, 0, 7, 0, 0, 9], dtype=np.uint32)
    s = oracle.zvc_compress(x)
    bad = s.copy()
    bad[0] |= 0x80  # bit 7 is past n = 7
    assert oracle.zvc_decompress(bad, 7, 4)[1] & oracle.E_MASK_PAST_N
    assert oracle.zvc_decompress(s[:-1], 7, 4)[1] == oracle.E_SIZE
    assert oracle.zvc_decompress(np.concatenate([s, s[:4]]), 7, 4)[1] == oracle.E_SIZE
    bad = s.copy()
    bad[0] &= 0xFD  # drop element 1: one value too many
    assert oracle.zvc_decompress(bad, 7, 4)[1] == oracle.E_SIZE
    assert oracle.zvc_decompress(s[:2], 7, 4)[1] == oracle.E_SIZE


def test_rle_corruptions():
    x = np.zeros(1030, dtype=np.uint32)
    x[5:8] = 1
    x[1000:1026] = 2
    s = oracle.rle_compress(x)
    assert oracle.rle_decompress(s, 1030, 4)[1] == 0
    # run 1 of window 0 from 3 to 4: runs no longer sum to 1024, one nonzero too many
    bad = s.copy()
    bad[24 + 2] = 4
    e = oracle.rle_decompress(bad, 1030, 4)[1]
    assert e & oracle.E_RUN_SUM and e & oracle.E_VAL_COUNT
    # a zero-length run that is not the first
    bad = s.copy()
    bad[24 + 2] = 0
    assert oracle.rle_decompress(bad, 1030, 4)[1] & oracle.E_RUN_FORM
    # index decreasing
    bad = s.copy()
    bad[4] = 9  # run_off[1] = 9 > run_off[2] = 8
    assert oracle.rle_decompress(bad, 1030, 4)[1] & oracle.E_INDEX
    # truncation
    assert oracle.rle_decompress(s[:-2], 1030, 4)[1] & oracle.E_SIZE
    # odd entry count for 4-byte elements
    y = np.zeros(8, dtype=np.uint32)
    t = oracle.rle_compress(y)  # runs [8, 0]: p = 2
    bad = t.copy()
    bad[4] = 1  # run_off[1] = 1 (odd)
    assert oracle.rle_decompress(bad, 8, 4)[1] & oracle.E_RUN_FORM


# --------------------------------------------------------------------------
# offload image = chunk streams back to back
# --------------------------------------------------------------------------

def test_offload_stream_is_chunk_concatenation():
    from synth import iid_relu
    x = iid_relu(10000, 0.6, seed=4)
    img, sizes = oracle.offload_stream(x, 4096)
    assert len(sizes) == 3 and sum(sizes) == img.size
    b = x.view(np.uint32)
    lo = 0
    for k, sz in enumerate(sizes):
        part = img[lo:lo + sz]
        out, err = oracle.zvc_decompress(part, min(4096, b.size - 4096 * k), 4)
        assert err == 0 and np.array_equal(out, b[4096 * k: 4096 * (k + 1)])
        lo += sz


# --------------------------------------------------------------------------
# restore (prefetch) = every chunk decoded on its own, in order
# --------------------------------------------------------------------------

@pytest.mark.parametrize("algo", ["zvc", "rle"])
@pytest.mark.parametrize("esz", [4, 2])
def test_restore_inverts_the_offload_image(algo, esz):
    """The input itself is the expected value: restore(offload(x)) == x."""
    x = np.random.default_rng(esz).integers(1, 2 ** (8 * esz), size=3 * 4096 + 77, dtype=np.uint64)
    x = x.astype(np.uint32 if esz == 4 else np.uint16)
    x[np.random.default_rng(1).random(x.size) < 0.55] = 0
    x[100:3000] = 0  # a long zero run across a window edge
    img, sizes = oracle.offload_stream(x, 4096, algo)
    out, err = oracle.restore(img, sizes, x.size, esz, 4096, algo)
    assert err == 0 and np.array_equal(out, x)


def test_restore_reports_a_bad_chunk():
    """A mask bit added to chunk 1 claims a value the stream does not hold:
    the stream size no longer matches its masks (§V.A: the nonzero count is
    the mask's popcount), so the size error bit must be set."""
    x = np.zeros(3 * 4096, dtype=np.uint32)
    x[::7] = 5
    img, sizes = oracle.offload_stream(x, 4096)
    bad = img.copy()
    first_mask_of_chunk1 = sizes[0]
    assert bad[first_mask_of_chunk1] & 0x2 == 0  # element 4097 of x is zero
    bad[first_mask_of_chunk1] |= 0x2
    out, err = oracle.restore(bad, sizes, x.size, 4, 4096)
    assert err & oracle.E_SIZE
    assert np.array_equal(out[:4096], x[:4096]) and np.array_equal(out[8192:], x[8192:])


# --------------------------------------------------------------------------
# ReLU of the producing layer (fused epilogue): max(x, 0) on IEEE patterns
# --------------------------------------------------------------------------

# (pattern, ReLU pattern) worked by hand from the IEEE-754 field layouts:
# binary32 = 1 sign, 8 exponent, 23 mantissa bits; binary16 = 1/5/10;
# bfloat16 = 1/8/7 (the top half of a binary32).
RELU_HAND = {
    oracle.FMT_F32: [(0xBF800000, 0), (0x40000000, 0x40000000), (0x80000000, 0), (0x00000000, 0),
                     (0x7FC00000, 0x7FC00000), (0xFFC00001, 0xFFC00001), (0xFF800000, 0),
                     (0x7F800000, 0x7F800000), (0x80000001, 0), (0x00000001, 0x00000001),
                     (0xFF800001, 0xFF800001), (0xC2C80000, 0)],
    oracle.FMT_F16: [(0xBC00, 0), (0x3C00, 0x3C00), (0x8000, 0), (0x7E00, 0x7E00), (0xFE01, 0xFE01),
                     (0xFC00, 0), (0x7C00, 0x7C00), (0x8001, 0), (0x0001, 0x0001), (0xFC01, 0xFC01),
                     (0xFF80, 0xFF80)],
    oracle.FMT_BF16: [(0xBF80, 0), (0x3F80, 0x3F80), (0x8000, 0), (0x7FC0, 0x7FC0), (0xFFC1, 0xFFC1),
                      (0xFF80, 0), (0x7F80, 0x7F80), (0x8001, 0), (0x0001, 0x0001), (0xFF81, 0xFF81),
                      (0xFC00, 0)],
}


def relu_numpy(bits: np.ndarray, fmt: int) -> np.ndarray:
    """The same rule with library float compares: keep x where x is NaN or
    x > 0, else +0.0 (bf16 widened exactly to binary32 by a 16-bit shift)."""
    if fmt == oracle.FMT_F32:
        f = bits.view(np.float32)
    elif fmt == oracle.FMT_F16:
        f = bits.view(np.float16)
    else:
        f = (bits.astype(np.uint32) << 16).view(np.float32)
    with np.errstate(invalid="ignore"):
        keep = np.isnan(f) | (f > 0)
    return np.where(keep, bits, np.zeros_like(bits))


@pytest.mark.parametrize("fmt", [oracle.FMT_F32, oracle.FMT_F16, oracle.FMT_BF16])
def test_relu_hand_worked(fmt):
    dt = np.uint32 if fmt == oracle.FMT_F32 else np.uint16
    x = np.array([a for a, _ in RELU_HAND[fmt]], dtype=dt)
    want = np.array([b for _, b in RELU_HAND[fmt]], dtype=dt)
    assert np.array_equal(oracle.relu(x, fmt), want)
    assert np.array_equal(relu_numpy(x, fmt), want)


@pytest.mark.parametrize("fmt", [oracle.FMT_F16, oracle.FMT_BF16])
def test_relu_every_16bit_pattern(fmt):
    x = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    assert np.array_equal(oracle.relu(x, fmt), relu_numpy(x, fmt))


def test_relu_fp32_sampled_and_all_exponents():
    rng = np.random.default_rng(5)
    x = rng.integers(0, 1 << 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    # every exponent with mantissas 0, 1 and all ones, both signs
    e = np.arange(256, dtype=np.uint32) << 23
    extra = np.concatenate([e, e | 1, e | 0x7FFFFF])
    x = np.concatenate([x, extra, extra | 0x80000000])
    assert np.array_equal(oracle.relu(x, oracle.FMT_F32), relu_numpy(x, oracle.FMT_F32))


def test_relu_then_zvc_is_the_stream_of_the_relu_map():
    """The fused epilogue's expected stream: ZVC of ReLU(x); its size obeys the
    closed form with nnz counted by numpy's float compare."""
    rng = np.random.default_rng(8)
    x = rng.standard_normal(10000).astype(np.float32)
    y = oracle.relu(x.view(np.uint32), oracle.FMT_F32)
    nnz = int(np.count_nonzero(x > 0))
    assert oracle.zvc_compress(y).size == 4 * ((x.size + 31) // 32) + 4 * nnz


# --------------------------------------------------------------------------
# interleaved ZVC (per window: mask then values; 4 KB block index)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("esz", [4, 2])
@pytest.mark.parametrize("n", [1, 31, 32, 33, 1023, 1024, 1025, 2048, 2049, 5000, 3 * 2048 + 7])
def test_zvci_c_equals_rearranged_zvc_and_closed_form(esz, n):
    """The interleaved stream is the masks-then-values stream rearranged
    window by window (np_forms builds it from the packbits form), and its size
    is 4(Wr+1) + 4*ceil(n/32) + esz*nnz with nnz counted by numpy."""
    rng = np.random.default_rng(n * 7 + esz)
    dt = np.uint32 if esz == 4 else np.uint16
    x = rng.integers(1, 2 ** (8 * esz), size=n, dtype=np.uint64).astype(dt)
    x[rng.random(n) < 0.6] = 0
    x[n // 3: n // 2] = 0
    s = oracle.zvci_compress(x)
    assert bytes(s) == bytes(np_forms.zvci_compress(x))
    E = 4096 // esz
    nnz = int(np.count_nonzero(x))
    assert s.size == 4 * ((n + E - 1) // E + 1) + 4 * ((n + 31) // 32) + esz * nnz == oracle.zvci_size(x)
    # same masks and values as the masks-then-values stream, so the same payload size
    assert s.size - 4 * ((n + E - 1) // E + 1) == oracle.zvc_compress(x).size
    out, err = oracle.zvci_decompress(s, n, esz)
    assert err == 0 and np.array_equal(out, x)


def test_zvci_round_trips_special_patterns():
    x = np.array([0x80000000, 0, 1, 0x7FC00001, 0xFF800000, 0, 0x00800000] * 400, dtype=np.uint32)
    out, err = oracle.zvci_decompress(oracle.zvci_compress(x), x.size, 4)
    assert err == 0 and np.array_equal(out, x)


def test_zvci_corruptions_are_reported():
    x = np.zeros(3000, dtype=np.uint32)
    x[::5] = 9
    s = oracle.zvci_compress(x)  # Wr = 3 blocks, index = 16 bytes
    n = x.size
    bad = s.copy()
    bad[4:8] = np.frombuffer(np.uint32(1 << 20).tobytes(), np.uint8)  # val_off[1] too large
    assert oracle.zvci_decompress(bad, n, 4)[1] & oracle.E_INDEX or \
        oracle.zvci_decompress(bad, n, 4)[1] & oracle.E_VAL_COUNT
    bad = s.copy()
    bad[16] |= 0x02  # window 0 claims element 1, which is zero: one value too many
    assert oracle.zvci_decompress(bad, n, 4)[1] & oracle.E_VAL_COUNT
    assert oracle.zvci_decompress(s[:-4], n, 4)[1] & oracle.E_SIZE
    y = np.array([5, 0, 0], dtype=np.uint32)
    t = oracle.zvci_compress(y)  # index [0, 1], mask 0x1, value 5
    bad = np.concatenate([t, t[-4:]])
    bad[8] |= 0x10  # bit 4 of the only window: element 4 >= n
    assert oracle.zvci_decompress(bad, 3, 4)[1] & oracle.E_MASK_PAST_N
