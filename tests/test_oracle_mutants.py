"""Plant plausible mistakes in a copy of the oracle and check the pins catch them.

Each mutant is oracle.c with one textual edit (a swapped bit order, a dropped
term, an off-by-one, a float-style zero test ...), compiled with gcc into a
temporary library.  The pins run against it must fail for every mutant; the
pins used are the ones that do not depend on the oracle itself (hand-worked
streams, closed-form sizes with brute-force counts, the page's 32x all-zero
window, bitwise round trips of special patterns).
"""

import os

import numpy as np
import pytest

import oracle

import golden_io

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "mask_bit_order_reversed": ("mask |= (uint32_t)1 << i;", "mask |= (uint32_t)1 << (31 - i);"),
    "mask_polarity_inverted": ("if (idx < n && elem(src, idx, esz) != 0)", "if (idx < n && elem(src, idx, esz) == 0)"),
    "last_value_dropped": ("for (uint64_t idx = 0; idx < n; idx++) {\n        uint64_t v = elem(src, idx, esz);",
                           "for (uint64_t idx = 0; idx + 1 < n; idx++) {\n        uint64_t v = elem(src, idx, esz);"),
    "window_count_floor": ("uint64_t W = (n + 31) / 32;\n    /* masks", "uint64_t W = n / 32;\n    /* masks"),
    "size_esz_fixed_4": ("return 4 * ((n + 31) / 32) + (uint64_t)esz * nnz;", "return 4 * ((n + 31) / 32) + 4 * nnz;"),
    "negative_zero_is_zero": ("static uint64_t elem(const void *src, uint64_t i, int esz)\n{\n    return get_le(",
                              "static uint64_t elem(const void *src, uint64_t i, int esz)\n{\n    return ~(1ull << (8 * esz - 1)) & get_le("),
    "rle_no_padding": ("return (esz == 4 && (r & 1)) ? r + 1 : r;", "return r;"),
    "rle_nonzero_run_first": ("int kind = 0; /* 0 = zero run", "int kind = 1; /* 0 = zero run"),
    "rle_total_off_by_one": ("put_le(dst + 4 * Wr, ent, 4);", "put_le(dst + 4 * Wr, ent + 1, 4);"),
    "rle_window_8k": ("return 4096u / (unsigned)esz;", "return 8192u / (unsigned)esz;"),
    "rle_values_before_runs": ("uint64_t vpos = rpos + 2 * p;", "uint64_t vpos = rpos;"),
    "zvc_decode_bit_reversed": ("if ((mask >> (idx % 32)) & 1u)", "if ((mask >> (31 - idx % 32)) & 1u)"),
    "zvc_past_n_check_shifted": ("if (last >> (n % 32))", "if (last >> (n % 32 + 1))"),
    "zvci_index_counts_windows": ("put_le(dst + 4 * ((32 * w) / E), nnz, 4);", "put_le(dst + 4 * ((32 * w) / E), w, 4);"),
    "zvci_mask_bits_reversed": ("mask <<= 1;\n            if (idx < n && elem(src, idx, esz))\n                mask |= 1u;",
                                "mask >>= 1;\n            if (idx < n && elem(src, idx, esz))\n                mask |= 0x80000000u;"),
    "zvci_decode_block_skips_masks": ("uint64_t pos = hdr + 4 * b * wpb + (uint64_t)esz * v0, count = 0;",
                                      "uint64_t pos = hdr + (uint64_t)esz * v0, count = 0;"),
    "relu_nan_not_kept": ("uint64_t y = (sign && !is_nan) ? 0 : v;", "uint64_t y = sign ? 0 : v;"),
    "relu_inf_taken_for_nan": ("&& mantissa != 0;", "&& mantissa == 0;"),
    "relu_bf16_with_fp16_fields": ("else if (fmt == 2) { esz = 2; exp_bits = 8; man_bits = 7; }",
                                   "else if (fmt == 2) { esz = 2; exp_bits = 5; man_bits = 10; }"),
    "relu_sign_bit_one_low": ("uint64_t sign = v >> (exp_bits + man_bits);",
                              "uint64_t sign = v >> (exp_bits + man_bits - 1);"),
}


def _relu_pins_pass(lib) -> bool:
    from test_oracle_pins import RELU_HAND, relu_numpy
    for fmt, table in RELU_HAND.items():
        dt = np.uint32 if fmt == oracle.FMT_F32 else np.uint16
        x = np.array([a for a, _ in table], dtype=dt)
        if not np.array_equal(oracle.relu(x, fmt, lib), np.array([b for _, b in table], dtype=dt)):
            return False
    for fmt in (oracle.FMT_F16, oracle.FMT_BF16):
        x = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
        if not np.array_equal(oracle.relu(x, fmt, lib), relu_numpy(x, fmt)):
            return False
    return True


def _pins_pass(lib) -> bool:
    """True iff every independent pin passes against ``lib``."""
    try:
        for c in golden_io.all_cases():
            comp = {"zvc": oracle.zvc_compress, "rle": oracle.rle_compress,
                    "zvci": oracle.zvci_compress}[c["algo"]]
            dec = {"zvc": oracle.zvc_decompress, "rle": oracle.rle_decompress,
                   "zvci": oracle.zvci_decompress}[c["algo"]]
            if bytes(comp(c["x"], lib)) != bytes(c["stream"]):
                return False
            out, err = dec(c["stream"], c["n"], c["esz"], lib)
            if err != 0 or not np.array_equal(out, c["x"]):
                return False
        # all-zero window: 32x
        if oracle.zvc_compress(np.zeros(32, np.uint32), lib).size != 4:
            return False
        # closed form and round trip on random patterns with specials
        rng = np.random.default_rng(1)
        for esz in (2, 4):
            dt = np.uint32 if esz == 4 else np.uint16
            for n in (7, 33, 1000, 5000):
                x = rng.integers(0, 2 ** (8 * esz), size=n, dtype=np.uint64).astype(dt)
                x[rng.random(n) < 0.5] = 0
                x[::17] = 0x80000000 if esz == 4 else 0x8000
                nnz = sum(1 for v in x.tolist() if v != 0)
                if oracle.zvc_compress(x, lib).size != 4 * ((n + 31) // 32) + esz * nnz:
                    return False
                for comp, dec in ((oracle.zvc_compress, oracle.zvc_decompress),
                                  (oracle.rle_compress, oracle.rle_decompress)):
                    out, err = dec(comp(x, lib), n, esz, lib)
                    if err != 0 or not np.array_equal(out, x):
                        return False
        # a mask bit past n must be reported
        bad = oracle.zvc_compress(np.array([1, 0, 0], np.uint32), lib)
        bad[0] |= 0x08
        bad = np.concatenate([bad, bad[4:8]])
        if not (oracle.zvc_decompress(bad, 3, 4, lib)[1] & oracle.E_MASK_PAST_N):
            return False
        if not _relu_pins_pass(lib):
            return False
    except Exception:
        return False
    return True


def test_unmutated_oracle_passes_the_pin_suite(tmp_path):
    path = oracle.build(SRC, str(tmp_path / "lib_clean.so"))
    assert _pins_pass(oracle.load(path))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    mpath = tmp_path / f"{name}.c"
    mpath.write_text(src.replace(old, new))
    lib = oracle.load(oracle.build(str(mpath), str(tmp_path / f"{name}.so"), extra=("-w",)))
    assert not _pins_pass(lib), f"planted mistake {name} went unnoticed"
