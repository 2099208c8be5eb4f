"""Library-routine form of the codec -- TEST INFRASTRUCTURE ONLY.

The same definition as ``oracle.c``, written with numpy primitives instead of
loops, so that the two oracles can check each other:

* ZVC ("Compressing DMA Engine: Leveraging Activation Sparsity for Training
  Deep Neural Networks", §V.A): the 32-bit per-window masks are exactly
  ``np.packbits(nonzero, bitorder='little')`` read as little-endian u32, and
  the values section is boolean-mask compaction ``bits[bits != 0]``.
* RLE (§V.A, 4 KB window of §VII.A): the run boundaries of a window are the
  change points of its nonzero indicator with a virtual zero in front
  (``np.diff``); run lengths are the gaps between boundaries.
"""

from __future__ import annotations

import numpy as np


def _bits(x):
    x = np.ascontiguousarray(x).reshape(-1)
    return x.view(np.uint32 if x.dtype.itemsize == 4 else np.uint16)


def zvc_compress(x) -> np.ndarray:
    b = _bits(x)
    n = b.size
    nz = b != 0
    padded = np.zeros(((n + 31) // 32) * 32, dtype=bool)
    padded[:n] = nz
    masks = np.packbits(padded, bitorder="little").view("<u4")
    vals = b[nz].astype(b.dtype.newbyteorder("<"))
    return np.concatenate([masks.view(np.uint8), vals.view(np.uint8)])


def zvc_decompress(stream, n: int, esz: int) -> np.ndarray:
    s = np.asarray(stream, dtype=np.uint8)
    W = (n + 31) // 32
    masks = s[: 4 * W]
    nz = np.unpackbits(masks, bitorder="little")[:n].astype(bool)
    dt = np.dtype("<u4" if esz == 4 else "<u2")
    vals = s[4 * W:].view(dt)
    out = np.zeros(n, dtype=dt)
    out[nz] = vals[: int(nz.sum())]
    return out


def window_runs(nz: np.ndarray) -> np.ndarray:
    """Alternating run lengths (zero run first) of one window's indicator."""
    ch = np.flatnonzero(np.diff(np.concatenate([[0], nz.astype(np.int8)])))
    bounds = np.concatenate([[0], ch, [nz.size]])
    return np.diff(bounds).astype(np.uint16)


def rle_compress(x) -> np.ndarray:
    b = _bits(x)
    n, esz = b.size, b.dtype.itemsize
    E = 4096 // esz
    wr = (n + E - 1) // E
    dt = b.dtype.newbyteorder("<")
    blocks, run_off, val_off = [], [0], [0]
    for w in range(wr):
        seg = b[w * E: (w + 1) * E]
        nz = seg != 0
        runs = window_runs(nz)
        if esz == 4 and runs.size % 2 == 1:
            runs = np.concatenate([runs, np.zeros(1, np.uint16)])
        blocks.append(runs.astype("<u2").view(np.uint8))
        blocks.append(seg[nz].astype(dt).view(np.uint8))
        run_off.append(run_off[-1] + runs.size)
        val_off.append(val_off[-1] + int(nz.sum()))
    index = np.concatenate([np.asarray(run_off, "<u4"), np.asarray(val_off, "<u4")])
    return np.concatenate([index.view(np.uint8)] + blocks)


def rle_decompress(stream, n: int, esz: int) -> np.ndarray:
    s = np.asarray(stream, dtype=np.uint8)
    E = 4096 // esz
    wr = (n + E - 1) // E
    idx = s[: 8 * (wr + 1)].view("<u4")
    run_off, val_off = idx[: wr + 1], idx[wr + 1:]
    dt = np.dtype("<u4" if esz == 4 else "<u2")
    out = np.zeros(n, dtype=dt)
    base = 8 * (wr + 1)
    for w in range(wr):
        p = int(run_off[w + 1] - run_off[w])
        nv = int(val_off[w + 1] - val_off[w])
        at = base + 2 * int(run_off[w]) + esz * int(val_off[w])
        runs = s[at: at + 2 * p].view("<u2").astype(np.int64)
        if esz == 4 and p % 2 == 0 and p > 0 and runs[-1] == 0:
            runs = runs[:-1]
        kind = np.repeat(np.arange(runs.size) % 2, runs).astype(bool)
        vals = s[at + 2 * p: at + 2 * p + esz * nv].view(dt)
        seg = np.zeros(kind.size, dtype=dt)
        seg[kind] = vals
        out[w * E: w * E + seg.size] = seg
    return out


def zvci_from_zvc(zvc_stream, n: int, esz: int) -> np.ndarray:
    """The interleaved stream as a rearrangement of the masks-then-values
    stream (the two hold the same masks and the same values): window w's mask
    is followed by its popcount(mask_w) values; a u32 index of nonzeros before
    each 4 KB block (np.cumsum of the per-block popcounts) goes in front."""
    s = np.asarray(zvc_stream, dtype=np.uint8)
    W = (n + 31) // 32
    E = 4096 // esz
    wr = (n + E - 1) // E
    masks = s[: 4 * W].view("<u4")
    counts = np.unpackbits(masks.view(np.uint8), bitorder="little").reshape(W, 32).sum(axis=1).astype(np.int64)
    vals = s[4 * W:].reshape(-1, esz)
    starts = np.concatenate([np.zeros(1, np.int64), np.cumsum(counts)])
    parts = []
    for w in range(W):
        parts.append(masks[w: w + 1].view(np.uint8))
        parts.append(vals[starts[w]: starts[w + 1]].reshape(-1))
    per_block = np.add.reduceat(counts, np.arange(0, W, E // 32)) if W else np.zeros(0, np.int64)
    index = np.concatenate([np.zeros(1, np.int64), np.cumsum(per_block)]).astype("<u4")
    return np.concatenate([index.view(np.uint8)] + parts) if W else index.view(np.uint8)


def zvci_compress(x) -> np.ndarray:
    b = _bits(x)
    return zvci_from_zvc(zvc_compress(b), b.size, b.dtype.itemsize)
