"""CPU oracle for the ZVC / RLE activation codec -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its binding) never does, and this package never imports the product path.

Two independent forms of the same definition:

* ``oracle.c`` (loaded here through ctypes): plain scalar loops over the raw
  element bit patterns, following "Compressing DMA Engine: Leveraging
  Activation Sparsity for Training Deep Neural Networks", §V.A Compression
  Algorithm (ZVC: a 32-bit nonzero mask per 32 values, then the nonzero values;
  run-length coding of clustered zeros and nonzeros) and §VII.A Compression
  Efficiency (4 KB compression window).
* ``np_forms`` : the special case written with library routines
  (``np.packbits`` + boolean indexing for ZVC, ``np.diff`` change points for
  RLE), used to cross-check the loops.

Pins for both live in ``tests/test_oracle_*.py``; every pin is something other
than the oracle itself (hand-worked streams, closed forms, the page's 32x
all-zero window, exhaustive tiny cases, invariants, planted mistakes).
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle_mt.c")  # includes oracle.c
_LIB = os.path.join(_HERE, "liboracle.so")

# decode error bits (same meaning as the library's, defined here on their own)
E_MASK_PAST_N = 1 << 0
E_SIZE = 1 << 1
E_INDEX = 1 << 3
E_RUN_SUM = 1 << 4
E_VAL_COUNT = 1 << 5
E_RUN_FORM = 1 << 6

_lib = None


def build(src: str = _SRC, out: str = _LIB, extra=()) -> str:
    """Compile the oracle with plain gcc -O2 (no target-specific flags)."""
    cmd = ["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-shared", "-fPIC", "-pthread",
           *extra, src, "-o", out]
    subprocess.run(cmd, check=True)
    return out


def load(path: str | None = None):
    """Load the compiled oracle (building it first if it is missing)."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    p = path or _LIB
    if not os.path.exists(p):
        if path is not None:
            raise FileNotFoundError(p)
        build()
    lib = ctypes.CDLL(p)
    u64, u32p, u64p = ctypes.c_uint64, ctypes.POINTER(ctypes.c_uint32), ctypes.POINTER(ctypes.c_uint64)
    vp = ctypes.c_void_p
    for name in ("oracle_zvc_size", "oracle_rle_size", "oracle_zvci_size"):
        f = getattr(lib, name)
        f.restype = u64
        f.argtypes = [vp, u64, ctypes.c_int]
    for name in ("oracle_zvc_compress", "oracle_rle_compress", "oracle_zvci_compress"):
        f = getattr(lib, name)
        f.restype = ctypes.c_int
        f.argtypes = [vp, u64, ctypes.c_int, vp, u64, u64p]
    for name in ("oracle_zvc_decompress", "oracle_rle_decompress", "oracle_zvci_decompress"):
        f = getattr(lib, name)
        f.restype = ctypes.c_int
        f.argtypes = [vp, u64, u64, ctypes.c_int, vp, u32p]
    lib.oracle_relu.restype = ctypes.c_int
    lib.oracle_relu.argtypes = [vp, u64, ctypes.c_int, vp]
    # the threaded forms (oracle_mt.c); a library built from oracle.c alone
    # (the planted-mistake tests) has only the single-threaded functions
    for name in ("oracle_zvc_compress_mt", "oracle_rle_compress_mt"):
        if hasattr(lib, name):
            f = getattr(lib, name)
            f.restype = ctypes.c_int
            f.argtypes = [vp, u64, ctypes.c_int, vp, u64, u64p, ctypes.c_int]
    for name in ("oracle_zvc_decompress_mt", "oracle_rle_decompress_mt"):
        if hasattr(lib, name):
            f = getattr(lib, name)
            f.restype = ctypes.c_int
            f.argtypes = [vp, u64, u64, ctypes.c_int, vp, u32p, ctypes.c_int]
    if path is None:
        _lib = lib
    return lib


def _bits(x: np.ndarray) -> np.ndarray:
    """Flat, contiguous unsigned-integer view of the raw element patterns."""
    x = np.ascontiguousarray(x).reshape(-1)
    if x.dtype.itemsize == 4:
        return x.view(np.uint32)
    if x.dtype.itemsize == 2:
        return x.view(np.uint16)
    raise ValueError("elements must be 16 or 32 bits wide")


def max_zvc_bytes(n: int, esz: int) -> int:
    return 4 * ((n + 31) // 32) + esz * n


def max_rle_bytes(n: int, esz: int) -> int:
    E = 4096 // esz
    wr = (n + E - 1) // E
    return 8 * (wr + 1) + 2 * (n + 2 * wr) + esz * n


def _compress(fn, x, cap_fn, lib, *extra):
    b = _bits(x)
    n, esz = b.size, b.dtype.itemsize
    out = np.zeros(max(1, cap_fn(n, esz)), dtype=np.uint8)
    size = ctypes.c_uint64(0)
    rc = getattr(lib, fn)(b.ctypes.data, n, esz, out.ctypes.data, out.size, ctypes.byref(size), *extra)
    if rc != 0:
        raise RuntimeError(f"{fn} failed with {rc}")
    return out[: size.value].copy()


def _decompress(fn, stream, n, esz, lib, *extra):
    s = np.ascontiguousarray(np.asarray(stream, dtype=np.uint8))
    out = np.zeros(max(1, n), dtype=np.uint32 if esz == 4 else np.uint16)
    err = ctypes.c_uint32(0)
    rc = getattr(lib, fn)(s.ctypes.data if s.size else None, s.size, n, esz,
                          out.ctypes.data, ctypes.byref(err), *extra)
    if rc != 0:
        raise RuntimeError(f"{fn} failed with {rc}")
    return out[:n], err.value


def zvc_compress(x, lib=None) -> np.ndarray:
    """ZVC stream (uint8 array) of the raw element patterns of ``x``."""
    return _compress("oracle_zvc_compress", x, max_zvc_bytes, lib or load())


def zvc_decompress(stream, n: int, esz: int, lib=None):
    """(patterns, error bits) decoded from a ZVC stream."""
    return _decompress("oracle_zvc_decompress", stream, n, esz, lib or load())


def rle_compress(x, lib=None) -> np.ndarray:
    """RLE stream (uint8 array) of the raw element patterns of ``x``."""
    return _compress("oracle_rle_compress", x, max_rle_bytes, lib or load())


def rle_decompress(stream, n: int, esz: int, lib=None):
    """(patterns, error bits) decoded from an RLE stream."""
    return _decompress("oracle_rle_decompress", stream, n, esz, lib or load())


# The same definitions on several host threads: each thread counts its own
# range of windows, a prefix places the ranges, each thread writes its range.
# The results equal the single-threaded functions' byte for byte.

def zvc_compress_mt(x, threads: int, lib=None) -> np.ndarray:
    return _compress("oracle_zvc_compress_mt", x, max_zvc_bytes, lib or load(), int(threads))


def zvc_decompress_mt(stream, n: int, esz: int, threads: int, lib=None):
    return _decompress("oracle_zvc_decompress_mt", stream, n, esz, lib or load(), int(threads))


def rle_compress_mt(x, threads: int, lib=None) -> np.ndarray:
    return _compress("oracle_rle_compress_mt", x, max_rle_bytes, lib or load(), int(threads))


def rle_decompress_mt(stream, n: int, esz: int, threads: int, lib=None):
    return _decompress("oracle_rle_decompress_mt", stream, n, esz, lib or load(), int(threads))


def max_zvci_bytes(n: int, esz: int) -> int:
    E = 4096 // esz
    return 4 * ((n + E - 1) // E + 1) + 4 * ((n + 31) // 32) + esz * n


def zvci_compress(x, lib=None) -> np.ndarray:
    """Interleaved ZVC stream (per window: mask, then its nonzeros; a u32
    nonzero-count index per 4 KB block in front) of the patterns of ``x``."""
    return _compress("oracle_zvci_compress", x, max_zvci_bytes, lib or load())


def zvci_decompress(stream, n: int, esz: int, lib=None):
    """(patterns, error bits) decoded from an interleaved ZVC stream."""
    return _decompress("oracle_zvci_decompress", stream, n, esz, lib or load())


def zvci_size(x, lib=None) -> int:
    b = _bits(x)
    return int((lib or load()).oracle_zvci_size(b.ctypes.data, b.size, b.dtype.itemsize))


def zvc_size(x, lib=None) -> int:
    b = _bits(x)
    return int((lib or load()).oracle_zvc_size(b.ctypes.data, b.size, b.dtype.itemsize))


def rle_size(x, lib=None) -> int:
    b = _bits(x)
    return int((lib or load()).oracle_rle_size(b.ctypes.data, b.size, b.dtype.itemsize))


def offload_stream(x, chunk_elems: int, algo: str = "zvc", lib=None):
    """Host image of a chunked compressed offload: the streams of consecutive
    chunks of ``chunk_elems`` elements, each compressed on its own, laid back
    to back, plus each chunk's byte count."""
    b = _bits(x)
    comp = {"zvc": zvc_compress, "rle": rle_compress, "zvci": zvci_compress}[algo]
    parts = [comp(b[lo: lo + chunk_elems], lib) for lo in range(0, b.size, chunk_elems)]
    sizes = [p.size for p in parts]
    return (np.concatenate(parts) if parts else np.zeros(0, np.uint8)), sizes


def restore(image, chunk_bytes, n: int, esz: int, chunk_elems: int, algo: str = "zvc", lib=None):
    """Inverse of :func:`offload_stream`: chunk k of ``chunk_elems`` elements
    (the last one partial) is decoded on its own from the next
    ``chunk_bytes[k]`` bytes of ``image``.  Returns (patterns, OR of every
    chunk's error bits)."""
    img = np.ascontiguousarray(np.asarray(image, dtype=np.uint8))
    dec = {"zvc": zvc_decompress, "rle": rle_decompress, "zvci": zvci_decompress}[algo]
    out = np.zeros(n, dtype=np.uint32 if esz == 4 else np.uint16)
    err, off = 0, 0
    for k, size in enumerate(chunk_bytes):
        lo = k * chunk_elems
        m = min(chunk_elems, n - lo)
        part, e = dec(img[off: off + size], m, esz, lib)
        out[lo: lo + m] = part
        err |= e
        off += size
    return out, err


FMT_F32, FMT_F16, FMT_BF16 = 0, 1, 2


def relu(x, fmt: int, lib=None) -> np.ndarray:
    """ReLU of the raw patterns of ``x`` (fmt 0 = fp32, 1 = fp16, 2 = bf16):
    a NaN passes unchanged, any other value with the sign bit set becomes
    +0.0, everything else passes unchanged."""
    b = _bits(x)
    if b.dtype.itemsize != (4 if fmt == FMT_F32 else 2):
        raise ValueError("element size does not match the format")
    out = np.zeros(max(1, b.size), dtype=b.dtype)
    rc = (lib or load()).oracle_relu(b.ctypes.data, b.size, fmt, out.ctypes.data)
    if rc != 0:
        raise RuntimeError(f"oracle_relu failed with {rc}")
    return out[: b.size]
