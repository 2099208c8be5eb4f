"""The C ABI without a GPU: the library loads, exports every entry point that
include/cdma.h declares, sizes buffers by the closed forms, and rejects bad
arguments on the host before touching the device."""

import ctypes
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        for m in re.finditer(r"^[A-Za-z_][\w \t\*]*?\b(cdma_\w+)\s*\(", text, flags=re.M):
            names.add(m.group(1))
    return sorted(names)


@pytest.fixture(scope="module")
def cdma():
    import __graft_entry__
    __graft_entry__.ensure_built()
    import sparse_activation_compression_amd as m
    return m


def test_header_declares_the_boundary():
    names = _declared_functions()
    for required in ("cdma_compress", "cdma_decompress", "cdma_offload_async", "cdma_offload_wait",
                     "cdma_max_compressed_bytes", "cdma_workspace_bytes"):
        assert required in names


def test_library_exports_every_declared_symbol(cdma):
    lib = ctypes.CDLL(cdma.library_path())
    missing = [n for n in _declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


@pytest.mark.parametrize("esz", [2, 4])
@pytest.mark.parametrize("n", [0, 1, 31, 32, 33, 4096, 1 << 30])
def test_max_compressed_bytes_closed_forms(cdma, esz, n):
    assert cdma.cdma_max_compressed_bytes(0, esz, n) == 4 * ((n + 31) // 32) + esz * n
    E = 4096 // esz
    wr = (n + E - 1) // E
    assert cdma.cdma_max_compressed_bytes(1, esz, n) == 8 * (wr + 1) + 2 * (n + 2 * wr) + esz * n


@pytest.mark.parametrize("esz", [2, 4])
@pytest.mark.parametrize("n", [0, 1, 31, 32, 33, 4096, 1 << 30])
def test_interleaved_max_bytes_closed_form(cdma, esz, n):
    E = 4096 // esz
    assert cdma.cdma_max_compressed_bytes(2, esz, n) == 4 * ((n + E - 1) // E + 1) + 4 * ((n + 31) // 32) + esz * n
    assert cdma.cdma_workspace_bytes(2, esz, n) > 0


def test_sizes_reject_bad_algo_esz_n(cdma):
    assert cdma.cdma_max_compressed_bytes(3, 4, 10) == 0
    assert cdma.cdma_max_compressed_bytes(0, 3, 10) == 0
    assert cdma.cdma_max_compressed_bytes(0, 4, (1 << 31) + 1) == 0
    assert cdma.cdma_max_compressed_bytes(1, 4, (1 << 30) + 1) == 0
    assert cdma.cdma_workspace_bytes(0, 8, 10) == 0


def test_workspace_grows_with_tiles(cdma):
    a = cdma.cdma_workspace_bytes(0, 4, 1)
    b = cdma.cdma_workspace_bytes(0, 4, 1 << 30)
    assert 256 < a < b and b % 8 == 0


# Fake but aligned addresses: every call below must fail validation on the
# host, so nothing is ever dereferenced or enqueued.
P = 1 << 20


@pytest.mark.parametrize("args,status", [
    ((3, 4, P, 100, P, 10 ** 6, P, P, 10 ** 6, None), 1),          # bad algo
    ((2, 4, P, 100, P, 423, P, P, 10 ** 6, None), 2),              # interleaved: one byte short
    ((0, 3, P, 100, P, 10 ** 6, P, P, 10 ** 6, None), 1),          # bad element size
    ((0, 4, None, 100, P, 10 ** 6, P, P, 10 ** 6, None), 1),       # NULL source
    ((0, 4, P + 4, 100, P, 10 ** 6, P, P, 10 ** 6, None), 1),      # misaligned source
    ((0, 4, P, 100, P + 8, 10 ** 6, P, P, 10 ** 6, None), 1),      # misaligned destination
    ((0, 4, P, 100, P, 10 ** 6, None, P, 10 ** 6, None), 1),       # NULL size word
    ((0, 4, P, 100, P, 10 ** 6, P + 4, P, 10 ** 6, None), 1),      # misaligned size word
    ((0, 4, P, 100, P, 415, P, P, 10 ** 6, None), 2),              # destination one byte short
    ((0, 4, P, 100, P, 10 ** 6, P, P, 263, None), 2),              # workspace too small
    ((1, 4, P, (1 << 30) + 1, P, 1 << 40, P, P, 1 << 40, None), 1),  # RLE n limit
])
def test_compress_rejects_on_host(cdma, args, status):
    assert cdma.cdma_compress(*args) == status


@pytest.mark.parametrize("args,status", [
    ((5, 4, P, 100, None, 10, P, None, P, 10 ** 6, None), 1),
    ((0, 4, P + 2, 100, None, 10, P, None, P, 10 ** 6, None), 1),
    ((0, 4, P, 100, P + 4, 10, P, None, P, 10 ** 6, None), 1),     # misaligned size word
    ((0, 4, P, 100, None, 10, P + 4, None, P, 10 ** 6, None), 1),  # misaligned destination
    ((0, 4, P, 100, None, 10, P, P + 1, P, 10 ** 6, None), 1),     # misaligned error word
    ((0, 4, P, 100, None, 10, P, None, P, 8, None), 2),            # workspace too small
])
def test_decompress_rejects_on_host(cdma, args, status):
    assert cdma.cdma_decompress(*args) == status


# n = 0: RLE and interleaved ZVC still write an index, so they need a
# destination; ZVC writes nothing but the size word.  Every decoder reads the
# stream for n = 0 too (its index, or its size check), so a NULL stream with a
# nonzero capacity is rejected whatever n is.
@pytest.mark.parametrize("algo", [1, 2])
@pytest.mark.parametrize("dst", [None, P + 4])
def test_empty_compress_needs_a_destination_when_it_writes_an_index(cdma, algo, dst):
    assert cdma.cdma_compress(algo, 4, None, 0, dst, 10 ** 6, P, None, 0, None) == 1


def test_empty_zvc_compress_needs_no_destination(cdma):
    # nothing is enqueued only because the size word check fails first here
    assert cdma.cdma_compress(0, 4, None, 0, None, 0, P + 4, None, 0, None) == 1


@pytest.mark.parametrize("algo", [0, 1, 2])
def test_decompress_rejects_null_stream_with_capacity_even_when_empty(cdma, algo):
    assert cdma.cdma_decompress(algo, 4, None, 16, None, 0, None, P, None, 0, None) == 1
    assert cdma.cdma_decompress(algo, 4, None, 16, None, 100, P, P, P, 10 ** 6, None) == 1


def test_offload_rejects_on_host(cdma):
    sb = cdma.cdma_offload_scratch_bytes(0, 4, 4096, 2)
    assert sb > 0
    ok = dict(algo=0, esz=4, d_src=P, n=10000, chunk_elems=4096, h_dst=P, h_capacity=10 ** 6,
              d_scratch=P, scratch_bytes=sb, slots=2, compute_stream=16, copy_stream=32)

    def call(**kw):
        a = dict(ok, **kw)
        return cdma.cdma_offload_async(*a.values())

    assert call(chunk_elems=1000)[0] == 1          # not a multiple of 2048
    assert call(slots=0)[0] == 1
    assert call(copy_stream=16)[0] == 1            # same stream twice
    assert call(scratch_bytes=sb - 1)[0] == 2
    assert call(d_scratch=P + 16)[0] == 1          # scratch must be 256-byte aligned
    assert call(esz=8)[0] == 1
    assert call(h_dst=None)[0] == 1
    assert cdma.cdma_offload_scratch_bytes(0, 4, 0, 2) == 0
    assert cdma.cdma_offload_scratch_bytes(0, 4, 4096, 0) == 0


def test_status_strings(cdma):
    assert cdma.cdma_status_string(0) == "ok"
    assert cdma.cdma_status_string(2) == "buffer too small"
    assert "unknown" in cdma.cdma_status_string(99)


def test_prefetch_rejects_on_host(cdma):
    n, chunk = 10000, 4096
    sb = cdma.cdma_prefetch_scratch_bytes(0, 4, n, chunk, 2)
    assert sb > 0
    mx = [cdma.cdma_max_compressed_bytes(0, 4, m) for m in (4096, 4096, 10000 - 8192)]
    ok = dict(algo=0, esz=4, h_src=P, h_src_bytes=sum(mx), chunk_bytes=list(mx), n_chunks=3, n=n,
              chunk_elems=chunk, d_dst=P, d_error=None, d_scratch=P, scratch_bytes=sb, slots=2,
              compute_stream=16, copy_stream=32)

    def call(**kw):
        a = dict(ok, **kw)
        return cdma.cdma_prefetch_async(*a.values())[0]

    assert call(algo=3) == 1
    assert call(chunk_elems=1000) == 1                  # not a multiple of 2048
    assert call(n_chunks=2) == 1                         # must be ceil(n / chunk_elems)
    assert call(copy_stream=16) == 1                     # same stream twice
    assert call(d_dst=P + 4) == 1
    assert call(d_scratch=P + 16) == 1
    assert call(d_error=P + 2) == 1
    assert call(scratch_bytes=sb - 1) == 2
    assert call(h_src_bytes=sum(mx) - 1) == 2            # the image does not hold every chunk
    bad = list(mx)
    bad[2] += 1                                          # larger than any stream of the last chunk
    assert call(chunk_bytes=bad) == 3                    # CDMA_ERR_CORRUPT
    assert cdma.cdma_prefetch_scratch_bytes(0, 4, n, 1000, 2) == 0
    assert cdma.cdma_prefetch_scratch_bytes(0, 4, n, chunk, 0) == 0
    # one slot holds the largest chunk's stream, and the layout grows with the slots
    assert cdma.cdma_prefetch_scratch_bytes(0, 4, n, chunk, 3) - sb >= mx[0]


def test_relu_compress_rejects_on_host(cdma):
    n = 1000
    ok = dict(algo=0, fmt=0, d_src=P, n=n, d_act=8 * P, d_dst=2 * P, dst_capacity=10 ** 6, d_out_bytes=P,
              d_ws=P, ws_bytes=10 ** 6, stream=None)

    def call(**kw):
        a = dict(ok, **kw)
        return cdma.cdma_relu_compress(*a.values())

    assert call(fmt=3) == 1                        # unknown format
    assert call(algo=2) == 1                       # ZVC and RLE only
    assert call(algo=3) == 1
    assert call(d_act=8 * P + 4) == 1              # misaligned dense output
    assert call(d_act=P + 16) == 1                 # overlaps the input
    assert call(d_act=2 * P - 16) == 1             # overlaps the stream
    assert call(dst_capacity=4 * 32 + 4 * n - 1) == 2
    assert call(fmt=1, dst_capacity=4 * 32 + 2 * n - 1) == 2  # fp16: 2-byte elements
    assert call(d_src=P + 8) == 1
