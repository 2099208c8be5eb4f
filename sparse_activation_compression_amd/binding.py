"""ctypes binding of libcdma (see include/cdma.h for the full contract).

The ``cdma_*`` functions mirror the C entry points one to one and take plain
integers (device/host addresses, sizes, stream handles).  ``compress``,
``decompress`` and ``offload`` are thin helpers that take torch tensors, pass
their addresses and the current HIP stream, and allocate outputs and
workspaces with torch (used for device memory and streams only).
"""

from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libcdma.so")

ALGO_ZVC = 0
ALGO_RLE = 1
ALGO_ZVCI = 2

FMT_F32 = 0
FMT_F16 = 1
FMT_BF16 = 2

CDMA_OK = 0
CDMA_ERR_INVALID_ARG = 1
CDMA_ERR_CAPACITY = 2
CDMA_ERR_CORRUPT = 3
CDMA_ERR_HIP = 4
CDMA_ERR_INTERNAL = 5

CDMA_E_MASK_PAST_N = 1 << 0
CDMA_E_SIZE = 1 << 1
CDMA_E_INDEX = 1 << 3
CDMA_E_RUN_SUM = 1 << 4
CDMA_E_VAL_COUNT = 1 << 5
CDMA_E_RUN_FORM = 1 << 6

_ALGOS = {"zvc": ALGO_ZVC, "rle": ALGO_RLE, "zvci": ALGO_ZVCI, ALGO_ZVC: ALGO_ZVC, ALGO_RLE: ALGO_RLE,
          ALGO_ZVCI: ALGO_ZVCI}


class CdmaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status} ({cdma_status_string(status)})")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is missing: build it with __graft_entry__.build() "
            "(hipcc --offload-arch=gfx950); there is no fallback implementation")
    lib = ctypes.CDLL(_LIB_PATH)
    u64, i32, vp = ctypes.c_uint64, ctypes.c_int, ctypes.c_void_p
    sig = {
        "cdma_max_compressed_bytes": (u64, [i32, i32, u64]),
        "cdma_workspace_bytes": (u64, [i32, i32, u64]),
        "cdma_compress": (i32, [i32, i32, vp, u64, vp, u64, vp, vp, u64, vp]),
        "cdma_compress_noalloc": (i32, [i32, i32, vp, u64, vp, u64, vp, vp]),
        "cdma_relu_compress": (i32, [i32, i32, vp, u64, vp, vp, u64, vp, vp, u64, vp]),
        "cdma_decompress": (i32, [i32, i32, vp, u64, vp, u64, vp, vp, vp, u64, vp]),
        "cdma_offload_scratch_bytes": (u64, [i32, i32, u64, i32]),
        "cdma_offload_async": (i32, [i32, i32, vp, u64, u64, vp, u64, vp, u64, i32, vp, vp,
                                     ctypes.POINTER(vp)]),
        "cdma_offload_wait": (i32, [vp, ctypes.POINTER(u64), ctypes.POINTER(u64), u64,
                                    ctypes.POINTER(u64)]),
        "cdma_offload_destroy": (None, [vp]),
        "cdma_prefetch_scratch_bytes": (u64, [i32, i32, u64, u64, i32]),
        "cdma_prefetch_async": (i32, [i32, i32, vp, u64, ctypes.POINTER(u64), u64, u64, u64, vp, vp, vp, u64,
                                      i32, vp, vp, ctypes.POINTER(vp)]),
        "cdma_prefetch_wait": (i32, [vp]),
        "cdma_prefetch_destroy": (None, [vp]),
        "cdma_status_string": (ctypes.c_char_p, [i32]),
        "cdma_version": (i32, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib = _load()


# ---- one-to-one C entry points ----------------------------------------------

def cdma_max_compressed_bytes(algo: int, esz: int, n: int) -> int:
    return int(_lib.cdma_max_compressed_bytes(algo, esz, n))


def cdma_workspace_bytes(algo: int, esz: int, n: int) -> int:
    return int(_lib.cdma_workspace_bytes(algo, esz, n))


def cdma_compress(algo, esz, d_src, n, d_dst, dst_capacity, d_out_bytes, d_ws, ws_bytes, stream) -> int:
    return int(_lib.cdma_compress(algo, esz, d_src, n, d_dst, dst_capacity, d_out_bytes, d_ws,
                                  ws_bytes, stream))


def cdma_compress_noalloc(algo, esz, d_src, n, d_dst, dst_capacity, d_out_bytes, stream) -> int:
    return int(_lib.cdma_compress_noalloc(algo, esz, d_src, n, d_dst, dst_capacity, d_out_bytes, stream))


def cdma_relu_compress(algo, fmt, d_src, n, d_act, d_dst, dst_capacity, d_out_bytes, d_ws, ws_bytes,
                       stream) -> int:
    return int(_lib.cdma_relu_compress(algo, fmt, d_src, n, d_act, d_dst, dst_capacity, d_out_bytes, d_ws,
                                       ws_bytes, stream))


def cdma_decompress(algo, esz, d_src, src_capacity, d_src_bytes, n, d_dst, d_error, d_ws, ws_bytes,
                    stream) -> int:
    return int(_lib.cdma_decompress(algo, esz, d_src, src_capacity, d_src_bytes, n, d_dst, d_error,
                                    d_ws, ws_bytes, stream))


def cdma_offload_scratch_bytes(algo: int, esz: int, chunk_elems: int, slots: int) -> int:
    return int(_lib.cdma_offload_scratch_bytes(algo, esz, chunk_elems, slots))


def cdma_offload_async(algo, esz, d_src, n, chunk_elems, h_dst, h_capacity, d_scratch, scratch_bytes,
                       slots, compute_stream, copy_stream):
    """Returns (status, handle)."""
    h = ctypes.c_void_p(0)
    rc = int(_lib.cdma_offload_async(algo, esz, d_src, n, chunk_elems, h_dst, h_capacity, d_scratch,
                                     scratch_bytes, slots, compute_stream, copy_stream, ctypes.byref(h)))
    return rc, h.value


def cdma_offload_wait(handle, max_chunks: int):
    """Returns (status, total_bytes, chunk_bytes list)."""
    total, nch = ctypes.c_uint64(0), ctypes.c_uint64(0)
    arr = (ctypes.c_uint64 * max(1, max_chunks))()
    rc = int(_lib.cdma_offload_wait(handle, ctypes.byref(total), arr, max_chunks, ctypes.byref(nch)))
    return rc, int(total.value), [int(arr[k]) for k in range(min(nch.value, max_chunks))]


def cdma_offload_destroy(handle) -> None:
    _lib.cdma_offload_destroy(handle)


def cdma_prefetch_scratch_bytes(algo: int, esz: int, n: int, chunk_elems: int, slots: int) -> int:
    return int(_lib.cdma_prefetch_scratch_bytes(algo, esz, n, chunk_elems, slots))


def cdma_prefetch_async(algo, esz, h_src, h_src_bytes, chunk_bytes, n_chunks, n, chunk_elems, d_dst,
                        d_error, d_scratch, scratch_bytes, slots, compute_stream, copy_stream):
    """Returns (status, handle); ``chunk_bytes`` is a sequence of ints."""
    h = ctypes.c_void_p(0)
    arr = (ctypes.c_uint64 * max(1, len(chunk_bytes)))(*chunk_bytes)
    rc = int(_lib.cdma_prefetch_async(algo, esz, h_src, h_src_bytes, arr, n_chunks, n, chunk_elems, d_dst,
                                      d_error, d_scratch, scratch_bytes, slots, compute_stream, copy_stream,
                                      ctypes.byref(h)))
    return rc, h.value


def cdma_prefetch_wait(handle) -> int:
    return int(_lib.cdma_prefetch_wait(handle))


def cdma_prefetch_destroy(handle) -> None:
    _lib.cdma_prefetch_destroy(handle)


def cdma_status_string(status: int) -> str:
    return _lib.cdma_status_string(status).decode()


def cdma_version() -> int:
    return int(_lib.cdma_version())


# ---- tensor helpers ------------------------------------------------------------

def _stream_handle(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _on(stream):
    """Context in which the buffers a helper allocates for the caller (the
    workspace, the error word, outputs) are made and zeroed on ``stream``:
    the library's kernels run there, so the zeroing precedes them in stream
    order and the workspace, returned to ``stream``'s pool when the helper
    returns, is reused only by later work on that same stream."""
    import contextlib
    import torch
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _check(fn, rc):
    if rc != 0:
        raise CdmaError(fn, rc)


def _esz(t) -> int:
    esz = t.element_size()
    if esz not in (2, 4):
        raise ValueError("elements must be 2 or 4 bytes wide")
    return esz


def workspace(algo, esz: int, n: int, device):
    import torch
    return torch.empty(max(256, cdma_workspace_bytes(_ALGOS[algo], esz, n)), dtype=torch.uint8, device=device)


def compress(x, algo="zvc", dst=None, out_bytes=None, ws=None, stream=None):
    """Compress the raw patterns of contiguous device tensor ``x``.

    Returns (dst, out_bytes): ``dst`` is a uint8 device buffer of the maximal
    compressed size holding the stream in its first ``out_bytes[0]`` bytes;
    ``out_bytes`` is a 1-element int64 device tensor filled in stream order.
    With ``stream``, the work runs on that stream and any buffer made here is
    made on it; the caller orders ``x`` (and buffers passed in) before it.
    """
    import torch
    a = _ALGOS[algo]
    if not x.is_contiguous():
        raise ValueError("input must be contiguous")
    esz, n = _esz(x), x.numel()
    cap = cdma_max_compressed_bytes(a, esz, n)
    with _on(stream):
        if dst is None:
            dst = torch.empty(max(16, cap), dtype=torch.uint8, device=x.device)
        if out_bytes is None:
            out_bytes = torch.empty(1, dtype=torch.int64, device=x.device)
        if ws is None:
            ws = workspace(a, esz, n, x.device)
        rc = cdma_compress(a, esz, x.data_ptr(), n, dst.data_ptr(), dst.numel(), out_bytes.data_ptr(),
                           ws.data_ptr(), ws.numel(), _stream_handle(stream))
    _check("cdma_compress", rc)
    return dst, out_bytes


def _fmt_of(x) -> int:
    import torch
    fmts = {torch.float32: FMT_F32, torch.float16: FMT_F16, torch.bfloat16: FMT_BF16}
    if x.dtype not in fmts:
        raise ValueError("ReLU compression takes float32, float16 or bfloat16 tensors")
    return fmts[x.dtype]


def relu_compress(x, algo="zvc", act=None, dst=None, out_bytes=None, ws=None, stream=None):
    """Compress ReLU(x) straight from the pre-activation tensor ``x``
    (float32 / float16 / bfloat16, contiguous, on the device).

    ``act``: a tensor like ``x`` that receives ReLU(x) densely, True to
    allocate one, or None to skip the dense output.  Returns
    (dst, out_bytes, act) as :func:`compress` does, plus the dense output."""
    import torch
    a = _ALGOS[algo]
    if not x.is_contiguous():
        raise ValueError("input must be contiguous")
    fmt, esz, n = _fmt_of(x), x.element_size(), x.numel()
    cap = cdma_max_compressed_bytes(a, esz, n)
    with _on(stream):
        if act is True:
            act = torch.empty_like(x)
        if dst is None:
            dst = torch.empty(max(16, cap), dtype=torch.uint8, device=x.device)
        if out_bytes is None:
            out_bytes = torch.empty(1, dtype=torch.int64, device=x.device)
        if ws is None:
            ws = workspace(a, esz, n, x.device)
        rc = cdma_relu_compress(a, fmt, x.data_ptr(), n, act.data_ptr() if act is not None else None,
                                dst.data_ptr(), dst.numel(), out_bytes.data_ptr(), ws.data_ptr(), ws.numel(),
                                _stream_handle(stream))
    _check("cdma_relu_compress", rc)
    return dst, out_bytes, act


def decompress(src, n: int, esz: int, algo="zvc", src_bytes=None, out=None, error=None, ws=None,
               stream=None):
    """Decompress a stream held in uint8 device tensor ``src``.

    Returns (out, error): ``out`` holds n elements as int32 (esz 4) or int16
    (esz 2) bit patterns; ``error`` is a 1-element int32 device tensor of
    CDMA_E_* bits (zeroed here unless passed in).
    """
    import torch
    a = _ALGOS[algo]
    dev = src.device
    with _on(stream):
        if out is None:
            out = torch.empty(max(1, n), dtype=torch.int32 if esz == 4 else torch.int16, device=dev)[:n]
        if error is None:
            error = torch.zeros(1, dtype=torch.int32, device=dev)
        if ws is None:
            ws = workspace(a, esz, n, dev)
        rc = cdma_decompress(a, esz, src.data_ptr(), src.numel(),
                             src_bytes.data_ptr() if src_bytes is not None else None, n, out.data_ptr(),
                             error.data_ptr(), ws.data_ptr(), ws.numel(), _stream_handle(stream))
    _check("cdma_decompress", rc)
    return out, error


class Offload:
    """A running compressed offload; call wait() once for its result."""

    def __init__(self, handle, keep, max_chunks):
        self._h = handle
        self._keep = keep
        self._max = max_chunks
        self._result = None

    def wait(self):
        if self._result is None:
            rc, total, sizes = cdma_offload_wait(self._h, self._max)
            cdma_offload_destroy(self._h)
            self._h = None
            self._result = (rc, total, sizes)
            self._keep = None
        return self._result

    def __del__(self):
        if self._h is not None:
            cdma_offload_destroy(self._h)


def offload(x, h_dst, chunk_elems: int = 1 << 24, algo="zvc", slots: int = 3, scratch=None,
            compute_stream=None, copy_stream=None) -> Offload:
    """Start a compressed offload of device tensor ``x`` into pinned uint8
    host tensor ``h_dst``.  The work is ordered after everything already
    enqueued on the current stream.  Returns an :class:`Offload`."""
    import torch
    a = _ALGOS[algo]
    esz, n = _esz(x), x.numel()
    if scratch is None:
        scratch = torch.empty(max(256, cdma_offload_scratch_bytes(a, esz, chunk_elems, slots)),
                              dtype=torch.uint8, device=x.device)
    comp = compute_stream or torch.cuda.Stream(device=x.device)
    copy = copy_stream or torch.cuda.Stream(device=x.device)
    ready = torch.cuda.Event()
    ready.record(torch.cuda.current_stream(x.device))
    comp.wait_event(ready)
    rc, h = cdma_offload_async(a, esz, x.data_ptr(), n, chunk_elems, h_dst.data_ptr(), h_dst.numel(),
                               scratch.data_ptr(), scratch.numel(), slots, comp.cuda_stream,
                               copy.cuda_stream)
    _check("cdma_offload_async", rc)
    k = (n + chunk_elems - 1) // chunk_elems
    return Offload(h, (x, h_dst, scratch, comp, copy), max(1, k))


class Prefetch:
    """A running compressed prefetch; wait() returns (status, out, error)."""

    def __init__(self, handle, out, error, keep):
        self._h = handle
        self._out = out
        self._err = error
        self._keep = keep
        self._result = None

    def wait(self):
        if self._result is None:
            rc = cdma_prefetch_wait(self._h)
            cdma_prefetch_destroy(self._h)
            self._h = None
            self._keep = None
            self._result = (rc, self._out, self._err)
        return self._result

    def __del__(self):
        if self._h is not None:
            cdma_prefetch_destroy(self._h)


def prefetch(h_src, chunk_bytes, n: int, esz: int, chunk_elems: int = 1 << 24, algo="zvc", slots: int = 3,
             out=None, error=None, scratch=None, compute_stream=None, copy_stream=None, device=None) -> Prefetch:
    """Start a compressed prefetch of the host image ``h_src`` (pinned uint8
    tensor holding the chunk streams back to back, as :func:`offload` wrote
    them, with their sizes ``chunk_bytes``) into a device tensor of n
    elements of esz bytes.  Ordered after the work already enqueued on the
    current stream.  Returns a :class:`Prefetch`."""
    import torch
    a = _ALGOS[algo]
    dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
    if out is None:
        out = torch.empty(max(1, n), dtype=torch.int32 if esz == 4 else torch.int16, device=dev)[:n]
    if error is None:
        error = torch.zeros(1, dtype=torch.int32, device=dev)
    if scratch is None:
        scratch = torch.empty(max(256, cdma_prefetch_scratch_bytes(a, esz, n, chunk_elems, slots)),
                              dtype=torch.uint8, device=dev)
    comp = compute_stream or torch.cuda.Stream(device=dev)
    copy = copy_stream or torch.cuda.Stream(device=dev)
    ready = torch.cuda.Event()
    ready.record(torch.cuda.current_stream(dev))
    comp.wait_event(ready)
    copy.wait_event(ready)
    sizes = [int(v) for v in chunk_bytes]
    rc, h = cdma_prefetch_async(a, esz, h_src.data_ptr(), h_src.numel(), sizes, len(sizes), n, chunk_elems,
                                out.data_ptr(), error.data_ptr(), scratch.data_ptr(), scratch.numel(), slots,
                                comp.cuda_stream, copy.cuda_stream)
    _check("cdma_prefetch_async", rc)
    # the caller's stream sees the result once the compute stream is done
    torch.cuda.current_stream(dev).wait_stream(comp)
    return Prefetch(h, out, error, (h_src, scratch, comp, copy))
