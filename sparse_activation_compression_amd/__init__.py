"""MI355X-native compression of sparse activation maps for offload to host.

ZVC (a 32-bit nonzero mask per 32 elements, then the nonzero elements) and a
run-length variant, after "Compressing DMA Engine: Leveraging Activation
Sparsity for Training Deep Neural Networks", §V.A Compression Algorithm, run
as hand-written gfx950 HIP kernels behind the C ABI in ``include/cdma.h``.

This module is argument marshalling only: it loads ``libcdma.so`` (built
in-tree by ``__graft_entry__.build()``), exposes the C entry points under the
same names, and offers tensor-level helpers that pass device pointers and the
current HIP stream through.  Every step of the codec runs in the library's
kernels; there is no fallback path.
"""

from .binding import (  # noqa: F401
    ALGO_RLE,
    ALGO_ZVCI,
    ALGO_ZVC,
    CDMA_E_INDEX,
    CDMA_E_MASK_PAST_N,
    CDMA_E_RUN_FORM,
    CDMA_E_RUN_SUM,
    CDMA_E_SIZE,
    CDMA_E_VAL_COUNT,
    FMT_BF16,
    FMT_F16,
    FMT_F32,
    CdmaError,
    Offload,
    Prefetch,
    cdma_compress,
    cdma_decompress,
    cdma_max_compressed_bytes,
    cdma_offload_async,
    cdma_offload_destroy,
    cdma_offload_scratch_bytes,
    cdma_offload_wait,
    cdma_prefetch_async,
    cdma_prefetch_destroy,
    cdma_prefetch_scratch_bytes,
    cdma_prefetch_wait,
    cdma_relu_compress,
    cdma_compress_noalloc,
    cdma_status_string,
    cdma_version,
    cdma_workspace_bytes,
    compress,
    decompress,
    library_path,
    offload,
    prefetch,
    relu_compress,
)
