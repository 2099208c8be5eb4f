/*
 * cdma.h -- C ABI of libcdma: lossless compression of sparse activation maps
 * on MI355X (gfx950) for offload to host memory.
 *
 * The operations follow "Compressing DMA Engine: Leveraging Activation
 * Sparsity for Training Deep Neural Networks" (Rhu, O'Connor, Chatterjee,
 * Pool, Keckler; arXiv:1705.01626):
 *   - §V.A Compression Algorithm: zero-value compression (ZVC) -- per window
 *     of 32 values a 32-bit zero/nonzero mask, then the nonzero values -- and
 *     the run-length (RLE) variant that codes runs of zeros and nonzeros;
 *   - §VII.A Compression Efficiency: the 4 KB compression window (used here as
 *     the RLE window);
 *   - §V.D Software Interface: a compressed memory-copy call that reports the
 *     compressed size, and offload of every layer's activations to host
 *     memory with asynchronous copies (and their prefetch back, §II.B).
 *
 * Everything here is plain C: device and host pointers, sizes and status
 * codes.  A "stream" argument is a hipStream_t passed as void* (NULL = the
 * null stream).  All device work is enqueued on the given stream and runs in
 * stream order; nothing in cdma_compress / cdma_decompress synchronises.
 *
 * Element model.  The codec moves raw bit patterns of esz bytes (esz = 4 for
 * fp32 or any 32-bit type, 2 for fp16/bf16).  An element is "zero" iff every
 * bit is 0: -0.0, denormals, NaN and Inf are nonzero and are carried
 * verbatim, so decompress(compress(x)) == x bit for bit.
 *
 * Stream formats (little-endian, no header, no padding beyond what is said):
 *   ZVC: u32 mask[W], W = ceil(n/32), bit i of mask[w] = element 32w+i is
 *        nonzero (mask bits for indices >= n are 0); then the nonzero elements
 *        in ascending index order.  size = 4*ceil(n/32) + esz*nnz.
 *   RLE: windows of E = 4096/esz elements, Wr = ceil(n/E).  Per window the
 *        alternating run lengths, zero run first (the first may be 0, the
 *        others are >= 1), as u16; for esz == 4 an odd count is followed by
 *        one 0 entry.  p_w = entries incl. padding, v_w = nonzeros.  Stream =
 *        u32 run_off[Wr+1], u32 val_off[Wr+1] (exclusive prefix sums of p_w and
 *        v_w; entry Wr holds the totals), then block_w for each window: its
 *        p_w u16 entries followed by its v_w nonzero elements.
 *        size = 8*(Wr+1) + 2*sum(p_w) + esz*nnz.
 *   ZVCI: the same masks and values as ZVC, interleaved as the page describes
 *        one window (§V.A): per window its u32 mask, then its nonzero
 *        elements, windows in order.  In front, u32 val_off[Wr+1] with the
 *        nonzeros before each block of E = 4096/esz elements (entry Wr = nnz),
 *        so block b starts at 4*(Wr+1) + 4*b*(E/32) + esz*val_off[b] and decodes
 *        on its own.  size = 4*(Wr+1) + 4*ceil(n/32) + esz*nnz.
 *
 * Ownership.  The caller owns every buffer (sources, destinations,
 * workspaces, scratch, pinned host memory, size and error words) and keeps it
 * alive until the enqueued work has finished.  cdma_compress and
 * cdma_decompress allocate nothing.  cdma_offload_async allocates its handle,
 * a few events and one worker thread, released by cdma_offload_destroy, and
 * takes a small pinned array for the chunk sizes from a pool that the library
 * keeps for the life of the process (allocated on first need, reused by
 * later calls); cdma_prefetch_async the same without the thread, released by
 * cdma_prefetch_destroy.
 *
 * Errors.  Argument and capacity problems are found on the host before
 * anything is enqueued and are returned as a status.  A failing HIP call
 * returns CDMA_ERR_HIP.  Problems in a stream being decoded are found on the
 * device and OR-ed, in stream order, into the caller's error word as
 * CDMA_E_* bits.
 */
#ifndef CDMA_H
#define CDMA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define CDMA_OK              0
#define CDMA_ERR_INVALID_ARG 1  /* bad algo/esz, NULL or misaligned pointer, n too large */
#define CDMA_ERR_CAPACITY    2  /* destination, workspace or host buffer too small */
#define CDMA_ERR_CORRUPT     3  /* host-side decode check: a prefetch chunk size no stream can have */
#define CDMA_ERR_HIP         4  /* a HIP runtime call failed */
#define CDMA_ERR_INTERNAL    5  /* offload: a chunk's compressor reported that its cross-workgroup
                                   scan did not complete (never expected) */

/* algorithms */
#define CDMA_ALGO_ZVC  0
#define CDMA_ALGO_RLE  1
#define CDMA_ALGO_ZVCI 2  /* ZVC with each window's mask in front of its values */

/* decode error bits, OR-ed into *d_error by cdma_decompress */
#define CDMA_E_MASK_PAST_N (1u << 0) /* ZVC, ZVCI: mask bit set for an index >= n */
#define CDMA_E_SIZE        (1u << 1) /* with a size word: the size differs from what the
                                        stream's index or masks describe, or exceeds
                                        src_capacity; without one: the described data
                                        lies past src_capacity */
#define CDMA_E_INDEX       (1u << 3) /* RLE, ZVCI: index does not start at 0 or decreases */
#define CDMA_E_RUN_SUM     (1u << 4) /* RLE: runs do not sum to the window length */
#define CDMA_E_VAL_COUNT   (1u << 5) /* RLE: nonzero runs, ZVCI: a block's mask bits,
                                        disagree with val_off */
#define CDMA_E_RUN_FORM    (1u << 6) /* RLE: zero-length run other than the first, or bad padding */
#define CDMA_E_INTERNAL    (1u << 7) /* the cross-workgroup scan did not complete (never expected) */

/* value cdma_compress stores as the size when its cross-workgroup scan did
   not complete (never expected; the stream is then invalid) */
#define CDMA_SIZE_INTERNAL_ERROR 0xFFFFFFFFFFFFFFFFull

/* limits on n (elements) */
#define CDMA_ZVC_MAX_N (1ull << 31)
#define CDMA_RLE_MAX_N (1ull << 30)   /* ZVCI: as ZVC */

/*
 * Upper bound of the compressed size of n elements (the size of an all-dense
 * input), in bytes: what a caller allocates for a stream before its actual
 * size is known (§V.D sizes the host allocation from the compression ratio
 * observed; a device buffer for one call must hold the worst case).  Returns 0
 * for an invalid algo/esz or an n past the codec's limit.
 *   ZVC:  4*ceil(n/32) + esz*n
 *   RLE:  8*(ceil(n/E)+1) + 2*(n + 2*ceil(n/E)) + esz*n
 *   ZVCI: 4*(ceil(n/E)+1) + 4*ceil(n/32) + esz*n
 */
uint64_t cdma_max_compressed_bytes(int algo, int esz, uint64_t n);

/*
 * Device workspace (bytes) that cdma_compress / cdma_decompress need for n
 * elements (§V.D leaves all buffers to the caller; so does this library).
 * Layout: a 2 KB header (tile ticket counter, the two words that choose
 * static or ticketed tiles, eight ticket-class counters, each on a 128-byte
 * line of its own), then one 32-bit published aggregate per compress tile.
 * ZVC decompress reuses the same space for one 32-bit value offset per 16 KB
 * decompress tile, one total per 32 KB of masks and, for outputs over 1 GiB,
 * 4 KB of read-ahead counters per 1 GiB chunk.  The library clears what
 * it needs itself at the start of each call (with a kernel, not a memset).
 * Workspaces of calls that may overlap in time must be distinct.  Returns 0
 * for invalid input.
 */
uint64_t cdma_workspace_bytes(int algo, int esz, uint64_t n);

/*
 * Compress n elements of esz bytes (§V.A; the compressed size is reported as
 * §V.D's compressed copy call does).
 *   d_src        device, 16-byte aligned, n*esz bytes, read only.
 *   d_dst        device, 16-byte aligned, dst_capacity bytes; receives the
 *                stream.  dst_capacity must be >= cdma_max_compressed_bytes,
 *                else CDMA_ERR_CAPACITY and nothing is enqueued.
 *   d_out_bytes  device (or host-mapped) 8-byte aligned u64; receives the
 *                stream size in bytes when the work completes.
 *   d_ws         device, 8-byte aligned, ws_bytes >= cdma_workspace_bytes.
 * n = 0 is valid: the size word is set to 0.
 */
int cdma_compress(int algo, int esz, const void *d_src, uint64_t n,
                  void *d_dst, uint64_t dst_capacity, uint64_t *d_out_bytes,
                  void *d_ws, uint64_t ws_bytes, void *stream);

/*
 * cdma_compress without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same stream, size word and errors as
 * cdma_compress.  The workspace is a 1 MiB array that the library holds on
 * each GPU it runs on until the process ends; that covers every n the three
 * codecs accept (a larger need would return CDMA_ERR_CAPACITY, before
 * anything is enqueued).  The call allocates nothing: the array's device
 * address is looked up once per device on the first call.  Every call on one
 * GPU shares that array, and each call clears what it needs there first, so
 * calls that may overlap in time on one GPU (other streams, other host
 * threads) race and must be serialised by the caller; use cdma_compress with
 * distinct workspaces for concurrent work.
 */
int cdma_compress_noalloc(int algo, int esz, const void *d_src, uint64_t n,
                          void *d_dst, uint64_t dst_capacity, uint64_t *d_out_bytes,
                          void *stream);

/* element formats of cdma_relu_compress (2- or 4-byte IEEE-style patterns) */
#define CDMA_FMT_F32  0
#define CDMA_FMT_F16  1
#define CDMA_FMT_BF16 2

/*
 * Fused producer epilogue: compress ReLU(x) straight from the pre-activation
 * values x, and optionally write ReLU(x) densely too.  The page compresses
 * activation maps while they are transferred out of GPU memory (§I, §V.B); on a GPU the
 * nearest equivalent is for the kernel that makes the activations to code
 * them as it writes them, so the map is not read a second time.  ReLU is
 * max(x, 0) on the element's pattern: a value with the sign bit set that is
 * not a NaN (-0.0, negative denormals and normals, -inf) becomes +0.0; NaNs
 * (either sign) and all other values pass unchanged.  NaN is decided on the
 * pattern for the format: fp32 |bits| > 0x7F800000, fp16 > 0x7C00, bf16 >
 * 0x7F80 (|bits| = the pattern without its sign bit).
 *   algo          CDMA_ALGO_ZVC or CDMA_ALGO_RLE.
 *   fmt           CDMA_FMT_F32 (esz 4), CDMA_FMT_F16 or CDMA_FMT_BF16 (esz 2).
 *   d_src         device, 16-byte aligned, n elements of x, read only.
 *   d_act         device, 16-byte aligned, n elements; receives ReLU(x), or
 *                 NULL to skip the dense output.  Must not overlap d_src or
 *                 d_dst (CDMA_ERR_INVALID_ARG).
 * The stream, its size word, the workspace and the errors are exactly those of
 * cdma_compress(algo, esz, ReLU(x), ...): the output stream is byte for byte
 * the stream of the ReLU'd map.
 */
int cdma_relu_compress(int algo, int fmt, const void *d_src, uint64_t n, void *d_act,
                       void *d_dst, uint64_t dst_capacity, uint64_t *d_out_bytes,
                       void *d_ws, uint64_t ws_bytes, void *stream);

/*
 * Decompress a stream back into n elements of esz bytes (§V.A; the inverse
 * of cdma_compress, as for the prefetch before reuse of §V.D).
 *   d_src         device, 16-byte aligned stream.
 *   src_capacity  bytes readable at d_src (the decoder never reads past it).
 *   d_src_bytes   device u64 with the stream's exact size, or NULL.  When
 *                 given, a size that disagrees with the stream's content or
 *                 exceeds src_capacity sets CDMA_E_SIZE, and bytes past it read
 *                 as 0; when NULL, src_capacity bounds the reads and data the
 *                 stream describes past it sets CDMA_E_SIZE.
 *   d_dst         device, 16-byte aligned, n*esz bytes, fully written.
 *   d_error       device u32 or NULL; CDMA_E_* bits are OR-ed into it (it is
 *                 not cleared).  After an error the output content is
 *                 unspecified but nothing outside d_dst is written.
 *   d_ws          device, 8-byte aligned, ws_bytes >= cdma_workspace_bytes.
 */
int cdma_decompress(int algo, int esz, const void *d_src, uint64_t src_capacity,
                    const uint64_t *d_src_bytes, uint64_t n, void *d_dst,
                    uint32_t *d_error, void *d_ws, uint64_t ws_bytes, void *stream);

/*
 * Compressed offload (§V.D: every layer's activations are offloaded to host
 * memory with asynchronous copies, the host allocation sized by the observed
 * compression ratio).  The input is cut into K = ceil(n/chunk_elems) chunks
 * that are compressed independently; chunk k's stream is copied to
 * h_dst + sum_{j<k} size_j with hipMemcpyAsync on copy_stream while later
 * chunks compress on compute_stream, through `slots` device staging slots.
 * The host image is the chunks' streams back to back.
 *   chunk_elems   multiple of 2048 (so no ZVC or RLE window straddles chunks).
 *   h_dst         pinned host memory (hipHostMalloc), h_capacity bytes.  If
 *                 the next chunk would not fit, no further chunk is copied and
 *                 cdma_offload_wait returns CDMA_ERR_CAPACITY; nothing past
 *                 h_capacity is ever written.
 *   d_scratch     device, 256-byte aligned, scratch_bytes >=
 *                 cdma_offload_scratch_bytes(algo, esz, chunk_elems, slots):
 *                 per slot, a chunk stream's staging, a compress workspace
 *                 and the device word its size is written to (copied to the
 *                 host on compute_stream, 8 bytes per chunk).
 *   slots         staging slots, >= 1 (2 or 3 overlap compression and copy).
 *   compute_stream, copy_stream  distinct streams (void* hipStream_t); the
 *                 caller enqueues nothing else on them until the wait returns.
 * Returns at once; the pipeline runs on a worker thread.  *out receives the
 * handle (NULL on error).  d_src must stay valid until cdma_offload_wait.
 */
typedef struct cdma_offload_s *cdma_offload_t;

uint64_t cdma_offload_scratch_bytes(int algo, int esz, uint64_t chunk_elems, int slots);

int cdma_offload_async(int algo, int esz, const void *d_src, uint64_t n,
                       uint64_t chunk_elems, void *h_dst, uint64_t h_capacity,
                       void *d_scratch, uint64_t scratch_bytes, int slots,
                       void *compute_stream, void *copy_stream, cdma_offload_t *out);

/*
 * Wait for an offload to finish.  *total_bytes receives the bytes written to
 * h_dst, chunk_bytes[k] (for k < max_chunks) each chunk's stream size and
 * *n_chunks the number of chunks copied.  Any output pointer may be NULL.
 * Returns CDMA_OK, CDMA_ERR_CAPACITY (host buffer too small; the sizes cover
 * the chunks copied), CDMA_ERR_INTERNAL (a chunk's compressor reported an
 * incomplete scan; no further chunk is copied) or CDMA_ERR_HIP.  May be
 * called once per handle.
 */
int cdma_offload_wait(cdma_offload_t h, uint64_t *total_bytes, uint64_t *chunk_bytes,
                      uint64_t max_chunks, uint64_t *n_chunks);

/* Release a handle (waits for it first if cdma_offload_wait was not called). */
void cdma_offload_destroy(cdma_offload_t h);

/*
 * Compressed prefetch (§II.B: offloaded activations are brought back to the
 * GPU before the backward pass reuses them; §V.D: offload and prefetch use
 * asynchronous copies; §V.B: the decompression engine expands the data on
 * its way into GPU memory).  The inverse of cdma_offload_async: h_src holds
 * the chunk streams back to back, chunk k's stream (chunk_bytes[k] bytes) is
 * copied host-to-device with hipMemcpyAsync on copy_stream into staging slot
 * k % slots and decompressed on compute_stream into elements
 * [k*chunk_elems, min(n, (k+1)*chunk_elems)) of d_dst, while later chunks are
 * copied.  Every chunk size is known at the call, so the whole pipeline is
 * enqueued before it returns; no host thread is used.
 *   h_src         pinned host memory (hipHostMalloc), h_src_bytes readable;
 *                 the sum of chunk_bytes must fit, else CDMA_ERR_CAPACITY.
 *   chunk_bytes   host array of n_chunks = ceil(n/chunk_elems) stream sizes,
 *                 as cdma_offload_wait reported them; read during the call
 *                 only.  A size larger than its chunk's
 *                 cdma_max_compressed_bytes is rejected with CDMA_ERR_CORRUPT
 *                 before anything is enqueued (it could not fit a slot).
 *   chunk_elems   multiple of 2048, the value the offload used.
 *   d_dst         device, 16-byte aligned, n*esz bytes, fully written.
 *   d_error       device u32 or NULL; every chunk's CDMA_E_* bits (as
 *                 cdma_decompress reports them) are OR-ed into it.
 *   d_scratch     device, 256-byte aligned, scratch_bytes >=
 *                 cdma_prefetch_scratch_bytes(algo, esz, n, chunk_elems, slots):
 *                 the chunk sizes, one decompress workspace and the slots.
 *   compute_stream, copy_stream  distinct streams; as for the offload.
 * On success *out receives a handle; on any error nothing is left running
 * and *out is NULL.  h_src, d_dst and d_scratch must stay valid until
 * cdma_prefetch_wait returns.
 */
typedef struct cdma_prefetch_s *cdma_prefetch_t;

uint64_t cdma_prefetch_scratch_bytes(int algo, int esz, uint64_t n, uint64_t chunk_elems, int slots);

int cdma_prefetch_async(int algo, int esz, const void *h_src, uint64_t h_src_bytes,
                        const uint64_t *chunk_bytes, uint64_t n_chunks, uint64_t n,
                        uint64_t chunk_elems, void *d_dst, uint32_t *d_error,
                        void *d_scratch, uint64_t scratch_bytes, int slots,
                        void *compute_stream, void *copy_stream, cdma_prefetch_t *out);

/* Wait until every chunk is decompressed.  Returns CDMA_OK or CDMA_ERR_HIP;
   decode problems are in *d_error.  May be called more than once. */
int cdma_prefetch_wait(cdma_prefetch_t h);

/* Release a handle (waits for it first). */
void cdma_prefetch_destroy(cdma_prefetch_t h);

/* Static description of a status code (the CDMA_OK ... CDMA_ERR_* values
   above; "unknown status" otherwise).  The returned string is never freed. */
const char *cdma_status_string(int status);

/* Library version as 10000*major + 100*minor + patch. */
int cdma_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CDMA_H */
