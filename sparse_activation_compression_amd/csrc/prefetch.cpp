// prefetch.cpp -- compressed prefetch: bring an offloaded activation buffer
// back from pinned host memory, overlapping the host-to-device copy of each
// chunk's stream with the decompression of earlier chunks.
//
// "Compressing DMA Engine: Leveraging Activation Sparsity for Training Deep
// Neural Networks", §II.B (the offloaded activations are prefetched back to
// the GPU before the backward pass reuses them) and §V.D Software Interface
// (offload and prefetch go through asynchronous copies); §V.B has the
// decompression engine expand the compressed data on its way into GPU memory.
// Here the copy engine moves the compressed bytes and the expansion is the
// decompression kernel.  Every chunk size is known up front (the offload
// returned them), so the whole pipeline is enqueued at once, with no host
// thread:
//
//   copy stream:    [sizes -> device]  wait freed[s] -> copy chunk k into
//                   slot s = k % slots -> record copied[s]
//   compute stream: wait copied[s] -> decompress slot s into chunk k of the
//                   output -> record freed[s]
//
// A stream waits on the most recent record of an event at the time the wait
// is enqueued, so enqueueing chunk by chunk in order pairs every wait with the
// record of the right chunk.
#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include <vector>

#include "cdma.h"
#include "pinned_pool.hpp"

namespace {

constexpr uint64_t kAlign = 256;
uint64_t align_up(uint64_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct PrefetchLayout {
  uint64_t sizes_bytes, ws_bytes, slot_bytes, total;
};

// scratch = [K stream sizes (u64)] [decompress workspace] [slots x staging]
PrefetchLayout prefetch_layout(int algo, int esz, uint64_t n, uint64_t chunk, int slots) {
  PrefetchLayout L{};
  const uint64_t K = (n + chunk - 1) / chunk;
  const uint64_t first = n < chunk ? n : chunk;  // the largest chunk
  L.sizes_bytes = align_up(8 * (K > 0 ? K : 1));
  L.ws_bytes = align_up(cdma_workspace_bytes(algo, esz, first));
  L.slot_bytes = align_up(cdma_max_compressed_bytes(algo, esz, first));
  L.total = L.sizes_bytes + L.ws_bytes + L.slot_bytes * (uint64_t)slots;
  return L;
}

bool args_ok(int algo, int esz, uint64_t chunk, int slots) {
  if ((algo != CDMA_ALGO_ZVC && algo != CDMA_ALGO_RLE && algo != CDMA_ALGO_ZVCI) || (esz != 2 && esz != 4))
    return false;
  if (slots < 1 || chunk == 0 || chunk % 2048 != 0) return false;
  return cdma_max_compressed_bytes(algo, esz, chunk) != 0;
}

}  // namespace

struct cdma_prefetch_s {
  int device = 0;
  hipStream_t comp = nullptr, copy = nullptr;
  uint64_t* h_sizes = nullptr;  // pinned copy of the chunk sizes (source of one H2D copy), from the pool
  std::vector<hipEvent_t> copied, freed;
  hipEvent_t done = nullptr;
  int status = CDMA_OK;
  bool waited = false;

  int wait() {
    if (!waited) {
      waited = true;
      if (status == CDMA_OK && done && hipEventSynchronize(done) != hipSuccess) status = CDMA_ERR_HIP;
      // a failed enqueue may have left work behind: drain both streams before
      // the caller may reuse the scratch, the host image or the output
      if (status != CDMA_OK) {
        (void)hipStreamSynchronize(comp);
        (void)hipStreamSynchronize(copy);
      }
    }
    return status;
  }

  ~cdma_prefetch_s() {
    wait();
    for (hipEvent_t e : copied) (void)hipEventDestroy(e);
    for (hipEvent_t e : freed) (void)hipEventDestroy(e);
    if (done) (void)hipEventDestroy(done);
    cdma::pinned_release(h_sizes);  // after wait(): the copy out of it has finished
  }
};

extern "C" {

uint64_t cdma_prefetch_scratch_bytes(int algo, int esz, uint64_t n, uint64_t chunk_elems, int slots) {
  if (!args_ok(algo, esz, chunk_elems, slots)) return 0;
  if (cdma_max_compressed_bytes(algo, esz, n) == 0 && n != 0) return 0;
  return prefetch_layout(algo, esz, n, chunk_elems, slots).total;
}

int cdma_prefetch_async(int algo, int esz, const void* h_src, uint64_t h_src_bytes, const uint64_t* chunk_bytes,
                        uint64_t n_chunks, uint64_t n, uint64_t chunk_elems, void* d_dst, uint32_t* d_error,
                        void* d_scratch, uint64_t scratch_bytes, int slots, void* compute_stream,
                        void* copy_stream, cdma_prefetch_t* out) {
  if (!out) return CDMA_ERR_INVALID_ARG;
  *out = nullptr;
  if (!args_ok(algo, esz, chunk_elems, slots)) return CDMA_ERR_INVALID_ARG;
  if (n > (algo == CDMA_ALGO_RLE ? CDMA_RLE_MAX_N : CDMA_ZVC_MAX_N)) return CDMA_ERR_INVALID_ARG;
  if (compute_stream == copy_stream) return CDMA_ERR_INVALID_ARG;
  const uint64_t K = (n + chunk_elems - 1) / chunk_elems;
  if (n_chunks != K) return CDMA_ERR_INVALID_ARG;
  if (d_error && (reinterpret_cast<uintptr_t>(d_error) & 3)) return CDMA_ERR_INVALID_ARG;
  if (n > 0) {
    if (!h_src || !chunk_bytes || !d_dst || !d_scratch) return CDMA_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(d_dst) & 15) || (reinterpret_cast<uintptr_t>(d_scratch) & (kAlign - 1)))
      return CDMA_ERR_INVALID_ARG;
    if (scratch_bytes < cdma_prefetch_scratch_bytes(algo, esz, n, chunk_elems, slots)) return CDMA_ERR_CAPACITY;
    // a size no stream of its chunk can have would overflow a staging slot
    uint64_t total = 0;
    for (uint64_t k = 0; k < K; ++k) {
      const uint64_t len = n - k * chunk_elems < chunk_elems ? n - k * chunk_elems : chunk_elems;
      if (chunk_bytes[k] > cdma_max_compressed_bytes(algo, esz, len)) return CDMA_ERR_CORRUPT;
      total += chunk_bytes[k];
    }
    if (total > h_src_bytes) return CDMA_ERR_CAPACITY;
  }

  cdma_prefetch_s* h = new cdma_prefetch_s();
  h->comp = static_cast<hipStream_t>(compute_stream);
  h->copy = static_cast<hipStream_t>(copy_stream);
  if (n == 0) {
    *out = h;
    return CDMA_OK;
  }

  const PrefetchLayout L = prefetch_layout(algo, esz, n, chunk_elems, slots);
  uint8_t* scratch = static_cast<uint8_t*>(d_scratch);
  uint64_t* d_sizes = reinterpret_cast<uint64_t*>(scratch);
  uint8_t* ws = scratch + L.sizes_bytes;
  auto slot = [&](uint64_t s) { return scratch + L.sizes_bytes + L.ws_bytes + s * L.slot_bytes; };
  const uint8_t* src = static_cast<const uint8_t*>(h_src);
  uint8_t* dst = static_cast<uint8_t*>(d_dst);

  bool ok = hipGetDevice(&h->device) == hipSuccess;
  if (ok) h->h_sizes = static_cast<uint64_t*>(cdma::pinned_acquire(K * sizeof(uint64_t)));
  ok = ok && h->h_sizes != nullptr;
  for (int s = 0; ok && s < slots; ++s) {
    hipEvent_t a = nullptr, b = nullptr;
    ok = hipEventCreateWithFlags(&a, hipEventDisableTiming) == hipSuccess;
    if (ok) h->copied.push_back(a);
    ok = ok && hipEventCreateWithFlags(&b, hipEventDisableTiming) == hipSuccess;
    if (ok) h->freed.push_back(b);
  }
  ok = ok && hipEventCreateWithFlags(&h->done, hipEventDisableTiming) == hipSuccess;
  if (!ok) {
    h->status = CDMA_ERR_HIP;
    delete h;
    return CDMA_ERR_HIP;
  }
  for (uint64_t k = 0; k < K; ++k) h->h_sizes[k] = chunk_bytes[k];

  int rc = CDMA_OK;
  if (hipMemcpyAsync(d_sizes, h->h_sizes, K * sizeof(uint64_t), hipMemcpyHostToDevice, h->copy) != hipSuccess)
    rc = CDMA_ERR_HIP;
  uint64_t off = 0;
  for (uint64_t k = 0; k < K && rc == CDMA_OK; ++k) {
    const int s = (int)(k % (uint64_t)slots);
    const uint64_t lo = k * chunk_elems;
    const uint64_t len = n - lo < chunk_elems ? n - lo : chunk_elems;
    const uint64_t size = chunk_bytes[k];
    if (k >= (uint64_t)slots && hipStreamWaitEvent(h->copy, h->freed[s], 0) != hipSuccess) rc = CDMA_ERR_HIP;
    if (rc == CDMA_OK && size &&
        hipMemcpyAsync(slot(s), src + off, size, hipMemcpyHostToDevice, h->copy) != hipSuccess)
      rc = CDMA_ERR_HIP;
    if (rc == CDMA_OK && hipEventRecord(h->copied[s], h->copy) != hipSuccess) rc = CDMA_ERR_HIP;
    if (rc == CDMA_OK && hipStreamWaitEvent(h->comp, h->copied[s], 0) != hipSuccess) rc = CDMA_ERR_HIP;
    if (rc == CDMA_OK)
      rc = cdma_decompress(algo, esz, slot(s), L.slot_bytes, d_sizes + k, len, dst + lo * (uint64_t)esz, d_error,
                           ws, L.ws_bytes, h->comp);
    if (rc == CDMA_OK && hipEventRecord(h->freed[s], h->comp) != hipSuccess) rc = CDMA_ERR_HIP;
    off += size;
  }
  // done = the last decompress; the copy stream's work all precedes it
  if (rc == CDMA_OK && hipEventRecord(h->done, h->comp) != hipSuccess) rc = CDMA_ERR_HIP;
  h->status = rc;
  if (rc != CDMA_OK) {  // drain what was enqueued before the failure, then give up
    delete h;
    return rc;
  }
  *out = h;
  return CDMA_OK;
}

int cdma_prefetch_wait(cdma_prefetch_t h) {
  if (!h) return CDMA_ERR_INVALID_ARG;
  return h->wait();
}

void cdma_prefetch_destroy(cdma_prefetch_t h) { delete h; }

}  // extern "C"
