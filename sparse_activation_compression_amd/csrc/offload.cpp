// offload.cpp -- compressed offload of an activation buffer to pinned host
// memory, overlapping compression with the device-to-host copy.
//
// "Compressing DMA Engine: Leveraging Activation Sparsity for Training Deep
// Neural Networks", §V.D Software Interface: the memory manager offloads every
// layer's activations with asynchronous copies and sizes the host allocation
// by the observed compression ratio; the compressed copy call reports the
// compressed size.  On MI355X the compressor is a kernel and the link is
// driven by the SDMA engines through hipMemcpyAsync, so the two are
// pipelined over chunks:
//
//   compute stream:  [compress k into slot s, size into the slot's device
//                    size word] -> [copy the 8-byte size to pinned host
//                    memory] -> record comp_done[s]
//   worker thread:   wait comp_done[s] -> read size_k -> check the host
//                    capacity -> hipMemcpyAsync(size_k bytes, copy stream)
//                    -> record copy_done[s] -> compute stream waits
//                    copy_done[s] before compressing chunk k + slots into
//                    the same staging slot.
// The size reaches the host by a copy, so nothing depends on device atomics
// to host memory over the link.
//
// The copy needs the size on the host, so one host round trip per chunk is
// unavoidable; with >= 2 slots it overlaps the previous chunk's copy.
#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include <thread>
#include <vector>

#include "cdma.h"
#include "pinned_pool.hpp"

namespace {

constexpr uint64_t kAlign = 256;
uint64_t align_up(uint64_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Scratch slot = [stream staging][compress workspace][size word]
struct SlotLayout {
  uint64_t stream_bytes, ws_bytes, slot_bytes;
};

SlotLayout slot_layout(int algo, int esz, uint64_t chunk) {
  SlotLayout L;
  L.stream_bytes = align_up(cdma_max_compressed_bytes(algo, esz, chunk));
  L.ws_bytes = align_up(cdma_workspace_bytes(algo, esz, chunk));
  L.slot_bytes = L.stream_bytes + L.ws_bytes + kAlign;
  return L;
}

}  // namespace

struct cdma_offload_s {
  int algo = 0, esz = 0, device = 0, slots = 0;
  const uint8_t* src = nullptr;
  uint64_t n = 0, chunk = 0, K = 0, h_cap = 0;
  uint8_t* h_dst = nullptr;
  uint8_t* scratch = nullptr;
  SlotLayout L{};
  hipStream_t comp = nullptr, copy = nullptr;
  uint64_t* h_sizes = nullptr;  // pinned (from the pool): each chunk's size, copied from its slot
  std::vector<hipEvent_t> comp_done, copy_done;
  std::vector<uint64_t> chunk_bytes;
  uint64_t total = 0, copied = 0;
  int status = CDMA_OK;
  std::thread worker;
  bool joined = false;

  uint8_t* slot_stream(int s) const { return scratch + (uint64_t)s * L.slot_bytes; }
  uint8_t* slot_ws(int s) const { return slot_stream(s) + L.stream_bytes; }
  uint64_t* slot_size(int s) const { return reinterpret_cast<uint64_t*>(slot_ws(s) + L.ws_bytes); }

  int enqueue_compress(uint64_t k) {
    const int s = (int)(k % (uint64_t)slots);
    const uint64_t lo = k * chunk;
    const uint64_t len = n - lo < chunk ? n - lo : chunk;
    int rc = cdma_compress(algo, esz, src + lo * (uint64_t)esz, len, slot_stream(s), L.stream_bytes,
                           slot_size(s), slot_ws(s), L.ws_bytes, comp);
    if (rc != CDMA_OK) return rc;
    if (hipMemcpyAsync(h_sizes + k, slot_size(s), sizeof(uint64_t), hipMemcpyDeviceToHost, comp) != hipSuccess)
      return CDMA_ERR_HIP;
    return hipEventRecord(comp_done[s], comp) == hipSuccess ? CDMA_OK : CDMA_ERR_HIP;
  }

  void run() {
    if (hipSetDevice(device) != hipSuccess) {
      status = CDMA_ERR_HIP;
      return;
    }
    int rc = CDMA_OK;
    for (uint64_t k = 0; k < K && k < (uint64_t)slots && rc == CDMA_OK; ++k) rc = enqueue_compress(k);
    for (uint64_t k = 0; k < K && rc == CDMA_OK; ++k) {
      const int s = (int)(k % (uint64_t)slots);
      if (hipEventSynchronize(comp_done[s]) != hipSuccess) {
        rc = CDMA_ERR_HIP;
        break;
      }
      const uint64_t size = *static_cast<volatile uint64_t*>(h_sizes + k);
      if (size == CDMA_SIZE_INTERNAL_ERROR) {  // the compressor's scan did not complete
        rc = CDMA_ERR_INTERNAL;
        break;
      }
      if (size > h_cap - total) {
        rc = CDMA_ERR_CAPACITY;
        break;
      }
      if (size && hipMemcpyAsync(h_dst + total, slot_stream(s), size, hipMemcpyDeviceToHost, copy) != hipSuccess) {
        rc = CDMA_ERR_HIP;
        break;
      }
      if (hipEventRecord(copy_done[s], copy) != hipSuccess) {
        rc = CDMA_ERR_HIP;
        break;
      }
      chunk_bytes[k] = size;
      total += size;
      copied = k + 1;
      if (k + slots < K) {
        if (hipStreamWaitEvent(comp, copy_done[s], 0) != hipSuccess) {
          rc = CDMA_ERR_HIP;
          break;
        }
        rc = enqueue_compress(k + slots);
      }
    }
    // drain both streams: no staging slot or host byte may still be in use
    if (hipStreamSynchronize(comp) != hipSuccess && rc == CDMA_OK) rc = CDMA_ERR_HIP;
    if (hipStreamSynchronize(copy) != hipSuccess && rc == CDMA_OK) rc = CDMA_ERR_HIP;
    status = rc;
  }

  void join() {
    if (!joined && worker.joinable()) worker.join();
    joined = true;
  }

  ~cdma_offload_s() {
    join();
    for (hipEvent_t e : comp_done) (void)hipEventDestroy(e);
    for (hipEvent_t e : copy_done) (void)hipEventDestroy(e);
    cdma::pinned_release(h_sizes);
  }
};

extern "C" {

uint64_t cdma_offload_scratch_bytes(int algo, int esz, uint64_t chunk_elems, int slots) {
  if (slots < 1 || chunk_elems == 0 || cdma_max_compressed_bytes(algo, esz, chunk_elems) == 0) return 0;
  return slot_layout(algo, esz, chunk_elems).slot_bytes * (uint64_t)slots;
}

int cdma_offload_async(int algo, int esz, const void* d_src, uint64_t n, uint64_t chunk_elems, void* h_dst,
                       uint64_t h_capacity, void* d_scratch, uint64_t scratch_bytes, int slots,
                       void* compute_stream, void* copy_stream, cdma_offload_t* out) {
  if (!out) return CDMA_ERR_INVALID_ARG;
  *out = nullptr;
  if ((algo != CDMA_ALGO_ZVC && algo != CDMA_ALGO_RLE && algo != CDMA_ALGO_ZVCI) || (esz != 2 && esz != 4))
    return CDMA_ERR_INVALID_ARG;
  if (slots < 1 || chunk_elems == 0 || chunk_elems % 2048 != 0) return CDMA_ERR_INVALID_ARG;
  if (cdma_max_compressed_bytes(algo, esz, chunk_elems) == 0) return CDMA_ERR_INVALID_ARG;
  if (compute_stream == copy_stream) return CDMA_ERR_INVALID_ARG;
  if (n > 0) {
    if (!d_src || !h_dst || !d_scratch) return CDMA_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(d_src) & 15) || (reinterpret_cast<uintptr_t>(d_scratch) & (kAlign - 1)))
      return CDMA_ERR_INVALID_ARG;
    if (scratch_bytes < cdma_offload_scratch_bytes(algo, esz, chunk_elems, slots)) return CDMA_ERR_CAPACITY;
  }
  cdma_offload_s* h = new cdma_offload_s();
  h->algo = algo;
  h->esz = esz;
  h->slots = slots;
  h->src = static_cast<const uint8_t*>(d_src);
  h->n = n;
  h->chunk = chunk_elems;
  h->K = (n + chunk_elems - 1) / chunk_elems;
  h->h_dst = static_cast<uint8_t*>(h_dst);
  h->h_cap = h_capacity;
  h->scratch = static_cast<uint8_t*>(d_scratch);
  h->L = slot_layout(algo, esz, chunk_elems);
  h->comp = static_cast<hipStream_t>(compute_stream);
  h->copy = static_cast<hipStream_t>(copy_stream);
  h->chunk_bytes.assign(h->K, 0);
  bool ok = hipGetDevice(&h->device) == hipSuccess;
  if (ok && h->K > 0) {
    h->h_sizes = static_cast<uint64_t*>(cdma::pinned_acquire(h->K * sizeof(uint64_t)));
    ok = h->h_sizes != nullptr;
    for (int s = 0; ok && s < slots; ++s) {
      hipEvent_t a = nullptr, b = nullptr;
      ok = hipEventCreateWithFlags(&a, hipEventDisableTiming) == hipSuccess;
      if (ok) h->comp_done.push_back(a);
      ok = ok && hipEventCreateWithFlags(&b, hipEventDisableTiming) == hipSuccess;
      if (ok) h->copy_done.push_back(b);
    }
  }
  if (!ok) {
    delete h;
    return CDMA_ERR_HIP;
  }
  h->worker = std::thread([h] { h->run(); });
  *out = h;
  return CDMA_OK;
}

int cdma_offload_wait(cdma_offload_t h, uint64_t* total_bytes, uint64_t* chunk_bytes, uint64_t max_chunks,
                      uint64_t* n_chunks) {
  if (!h) return CDMA_ERR_INVALID_ARG;
  h->join();
  if (total_bytes) *total_bytes = h->total;
  if (n_chunks) *n_chunks = h->copied;
  if (chunk_bytes)
    for (uint64_t k = 0; k < h->copied && k < max_chunks; ++k) chunk_bytes[k] = h->chunk_bytes[k];
  return h->status;
}

void cdma_offload_destroy(cdma_offload_t h) { delete h; }

}  // extern "C"
