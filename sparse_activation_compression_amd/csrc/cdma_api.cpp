// cdma_api.cpp -- the C ABI of libcdma: argument checks, sizing and dispatch.
//
// Every check that can be made on the host is made here, before anything is
// enqueued, so a bad call never reaches the GPU.
#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "cdma.h"
#include "launch.hpp"

namespace {

bool algo_ok(int algo) { return algo == CDMA_ALGO_ZVC || algo == CDMA_ALGO_RLE || algo == CDMA_ALGO_ZVCI; }
bool esz_ok(int esz) { return esz == 2 || esz == 4; }
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
uint64_t max_n(int algo) { return algo == CDMA_ALGO_RLE ? CDMA_RLE_MAX_N : CDMA_ZVC_MAX_N; }
uint64_t rle_window(int esz) { return 4096u / (unsigned)esz; }

// Whether compressing n elements writes stream bytes: every nonempty input
// does, and so does an empty one for the codecs whose stream opens with an
// index (RLE: 8 bytes, interleaved ZVC: 4 bytes).
bool writes_stream(int algo, uint64_t n) { return n > 0 || algo != CDMA_ALGO_ZVC; }

uint64_t tiles(int algo, int esz, uint64_t n) {
  if (algo == CDMA_ALGO_ZVC) return cdma::zvc_tiles(esz, n);
  return algo == CDMA_ALGO_RLE ? cdma::rle_compress_tiles(esz, n) : cdma::zvci_compress_tiles(esz, n);
}

}  // namespace

extern "C" {

uint64_t cdma_max_compressed_bytes(int algo, int esz, uint64_t n) {
  if (!algo_ok(algo) || !esz_ok(esz) || n > max_n(algo)) return 0;
  if (algo == CDMA_ALGO_ZVC) return 4 * ((n + 31) / 32) + (uint64_t)esz * n;
  const uint64_t wr = (n + rle_window(esz) - 1) / rle_window(esz);
  if (algo == CDMA_ALGO_ZVCI) return 4 * (wr + 1) + 4 * ((n + 31) / 32) + (uint64_t)esz * n;
  return 8 * (wr + 1) + 2 * (n + 2 * wr) + (uint64_t)esz * n;
}

uint64_t cdma_workspace_bytes(int algo, int esz, uint64_t n) {
  if (!algo_ok(algo) || !esz_ok(esz) || n > max_n(algo)) return 0;
  // counter and one scan status word per compress tile; ZVC decompress keeps a
  // value offset per (smaller) decompress tile in the same space
  const uint64_t t = tiles(algo, esz, n);
  return algo == CDMA_ALGO_ZVC ? cdma::kWsHeader + 12 * t + 16 : cdma::kWsHeader + 8 * t;
}

int cdma_compress(int algo, int esz, const void* d_src, uint64_t n, void* d_dst, uint64_t dst_capacity,
                  uint64_t* d_out_bytes, void* d_ws, uint64_t ws_bytes, void* stream) {
  if (!algo_ok(algo) || !esz_ok(esz) || n > max_n(algo)) return CDMA_ERR_INVALID_ARG;
  if (!d_out_bytes || !aligned(d_out_bytes, 8)) return CDMA_ERR_INVALID_ARG;
  if (writes_stream(algo, n) && (!d_dst || !aligned(d_dst, 16))) return CDMA_ERR_INVALID_ARG;
  if (dst_capacity < cdma_max_compressed_bytes(algo, esz, n)) return CDMA_ERR_CAPACITY;
  if (n > 0) {
    if (!d_src || !d_ws) return CDMA_ERR_INVALID_ARG;
    if (!aligned(d_src, 16) || !aligned(d_ws, 8)) return CDMA_ERR_INVALID_ARG;
    if (ws_bytes < cdma_workspace_bytes(algo, esz, n)) return CDMA_ERR_CAPACITY;
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e =
      algo == CDMA_ALGO_ZVC   ? cdma::zvc_compress_launch(esz, 0, d_src, n, nullptr, d_dst, d_out_bytes, d_ws, s)
      : algo == CDMA_ALGO_RLE ? cdma::rle_compress_launch(esz, 0, d_src, n, nullptr, d_dst, d_out_bytes, d_ws, s)
                              : cdma::zvci_compress_launch(esz, d_src, n, d_dst, d_out_bytes, d_ws, s);
  return e == hipSuccess ? CDMA_OK : CDMA_ERR_HIP;
}

int cdma_compress_noalloc(int algo, int esz, const void* d_src, uint64_t n, void* d_dst, uint64_t dst_capacity,
                          uint64_t* d_out_bytes, void* stream) {
  if (!algo_ok(algo) || !esz_ok(esz) || n > max_n(algo)) return CDMA_ERR_INVALID_ARG;
  if (!d_out_bytes || !aligned(d_out_bytes, 8)) return CDMA_ERR_INVALID_ARG;
  if (writes_stream(algo, n) && (!d_dst || !aligned(d_dst, 16))) return CDMA_ERR_INVALID_ARG;
  if (dst_capacity < cdma_max_compressed_bytes(algo, esz, n)) return CDMA_ERR_CAPACITY;
  if (n > 0 && (!d_src || !aligned(d_src, 16))) return CDMA_ERR_INVALID_ARG;
  if (cdma::compress_workspace_bytes(algo, esz, n) > cdma::static_scratch_bytes()) return CDMA_ERR_CAPACITY;
  void* ws = nullptr;
  if (n > 0 && cdma::static_scratch(&ws) != hipSuccess) return CDMA_ERR_HIP;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e =
      algo == CDMA_ALGO_ZVC   ? cdma::zvc_compress_launch(esz, 0, d_src, n, nullptr, d_dst, d_out_bytes, ws, s)
      : algo == CDMA_ALGO_RLE ? cdma::rle_compress_launch(esz, 0, d_src, n, nullptr, d_dst, d_out_bytes, ws, s)
                              : cdma::zvci_compress_launch(esz, d_src, n, d_dst, d_out_bytes, ws, s);
  return e == hipSuccess ? CDMA_OK : CDMA_ERR_HIP;
}

int cdma_relu_compress(int algo, int fmt, const void* d_src, uint64_t n, void* d_act, void* d_dst,
                       uint64_t dst_capacity, uint64_t* d_out_bytes, void* d_ws, uint64_t ws_bytes, void* stream) {
  if (fmt != CDMA_FMT_F32 && fmt != CDMA_FMT_F16 && fmt != CDMA_FMT_BF16) return CDMA_ERR_INVALID_ARG;
  const int esz = fmt == CDMA_FMT_F32 ? 4 : 2;
  if ((algo != CDMA_ALGO_ZVC && algo != CDMA_ALGO_RLE) || n > max_n(algo)) return CDMA_ERR_INVALID_ARG;
  if (!d_out_bytes || !aligned(d_out_bytes, 8)) return CDMA_ERR_INVALID_ARG;
  if (writes_stream(algo, n) && (!d_dst || !aligned(d_dst, 16))) return CDMA_ERR_INVALID_ARG;
  if (dst_capacity < cdma_max_compressed_bytes(algo, esz, n)) return CDMA_ERR_CAPACITY;
  if (n > 0) {
    if (!d_src || !d_ws) return CDMA_ERR_INVALID_ARG;
    if (!aligned(d_src, 16) || !aligned(d_ws, 8)) return CDMA_ERR_INVALID_ARG;
    if (d_act) {
      // the dense output is written while later tiles of the input are still
      // being read, so it must not overlap the input (or the stream)
      const uintptr_t a = reinterpret_cast<uintptr_t>(d_act), bytes = (uintptr_t)(n * (uint64_t)esz);
      const uintptr_t x = reinterpret_cast<uintptr_t>(d_src), y = reinterpret_cast<uintptr_t>(d_dst);
      if (!aligned(d_act, 16)) return CDMA_ERR_INVALID_ARG;
      if (a < x + bytes && x < a + bytes) return CDMA_ERR_INVALID_ARG;
      if (a < y + dst_capacity && y < a + bytes) return CDMA_ERR_INVALID_ARG;
    }
    if (ws_bytes < cdma_workspace_bytes(algo, esz, n)) return CDMA_ERR_CAPACITY;
  }
  const int op = fmt == CDMA_FMT_F32 ? 1 : fmt == CDMA_FMT_F16 ? 2 : 3;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = algo == CDMA_ALGO_ZVC
                           ? cdma::zvc_compress_launch(esz, op, d_src, n, d_act, d_dst, d_out_bytes, d_ws, s)
                           : cdma::rle_compress_launch(esz, op, d_src, n, d_act, d_dst, d_out_bytes, d_ws, s);
  return e == hipSuccess ? CDMA_OK : CDMA_ERR_HIP;
}

int cdma_decompress(int algo, int esz, const void* d_src, uint64_t src_capacity, const uint64_t* d_src_bytes,
                    uint64_t n, void* d_dst, uint32_t* d_error, void* d_ws, uint64_t ws_bytes, void* stream) {
  if (!algo_ok(algo) || !esz_ok(esz) || n > max_n(algo)) return CDMA_ERR_INVALID_ARG;
  if (d_src_bytes && !aligned(d_src_bytes, 8)) return CDMA_ERR_INVALID_ARG;
  if (d_error && !aligned(d_error, 4)) return CDMA_ERR_INVALID_ARG;
  // the stream is read whatever n is (an empty RLE or interleaved stream still
  // has its index, checked on the device)
  if (src_capacity > 0 && !d_src) return CDMA_ERR_INVALID_ARG;
  if (n > 0) {
    if (!d_dst || !d_ws) return CDMA_ERR_INVALID_ARG;
    if (!aligned(d_src, 16) || !aligned(d_dst, 16) || !aligned(d_ws, 8)) return CDMA_ERR_INVALID_ARG;
    if (ws_bytes < cdma_workspace_bytes(algo, esz, n)) return CDMA_ERR_CAPACITY;
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e =
      algo == CDMA_ALGO_ZVC
          ? cdma::zvc_decompress_launch(esz, d_src, src_capacity, d_src_bytes, n, d_dst, d_error, d_ws, s)
      : algo == CDMA_ALGO_RLE
          ? cdma::rle_decompress_launch(esz, d_src, src_capacity, d_src_bytes, n, d_dst, d_error, d_ws, s)
          : cdma::zvci_decompress_launch(esz, d_src, src_capacity, d_src_bytes, n, d_dst, d_error, s);
  return e == hipSuccess ? CDMA_OK : CDMA_ERR_HIP;
}

const char* cdma_status_string(int status) {
  switch (status) {
    case CDMA_OK: return "ok";
    case CDMA_ERR_INVALID_ARG: return "invalid argument";
    case CDMA_ERR_CAPACITY: return "buffer too small";
    case CDMA_ERR_CORRUPT: return "corrupt stream";
    case CDMA_ERR_HIP: return "HIP runtime error";
    case CDMA_ERR_INTERNAL: return "internal error";
    default: return "unknown status";
  }
}

int cdma_version(void) { return 100; }

}  // extern "C"
