// launch.hpp -- host-side entry points into the device code (kernels.hip).
// Arguments are already validated by the C ABI layer; these only size grids,
// clear workspaces and enqueue kernels on the given stream.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace cdma {

constexpr uint64_t kWsHeader = 2048;  // ticket counter, start-mode words, ticket-class counters

uint64_t zvc_tiles(int esz, uint64_t n);           // decompress tiles
uint64_t zvc_compress_tiles(int esz, uint64_t n);  // compress tiles (fewer, larger)
uint64_t rle_compress_tiles(int esz, uint64_t n);  // compress tiles (fewer, larger)
uint64_t zvci_compress_tiles(int esz, uint64_t n);
// header + one 32-bit aggregate per compress tile (algo 0 ZVC, 1 RLE, 2 ZVCI)
uint64_t compress_workspace_bytes(int algo, int esz, uint64_t n);

// The per-GPU static workspace of cdma_compress_noalloc: its size, and the
// address of the current device's copy.
uint64_t static_scratch_bytes();
hipError_t static_scratch(void** out);

// op: 0 = plain compression; 1/2/3 = ReLU of fp32/fp16/bf16 patterns coded
// (and stored densely to act unless it is null).
hipError_t zvc_compress_launch(int esz, int op, const void* src, uint64_t n, void* act, void* dst,
                               uint64_t* out_bytes, void* ws, hipStream_t s);
hipError_t zvc_decompress_launch(int esz, const void* src, uint64_t src_capacity, const uint64_t* src_bytes,
                                 uint64_t n, void* dst, uint32_t* error, void* ws, hipStream_t s);
hipError_t rle_compress_launch(int esz, int op, const void* src, uint64_t n, void* act, void* dst,
                               uint64_t* out_bytes, void* ws, hipStream_t s);
hipError_t rle_decompress_launch(int esz, const void* src, uint64_t src_capacity, const uint64_t* src_bytes,
                                 uint64_t n, void* dst, uint32_t* error, void* ws, hipStream_t s);

hipError_t zvci_compress_launch(int esz, const void* src, uint64_t n, void* dst, uint64_t* out_bytes, void* ws,
                                hipStream_t s);
hipError_t zvci_decompress_launch(int esz, const void* src, uint64_t src_capacity, const uint64_t* src_bytes,
                                  uint64_t n, void* dst, uint32_t* error, hipStream_t s);

}  // namespace cdma
