// kernels.hip -- instantiations and launchers of the gfx950 codec kernels.
#include <mutex>

#include "launch.hpp"
#include "zvc_compress.hpp"
#include "zvc_decompress.hpp"
#include "rle_kernels.hpp"
#include "zvci_kernels.hpp"

namespace cdma {

// 16-byte vectors per lane per tile: 4 -> 16 KB of input per workgroup.
#ifndef CDMA_ZVC_V
#define CDMA_ZVC_V 4
#endif
constexpr int kZvcV = CDMA_ZVC_V;

__global__ void fill_zero_u64_kernel(uint64_t* __restrict__ p, uint64_t count, uint64_t* __restrict__ extra) {
  const uint64_t i0 = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i0 == 0 && extra) *extra = 0;
  for (uint64_t i = i0; i < count; i += (uint64_t)gridDim.x * blockDim.x) p[i] = 0;
}

__global__ void store_u64_kernel(uint64_t* p, uint64_t v) {
  if (threadIdx.x == 0 && blockIdx.x == 0) *p = v;
}

// Read-ahead chunks of the ZVC expand pass: output bytes per chunk (0: no
// read-ahead workgroups) and read-ahead workgroups per chunk.
#ifndef CDMA_AHEAD_CHUNK_BYTES
#define CDMA_AHEAD_CHUNK_BYTES (1ull << 30)
#endif
#ifndef CDMA_AHEAD_GROUPS
#define CDMA_AHEAD_GROUPS 2048
#endif
constexpr uint32_t kAheadGroups = CDMA_AHEAD_GROUPS;
// Expand tiles of the previous chunk that follow a chunk's read-ahead group.
#ifndef CDMA_AHEAD_LEAD
#define CDMA_AHEAD_LEAD 0
#endif

// Warm the memory-side cache with the stream (see warm_whole); otherwise
// return at once.  Launched only when the output is large enough to warm.
constexpr unsigned kWarmGroups = 1024;
__global__ __launch_bounds__(256) void warm_stream_kernel(const uint8_t* __restrict__ src, uint64_t cap,
                                                          const uint64_t* __restrict__ src_bytes, uint64_t out) {
  const uint64_t claimed = src_bytes ? *src_bytes : cap;
  const uint64_t eff = claimed < cap ? claimed : cap;
  if (!warm_whole(eff, out)) return;
  warm_quads(src, 0, eff / 16, (uint64_t)blockIdx.x * 256 + threadIdx.x, (uint64_t)gridDim.x * 256);
}

static hipError_t warm_stream(const void* src, uint64_t cap, const uint64_t* src_bytes, uint64_t out,
                              hipStream_t s) {
  if (CDMA_WARM_BYTES == 0 || cap == 0 || out < (uint64_t)CDMA_WARM_MIN_OUT) return hipSuccess;
  warm_stream_kernel<<<kWarmGroups, 256, 0, s>>>(static_cast<const uint8_t*>(src), cap, src_bytes, out);
  return hipGetLastError();
}

// Clear the workspace header (ticket counter, start-mode words) and the
// per-tile aggregate words with a kernel (not a memset node), so the sequence
// stays correct if a caller captures it.
// The compressors report the stream size with atomic max, so *out_bytes is
// cleared here too.
static hipError_t clear_workspace(void* ws, uint64_t tiles, uint64_t* out_bytes, hipStream_t s) {
  const uint64_t words = (kWsHeader + 4 * tiles + 7) / 8;
  uint64_t blocks = (words + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  fill_zero_u64_kernel<<<(unsigned)blocks, 256, 0, s>>>(static_cast<uint64_t*>(ws), words, out_bytes);
  return hipGetLastError();
}

static_assert(4 * (kTicketClassWord0 + kTicketClassStride * kTicketClasses) <= kWsHeader,
              "ticket-class counters must lie in the workspace header");

static uint32_t* ws_counter(void* ws) { return static_cast<uint32_t*>(ws); }
static uint32_t* ws_agg(void* ws) {
  return reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(ws) + kWsHeader);
}

// ---- the workspace of the entry point that allocates nothing ----------------
//
// cdma_compress_noalloc takes its workspace from this array instead of from
// the caller: one copy per GPU, held until the process ends.  1 MiB covers
// the 2 KB header and one 32-bit aggregate per compress tile for every n that
// any compressor accepts (at most 2^31 / 15360 tiles).  Host code must not
// pass the array's name to a kernel: on the host it is a stand-in, not a
// device address; static_scratch() returns the address of the current
// device's copy, taken once per device with hipGetSymbolAddress.
constexpr uint64_t kStaticScratchBytes = 1ull << 20;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

uint64_t static_scratch_bytes() { return kStaticScratchBytes; }

hipError_t static_scratch(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* ptr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    ptr[dev] = p;
  }
  *out = ptr[dev];
  return hipSuccess;
}

uint64_t zvc_tiles(int esz, uint64_t n) {
  const uint64_t te = esz == 4 ? ZvcShape<4, kZvcV>::TE : ZvcShape<2, kZvcV>::TE;
  return (n + te - 1) / te;
}

uint64_t zvc_compress_tiles(int esz, uint64_t n) {
  const uint64_t te = esz == 4 ? ZvcCShape<4>::TE : ZvcCShape<2>::TE;
  return (n + te - 1) / te;
}

// Workgroups of `kernel` that fit on the current device at once (all CUs),
// cached per (kernel, device).
static uint64_t resident_groups(const void* kernel, int block = kBlock, int dyn_lds = 0) {
  struct Entry {
    const void* k;
    int dev;
    uint64_t groups;
  };
  static Entry cache[64];
  static int used = 0;
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < used; ++i)
    if (cache[i].k == kernel && cache[i].dev == dev) return cache[i].groups;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 1;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, dyn_lds) != hipSuccess || per_cu <= 0)
    per_cu = 1;
  const uint64_t groups = (uint64_t)cus * (uint64_t)per_cu;
  if (used < 64) cache[used++] = Entry{kernel, dev, groups};
  return groups;
}

template <int ESZ, int OP>
static hipError_t zvc_compress_t(const void* src, uint64_t n, void* act, void* dst, uint64_t* out_bytes, void* ws,
                                 hipStream_t s) {
  const uint64_t tiles = zvc_compress_tiles(ESZ, n);
  hipError_t e = clear_workspace(ws, tiles, out_bytes, s);
  if (e != hipSuccess) return e;
  if constexpr (OP == kOpNone) {
    // at most one tile per resident workgroup: one workgroup per tile, single pass
    auto one = zvc_compress_single_kernel<ESZ>;
    if (tiles <= resident_groups(reinterpret_cast<const void*>(one), kCBlock)) {
      one<<<(unsigned)tiles, kCBlock, 0, s>>>(static_cast<const uint8_t*>(src), n, static_cast<uint8_t*>(dst),
                                              out_bytes, ws_counter(ws), ws_agg(ws), (uint32_t)tiles);
      return hipGetLastError();
    }
  }
  // persistent grid: about one workgroup per CU, tiles static or by ticket
  auto kern = zvc_compress_kernel<ESZ, OP>;
  const uint64_t res = resident_groups(reinterpret_cast<const void*>(kern), kCBlock);
  const unsigned grid = (unsigned)(tiles < res ? tiles : res);
  kern<<<grid, kCBlock, 0, s>>>(static_cast<const uint8_t*>(src), n, static_cast<uint8_t*>(dst), out_bytes,
                                ws_counter(ws), ws_agg(ws), (uint32_t)tiles, static_cast<uint8_t*>(act));
  return hipGetLastError();
}

// Workgroups of the ZVC expand pass resident per CU.  Measured on the 4 GiB
// fp32 sweep with the count pass reading the masks without the non-temporal
// hint (percent of 8 TB/s at zero fraction 0 / 0.25 / 0.5 / 0.75 / 0.9 /
// 0.99 / 1, the last-level cache emptied by a 1 GiB read before each call):
// 7 per CU 77.2 / 74.5 / 75.2 / 73.8 / 65.9 / 70.2 / 76.7,
// 8 per CU (four-wave workgroups fill the CU) 76.3 / 73.9 / 73.6 / 73.3 /
// 66.0 / 75.0 / 76.8; with non-temporal mask reads 7 per CU gave 75.8 / 73.0
// / 73.5 / 72.5 / 66.7 / 64.9 / 71.5.  Fewer fall off steeply from s = 0.75
// up (5 per CU: 50 at s = 0.9 and 0.99).  Eight has the best floor across
// densities; the density is known only on the device, after the launch is
// fixed.  A build option.  fp16 (2^30 elements), 8 per CU: 74.3 / 72.6 /
// 73.1 / 70.8 / 61.2 / 64.8 / 73.3.
#ifndef CDMA_EXPAND_GROUPS
#define CDMA_EXPAND_GROUPS 8
#endif
#ifndef CDMA_EXPAND_GROUPS16
#define CDMA_EXPAND_GROUPS16 8
#endif
template <int ESZ>
constexpr int kExpandGroupsPerCU = ESZ == 4 ? CDMA_EXPAND_GROUPS : CDMA_EXPAND_GROUPS16;

// Dynamic LDS to reserve (and leave unused) so that at most `groups`
// workgroups of `kernel` fit in a CU's LDS; 0 if the kernel alone already
// limits it, or if the sizes cannot be read.  Cached per kernel and device.
static int expand_lds_pad(const void* kernel, int groups) {
  struct Entry {
    const void* k;
    int dev;
    int pad;
  };
  static Entry cache[16];
  static int used = 0;
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < used; ++i)
    if (cache[i].k == kernel && cache[i].dev == dev) return cache[i].pad;
  int pad = 0, lds_cu = 0;
  hipFuncAttributes attr;
  if (hipFuncGetAttributes(&attr, kernel) == hipSuccess &&
      hipDeviceGetAttribute(&lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) == hipSuccess &&
      lds_cu > 0) {
    // a per-group share between lds_cu/(groups+1) and lds_cu/groups, on a
    // 512-byte allocation boundary
    const int share = (lds_cu / groups) / 512 * 512;
    if (share * (groups + 1) > lds_cu && share > (int)attr.sharedSizeBytes) pad = share - (int)attr.sharedSizeBytes;
  }
  if (used < 16) cache[used++] = Entry{kernel, dev, pad};
  return pad;
}

template <int ESZ, int KQ>
static hipError_t zvc_decompress_kq(const void* src, uint64_t cap, const uint64_t* src_bytes, uint64_t n,
                                    void* dst, uint32_t* error, void* ws, hipStream_t s) {
  constexpr int WPT = ZvcShape<ESZ, kZvcV>::WPT;
  using C = ZvcScanShape<WPT, KQ>;
  const uint64_t tiles = zvc_tiles(ESZ, n);
  const uint64_t supers = (tiles + C::SUPER - 1) / C::SUPER;
  uint32_t* local = static_cast<uint32_t*>(ws);
  uint32_t* sup = local + tiles;
  hipError_t e;
  // read-ahead chunks (see zvc_expand_kernel): chunk_tiles tiles each
  constexpr uint64_t tile_bytes = (uint64_t)ZvcShape<ESZ, kZvcV>::TE * ESZ;
  const uint64_t chunk = CDMA_AHEAD_CHUNK_BYTES / tile_bytes;
  const uint64_t nchunks = chunk ? (tiles + chunk - 1) / chunk : 1;  // with read-ahead
  // a chunk is read ahead only when the stream can exceed what the count pass
  // leaves in the cache and still be a small share of the output
  const bool may_ahead = (uint64_t)ESZ * n / 100 * CDMA_WARM_MAX_PCT > (uint64_t)CDMA_WARM_BYTES;
  const uint32_t warm = chunk && may_ahead ? kAheadGroups : 0u;
  // read-ahead counters and flags, 128-byte aligned after sup[]
  uint32_t* sync = reinterpret_cast<uint32_t*>((reinterpret_cast<uintptr_t>(sup + supers + 1) + 127) & ~uintptr_t(127));
  zvc_count_kernel<WPT, KQ><<<(unsigned)supers, kBlock, 0, s>>>(static_cast<const uint8_t*>(src), cap, src_bytes,
                                                                      n, local, sup, error, (uint32_t)tiles,
                                                                      CDMA_WARM_BYTES > 0);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  zvc_scan_kernel<<<1, kScanBlock, 0, s>>>(sup, (uint32_t)supers, sync, warm ? (uint32_t)nchunks * kAheadSyncWords : 0u);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  auto kern = zvc_expand_kernel<ESZ, kZvcV>;
  const int pad = expand_lds_pad(reinterpret_cast<const void*>(kern), kExpandGroupsPerCU<ESZ>);
  const uint64_t window = resident_groups(reinterpret_cast<const void*>(kern), kBlock, pad);
  const uint64_t grid = tiles + (uint64_t)warm * nchunks;
  kern<<<(unsigned)grid, kBlock, pad, s>>>(static_cast<const uint8_t*>(src), cap, src_bytes, n,
                                           static_cast<uint8_t*>(dst), error, local, sup, (uint32_t)tiles,
                                           (uint32_t)C::SHIFT, warm ? (uint32_t)chunk : (uint32_t)tiles, warm,
                                           (uint32_t)window,
                                           (uint32_t)(CDMA_AHEAD_LEAD < chunk ? CDMA_AHEAD_LEAD : 0), sync);
  return hipGetLastError();
}

// Decode tiles up to which the count pass uses 4 KB super tiles (KQ = 1).
#ifndef CDMA_SMALL_SUPER_TILES
#define CDMA_SMALL_SUPER_TILES 16384
#endif

// decompress workspace: local[tiles], sup[supers + 1], then the read-ahead
// counters
template <int ESZ>
static hipError_t zvc_decompress_t(const void* src, uint64_t cap, const uint64_t* src_bytes, uint64_t n,
                                   void* dst, uint32_t* error, void* ws, hipStream_t s) {
  return zvc_tiles(ESZ, n) <= CDMA_SMALL_SUPER_TILES ? zvc_decompress_kq<ESZ, 1>(src, cap, src_bytes, n, dst, error, ws, s)
                                                      : zvc_decompress_kq<ESZ, 8>(src, cap, src_bytes, n, dst, error, ws, s);
}

// n = 0: the stream must be empty (ZVC) or the 8-byte zero index (RLE).
__global__ void empty_stream_check_kernel(const uint8_t* src, uint64_t cap, const uint64_t* src_bytes,
                                          uint32_t* error, int rle) {
  if (threadIdx.x != 0 || blockIdx.x != 0 || !error) return;
  const uint64_t claimed = src_bytes ? *src_bytes : cap;
  const uint64_t eff = claimed < cap ? claimed : cap;
  uint32_t e = 0;
  if (rle) {
    uint32_t idx = 0;
    for (uint64_t b = 0; b < 8 && b < eff; ++b) idx |= src[b];
    if (idx) e |= CDMA_E_INDEX;
    if (src_bytes && *src_bytes != 8) e |= CDMA_E_SIZE;
  } else if (src_bytes && *src_bytes != 0) {
    e |= CDMA_E_SIZE;
  }
  if (e) atomicOr(error, e);
}

hipError_t zvc_compress_launch(int esz, int op, const void* src, uint64_t n, void* act, void* dst,
                               uint64_t* out_bytes, void* ws, hipStream_t s) {
  if (n == 0) {
    store_u64_kernel<<<1, 64, 0, s>>>(out_bytes, 0);
    return hipGetLastError();
  }
  switch (op) {
    case kOpReluF32: return zvc_compress_t<4, kOpReluF32>(src, n, act, dst, out_bytes, ws, s);
    case kOpReluF16: return zvc_compress_t<2, kOpReluF16>(src, n, act, dst, out_bytes, ws, s);
    case kOpReluBF16: return zvc_compress_t<2, kOpReluBF16>(src, n, act, dst, out_bytes, ws, s);
    default:
      return esz == 4 ? zvc_compress_t<4, kOpNone>(src, n, nullptr, dst, out_bytes, ws, s)
                      : zvc_compress_t<2, kOpNone>(src, n, nullptr, dst, out_bytes, ws, s);
  }
}

hipError_t zvc_decompress_launch(int esz, const void* src, uint64_t cap, const uint64_t* src_bytes,
                                 uint64_t n, void* dst, uint32_t* error, void* ws, hipStream_t s) {
  if (n == 0) {
    empty_stream_check_kernel<<<1, 64, 0, s>>>(static_cast<const uint8_t*>(src), cap, src_bytes, error, 0);
    return hipGetLastError();
  }
  return esz == 4 ? zvc_decompress_t<4>(src, cap, src_bytes, n, dst, error, ws, s)
                  : zvc_decompress_t<2>(src, cap, src_bytes, n, dst, error, ws, s);
}

uint64_t rle_compress_tiles(int esz, uint64_t n) {
  const uint64_t te = esz == 4 ? RleCShape<4>::TE : RleCShape<2>::TE;
  return (n + te - 1) / te;
}

template <int ESZ, int OP>
static hipError_t rle_compress_t(const void* src, uint64_t n, void* act, void* dst, uint64_t* out_bytes, void* ws,
                                 hipStream_t s) {
  constexpr int block = RleCShape<ESZ>::BLOCK;
  const uint64_t tiles = rle_compress_tiles(ESZ, n);
  hipError_t e = clear_workspace(ws, tiles, out_bytes, s);
  if (e != hipSuccess) return e;
  auto kern = rle_compress_kernel<ESZ, OP>;
  const uint64_t res = resident_groups(reinterpret_cast<const void*>(kern), block);
  const unsigned grid = (unsigned)(tiles < res ? tiles : res);
  kern<<<grid, block, 0, s>>>(static_cast<const uint8_t*>(src), n, static_cast<uint8_t*>(dst), out_bytes,
                              ws_counter(ws), ws_agg(ws), (uint32_t)tiles, static_cast<uint8_t*>(act));
  return hipGetLastError();
}

template <int ESZ>
static hipError_t rle_decompress_t(const void* src, uint64_t cap, const uint64_t* src_bytes, uint64_t n,
                                   void* dst, uint32_t* error, hipStream_t s) {
  const uint64_t wins = (n + RleShape<ESZ>::E - 1) / RleShape<ESZ>::E;
  const uint64_t groups = (wins + kRleDecWaves - 1) / kRleDecWaves;
  const hipError_t e = warm_stream(src, cap, src_bytes, (uint64_t)ESZ * n, s);
  if (e != hipSuccess) return e;
  rle_decompress_kernel<ESZ><<<(unsigned)groups, kRleDecBlock, 0, s>>>(
      static_cast<const uint8_t*>(src), cap, src_bytes, n, static_cast<uint8_t*>(dst), error, (uint32_t)groups);
  return hipGetLastError();
}

// n = 0 still has a stream: the index of one window offset pair (8 bytes of zeros).
__global__ void rle_empty_kernel(uint8_t* dst, uint64_t* out_bytes) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    reinterpret_cast<uint32_t*>(dst)[0] = 0;
    reinterpret_cast<uint32_t*>(dst)[1] = 0;
    *out_bytes = 8;
  }
}

hipError_t rle_compress_launch(int esz, int op, const void* src, uint64_t n, void* act, void* dst,
                               uint64_t* out_bytes, void* ws, hipStream_t s) {
  if (n == 0) {
    rle_empty_kernel<<<1, 64, 0, s>>>(static_cast<uint8_t*>(dst), out_bytes);
    return hipGetLastError();
  }
  switch (op) {
    case kOpReluF32: return rle_compress_t<4, kOpReluF32>(src, n, act, dst, out_bytes, ws, s);
    case kOpReluF16: return rle_compress_t<2, kOpReluF16>(src, n, act, dst, out_bytes, ws, s);
    case kOpReluBF16: return rle_compress_t<2, kOpReluBF16>(src, n, act, dst, out_bytes, ws, s);
    default:
      return esz == 4 ? rle_compress_t<4, kOpNone>(src, n, nullptr, dst, out_bytes, ws, s)
                      : rle_compress_t<2, kOpNone>(src, n, nullptr, dst, out_bytes, ws, s);
  }
}

hipError_t rle_decompress_launch(int esz, const void* src, uint64_t cap, const uint64_t* src_bytes, uint64_t n,
                                 void* dst, uint32_t* error, void*, hipStream_t s) {
  if (n == 0) {
    empty_stream_check_kernel<<<1, 64, 0, s>>>(static_cast<const uint8_t*>(src), cap, src_bytes, error, 1);
    return hipGetLastError();
  }
  return esz == 4 ? rle_decompress_t<4>(src, cap, src_bytes, n, dst, error, s)
                  : rle_decompress_t<2>(src, cap, src_bytes, n, dst, error, s);
}

// Workspace bytes a compressor clears and uses: the header, then one 32-bit
// aggregate per compress tile.
uint64_t compress_workspace_bytes(int algo, int esz, uint64_t n) {
  const uint64_t t = algo == 0 ? zvc_compress_tiles(esz, n) : algo == 1 ? rle_compress_tiles(esz, n)
                                                                        : zvci_compress_tiles(esz, n);
  return kWsHeader + 4 * t;
}

uint64_t zvci_compress_tiles(int esz, uint64_t n) {
  const uint64_t te = esz == 4 ? ZviCShape<4>::TE : ZviCShape<2>::TE;
  return (n + te - 1) / te;
}

template <int ESZ>
static hipError_t zvci_compress_t(const void* src, uint64_t n, void* dst, uint64_t* out_bytes, void* ws,
                                  hipStream_t s) {
  constexpr int block = ZviCShape<ESZ>::BLOCK;
  const uint64_t tiles = zvci_compress_tiles(ESZ, n);
  hipError_t e = clear_workspace(ws, tiles, out_bytes, s);
  if (e != hipSuccess) return e;
  auto kern = zvci_compress_kernel<ESZ>;
  const uint64_t res = resident_groups(reinterpret_cast<const void*>(kern), block);
  const unsigned grid = (unsigned)(tiles < res ? tiles : res);
  kern<<<grid, block, 0, s>>>(static_cast<const uint8_t*>(src), n, static_cast<uint8_t*>(dst), out_bytes,
                              ws_counter(ws), ws_agg(ws), (uint32_t)tiles);
  return hipGetLastError();
}

// n = 0: the index of one entry (4 bytes of zeros).
__global__ void zvci_empty_kernel(uint8_t* dst, uint64_t* out_bytes) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    reinterpret_cast<uint32_t*>(dst)[0] = 0;
    *out_bytes = 4;
  }
}

hipError_t zvci_compress_launch(int esz, const void* src, uint64_t n, void* dst, uint64_t* out_bytes, void* ws,
                                hipStream_t s) {
  if (n == 0) {
    zvci_empty_kernel<<<1, 64, 0, s>>>(static_cast<uint8_t*>(dst), out_bytes);
    return hipGetLastError();
  }
  return esz == 4 ? zvci_compress_t<4>(src, n, dst, out_bytes, ws, s) : zvci_compress_t<2>(src, n, dst, out_bytes, ws, s);
}

// n = 0: the stream must be the 4-byte zero index.
__global__ void zvci_empty_check_kernel(const uint8_t* src, uint64_t cap, const uint64_t* src_bytes,
                                        uint32_t* error) {
  if (threadIdx.x != 0 || blockIdx.x != 0 || !error) return;
  const uint64_t claimed = src_bytes ? *src_bytes : cap;
  const uint64_t eff = claimed < cap ? claimed : cap;
  uint32_t idx = 0, e = 0;
  for (uint64_t b = 0; b < 4 && b < eff; ++b) idx |= src[b];
  if (idx) e |= CDMA_E_INDEX;
  if (src_bytes && *src_bytes != 4) e |= CDMA_E_SIZE;
  if (e) atomicOr(error, e);
}

hipError_t zvci_decompress_launch(int esz, const void* src, uint64_t cap, const uint64_t* src_bytes, uint64_t n,
                                  void* dst, uint32_t* error, hipStream_t s) {
  if (n == 0) {
    zvci_empty_check_kernel<<<1, 64, 0, s>>>(static_cast<const uint8_t*>(src), cap, src_bytes, error);
    return hipGetLastError();
  }
  const uint64_t E = 4096 / (uint64_t)esz;
  const uint64_t blocks = (n + E - 1) / E;
  const unsigned grid = (unsigned)((blocks + kWaves - 1) / kWaves);
  const hipError_t e = warm_stream(src, cap, src_bytes, (uint64_t)esz * n, s);
  if (e != hipSuccess) return e;
  if (esz == 4)
    zvci_decompress_kernel<4><<<grid, kBlock, 0, s>>>(static_cast<const uint8_t*>(src), cap, src_bytes, n,
                                                     static_cast<uint8_t*>(dst), error, grid);
  else
    zvci_decompress_kernel<2><<<grid, kBlock, 0, s>>>(static_cast<const uint8_t*>(src), cap, src_bytes, n,
                                                     static_cast<uint8_t*>(dst), error, grid);
  return hipGetLastError();
}

}  // namespace cdma
