// device_common.hpp -- wave-level primitives and the cross-workgroup offset
// machinery shared by the gfx950 codec kernels.
//
// The codec is stream compaction (compress) and expansion (decompress): the
// only arithmetic is integer compares, popcounts and prefix sums, which is
// what "Compressing DMA Engine: Leveraging Activation Sparsity for Training
// Deep Neural Networks" (§V.A Compression Algorithm, §V.B Compressing DMA
// Engine Architecture) names as the cost of its hardware units.  Here the
// prefix sums run at three levels: DPP scans inside a 64-lane wavefront, an
// LDS pass across the wavefronts of a workgroup, and, across workgroups, a
// chain sum per persistent workgroup over the 32-bit aggregates that every
// compress tile publishes (see chain_sum below).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cdma.h"

namespace cdma {

constexpr int kBlock = 256;  // threads per workgroup: 4 wave64s
constexpr int kWaves = kBlock / 64;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Streaming accesses.  The activation map is read once and the stream
// written once, so the bulk loads and stores carry the non-temporal hint:
// on gfx950 it lifts a pure streaming read from about 6.3 to 7.1 TB/s.
#ifndef CDMA_NT_LOAD
#define CDMA_NT_LOAD 1
#endif
#ifndef CDMA_NT_STORE
#define CDMA_NT_STORE 1
#endif

// Buffer resource word 3 for raw (untyped, unswizzled) buffer accesses on
// gfx9-family parts, and the cache-policy operand of buffer loads (bit 1 =
// non-temporal).
constexpr int kBufferFlags = 0x00020000;
constexpr int kLoadAux = CDMA_NT_LOAD ? 2 : 0;

template <typename T>
__device__ __forceinline__ T ld_stream(const T* p) {
  if constexpr (CDMA_NT_LOAD) return __builtin_nontemporal_load(p);
  else return *p;
}

// A load of data that is read again soon (the decoder's masks: the count
// pass reads them, then the expand pass): without the non-temporal hint the
// lines are kept by the memory-side cache, so the second read does not
// reach HBM and does not interleave reads with the expand pass's writes.
#ifndef CDMA_MASK_KEEP
#define CDMA_MASK_KEEP 1
#endif
template <typename T>
__device__ __forceinline__ T ld_keep(const T* p) {
  if constexpr (CDMA_MASK_KEEP) return *p;
  else return ld_stream(p);
}

template <typename T>
__device__ __forceinline__ void st_stream(T* p, T v) {
  if constexpr (CDMA_NT_STORE) __builtin_nontemporal_store(v, p);
  else *p = v;
}

// ---- lane helpers ----------------------------------------------------------

__device__ __forceinline__ uint32_t lane_id() {
  return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

// OR of the value across lane groups of 2, 4 and 8 (DPP, no LDS traffic).
__device__ __forceinline__ uint32_t or_lanes_xor1(uint32_t v) {
  return v | (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);  // quad_perm 1,0,3,2
}
__device__ __forceinline__ uint32_t or_lanes_xor2(uint32_t v) {
  return v | (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);  // quad_perm 2,3,0,1
}
__device__ __forceinline__ uint32_t or_lanes_half_mirror(uint32_t v) {
  return v | (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false);  // row_half_mirror
}

// OR over each aligned group of G lanes (G = 4 or 8); every lane of the group
// receives the result.
template <int G>
__device__ __forceinline__ uint32_t group_or(uint32_t v) {
  static_assert(G == 4 || G == 8, "lane group must be 4 or 8");
  v = or_lanes_xor1(v);
  v = or_lanes_xor2(v);
  if constexpr (G == 8) v = or_lanes_half_mirror(v);
  return v;
}

// Inclusive prefix sum across the 64 lanes of a wavefront (Hillis-Steele in
// rows of 16 with row_shr, then row_bcast:15 / row_bcast:31 to carry row
// totals).  Lanes whose DPP source is out of range add 0.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true);   // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true);   // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true);   // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true);   // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return v;
}

__device__ __forceinline__ uint32_t read_lane(uint32_t v, int lane) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, lane);
}

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Size a compressor reports when a chain sum hit its spin bound.
constexpr uint64_t kSizeInternalError = CDMA_SIZE_INTERNAL_ERROR;

// ---- tile offsets: per-workgroup chaining over published aggregates --------
//
// A persistent workgroup takes its tiles in increasing order, so the exclusive
// prefix of its tile t is the inclusive prefix of its own previous tile tp plus
// the aggregates of the tiles strictly between tp and t (of all tiles before t,
// for its first tile).  A tile therefore publishes only its aggregate, and no
// workgroup ever waits for another one's prefix, only for aggregates, which
// every tile publishes as soon as it is classified.  agg[t] holds the
// aggregate plus one (0 = not yet published), written and read with
// single-copy-atomic agent-scope 32-bit accesses; the workspace is cleared
// before each launch.

__device__ __forceinline__ void agg_publish(uint32_t* agg, uint32_t t, uint32_t v) {
  __hip_atomic_store(&agg[t], v + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t agg_load(const uint32_t* agg, uint64_t i) {
  return __hip_atomic_load(const_cast<uint32_t*>(agg) + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Upper bound on polling rounds of one chain sum.  A tile's aggregate appears
// a few microseconds after its ticket is drawn, so a healthy wait is a few
// rounds; the bound only turns an impossible wait into a reported error
// instead of a wave that never finishes.
constexpr uint32_t kChainSpinLimit = 1u << 21;

// Aggregate words read per lane per round: one round covers 64*kChainK tiles.
#ifndef CDMA_CHAIN_K
#define CDMA_CHAIN_K 4
#endif
constexpr int kChainK = CDMA_CHAIN_K;

struct ChainRound {
  uint32_t w[kChainK];
};

// Issue the reads of agg[lo + k*64 + lane] for the round starting at lo;
// slots at or past hi read as a published zero.  With lazy chain reads every
// slot issues a load (slots past hi read agg[hi - 1], whose value is ignored),
// so nothing consumes a value here and the wave does not wait for the round
// until chain_sum needs it.
#ifndef CDMA_CHAIN_LAZY
#define CDMA_CHAIN_LAZY 1
#endif
#ifndef CDMA_CHAIN_SUM32
#define CDMA_CHAIN_SUM32 0
#endif
__device__ __forceinline__ void chain_issue(const uint32_t* agg, uint64_t lo, uint64_t hi, ChainRound& r) {
  const uint32_t lane = lane_id();
#pragma unroll
  for (int k = 0; k < kChainK; ++k) {
    const uint64_t i = lo + (uint64_t)(k * 64) + lane;
    if constexpr (CDMA_CHAIN_LAZY) r.w[k] = agg_load(agg, i < hi ? i : (hi > 0 ? hi - 1 : 0));
    else r.w[k] = i < hi ? agg_load(agg, i) : 1u;
  }
}

// ---- tile assignment mode, decided once per launch --------------------------
//
// Static tiles (workgroup b takes b, b+G, b+2G, ...) need no ticket atomic:
// the one counter word taken by every workgroup is a contended atomic, about
// a tenth of the ZVC compressor's time when tiles are sparse.  (Its tiles all
// cost about the same; the run-length and interleaved compressors, whose tile
// costs vary, keep tickets, which balance the load: static tiles made them up
// to 6 % slower on dense inputs.)  But a workgroup may
// then wait for a tile whose owner has not been dispatched yet (other work can
// hold the CUs), which tickets never do.  Static is therefore used only when
// every workgroup of the grid has started: each counts itself in, the one that
// completes the count selects static, and one that has waited too long for
// that selects tickets, both by compare-and-swap from "undecided", so every
// workgroup follows the same choice.  The two words sit in the cleared
// workspace header after the ticket counter.
constexpr uint32_t kModeTickets = 1, kModeStatic = 2;
constexpr uint32_t kModeSpinLimit = 64;  // polls (each an agent-scope round trip) before choosing tickets

__device__ __forceinline__ uint32_t start_mode(uint32_t* counter) {
  uint32_t* started = counter + 16;
  uint32_t* mode = counter + 32;
  const uint32_t arrived = __hip_atomic_fetch_add(started, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1;
  if (arrived == gridDim.x) {
    uint32_t undecided = 0;
    __hip_atomic_compare_exchange_strong(mode, &undecided, kModeStatic, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
  }
  uint32_t spins = 0, m;
  while ((m = __hip_atomic_load(mode, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) == 0) {
    if (++spins > kModeSpinLimit) {
      uint32_t undecided = 0;
      __hip_atomic_compare_exchange_strong(mode, &undecided, kModeTickets, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_s_sleep(2);
  }
  return m;
}

// ---- warming the memory-side cache ------------------------------------------
//
// A decoder's HBM traffic is mostly its output; the few percent of stream
// reads mixed into that write stream cost far more than their bytes (on this
// GPU a write stream with 3 % reads from HBM runs about ten points of peak
// slower than one whose reads hit the 256 MB memory-side cache).  So when the
// whole stream fits in that cache (CDMA_WARM_BYTES) and is a small share of a
// large output (at most CDMA_WARM_MAX_PCT percent of at least
// CDMA_WARM_MIN_OUT bytes), the decoder first reads it once with caching
// loads (a pure read pass), and the decode's own reads then hit the cache.
// Outputs are written with non-temporal stores, which leave the cached
// stream in place.  Larger streams are not warmed whole (the decode would
// evict them before it reached them), and neither are streams that are a
// large share of their output or of a small output: there the extra pass
// costs more than it saves (the maps of a few hundred MB whose stream is half
// their size decoded up to 50 % slower with it).
#ifndef CDMA_WARM_BYTES
#define CDMA_WARM_BYTES (192ull << 20)
#endif
#ifndef CDMA_WARM_MAX_PCT
#define CDMA_WARM_MAX_PCT 20
#endif
#ifndef CDMA_WARM_MIN_OUT
#define CDMA_WARM_MIN_OUT (512ull << 20)
#endif

// Whether a stream of eff bytes decoding to out bytes is read ahead whole.
__host__ __device__ __forceinline__ bool warm_whole(uint64_t eff, uint64_t out) {
  return eff <= (uint64_t)CDMA_WARM_BYTES && out >= (uint64_t)CDMA_WARM_MIN_OUT &&
         eff * 100 <= out * CDMA_WARM_MAX_PCT;
}

// Read quads [q0, q1) of p: thread `start` of `stride` takes every
// stride-th quad, four loads in flight per trip.
__device__ __forceinline__ void warm_quads(const uint8_t* __restrict__ p, uint64_t q0, uint64_t q1, uint64_t start,
                                           uint64_t stride) {
  const u32x4* v = reinterpret_cast<const u32x4*>(p);
  u32x4 acc = {0u, 0u, 0u, 0u};
  uint64_t i = q0 + start;
  for (; i + 3 * stride < q1; i += 4 * stride) {
    const u32x4 a = v[i], b = v[i + stride], c = v[i + 2 * stride], d = v[i + 3 * stride];
    acc ^= a ^ b ^ c ^ d;
  }
  for (; i < q1; i += stride) acc ^= v[i];
  const uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
  asm volatile("" ::"v"(x));  // the loads are the point; keep them
}

// ---- XCD-aware tile order -------------------------------------------------
//
// Consecutive workgroups of a launch are spread over the GPU's XCDs round
// robin, and each XCD has its own L2.  A one-tile-per-workgroup decoder maps
// workgroup b to tile xcd_tile(b, G) instead, so that each XCD takes one
// contiguous range of tiles (a bijection of [0, G) for any G): neighbouring
// tiles, whose compressed data share cache lines when it is sparse, then meet
// in one L2.  Correctness does not depend on the dispatch order.
#ifndef CDMA_XCD_ORDER
#define CDMA_XCD_ORDER 1
#endif
constexpr uint32_t kXcds = 8;

__device__ __forceinline__ uint32_t xcd_tile(uint32_t b, uint32_t g) {
  if constexpr (!CDMA_XCD_ORDER) return b;
  const uint32_t q = g / kXcds, r = g % kXcds, x = b % kXcds, i = b / kXcds;
  return x * q + (x < r ? x : r) + i;
}

// ---- ticket classes -----------------------------------------------------------
//
// The run-length and interleaved compressors keep tickets (their tile costs
// vary), but once every workgroup of the grid has started (start_mode chose
// static) they spread the draws over up to kTicketClasses counters, each on a
// cache line of its own: workgroup b draws from class c = b % C and receives
// tiles c, c + C, c + 2C, ... in increasing order, so each counter takes a
// C-th of the atomics.  Progress: let u be the smallest tile whose aggregate
// is unpublished.  If u has been drawn, its holder is running and waits only
// for tiles below u before publishing it.  If not, every workgroup of u's
// class holds smaller tiles of that class, all published, so one of them
// finishes its iteration and draws again; the class has running workgroups
// because all of them have started.  Otherwise (not all started) the one
// counter is used, as its argument needs no co-residency.
constexpr uint32_t kTicketClasses = 8;
constexpr uint32_t kTicketClassWord0 = 256;   // first class counter: byte 1024 of the header
constexpr uint32_t kTicketClassStride = 32;   // words (128 bytes) from one class counter to the next

struct Tickets {
  uint32_t* ctr;
  uint32_t cls, ncls;
  // The counter value of a draw and the tile it stands for.  A caller that
  // draws ahead keeps the raw value and converts it where it uses the tile:
  // arithmetic on the atomic's result right after the draw would make the
  // wave wait for the atomic there.
  __device__ __forceinline__ uint32_t raw() const {
    return __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __device__ __forceinline__ uint32_t tile(uint32_t r) const { return cls + ncls * r; }
  __device__ __forceinline__ uint32_t draw() const { return tile(raw()); }
};

__device__ __forceinline__ Tickets ticket_source(uint32_t* counter, uint32_t mode) {
  Tickets k{counter, 0u, 1u};
  if (mode == kModeStatic) {
    k.ncls = gridDim.x < kTicketClasses ? gridDim.x : kTicketClasses;
    k.cls = blockIdx.x % k.ncls;
    k.ctr = counter + kTicketClassWord0 + kTicketClassStride * k.cls;
  }
  return k;
}

// Sum over tiles [lo, hi) of dec(aggregate), where r holds the first round
// (issued from lo).  Unpublished words are read again until they appear;
// further rounds are issued as needed.  Uniform result; *stuck is set (and the
// result meaningless) if the spin bound was hit.  Called by a whole wave.
template <bool kFirstRoundApart = false, typename Dec>
__device__ __forceinline__ uint64_t chain_sum(const uint32_t* agg, uint64_t lo, uint64_t hi, ChainRound& r,
                                              bool* stuck, Dec dec) {
  const uint32_t lane = lane_id();
  *stuck = false;
  uint64_t sum = 0, base = lo;
  uint32_t spins = 0;
  // Optionally the first round's check comes before the loop, where it
  // waits only for the round's own loads and what precedes them (the loop's
  // reloads make the compiler wait for every memory operation of the wave).
  if constexpr (kFirstRoundApart) {
    bool missing = false;
#pragma unroll
    for (int k = 0; k < kChainK; ++k) {
      if constexpr (CDMA_CHAIN_LAZY)
        if (base + (uint64_t)(k * 64) + lane >= hi) r.w[k] = 1u;
      missing |= r.w[k] == 0;
    }
    if (!__ballot(missing)) {
      uint64_t part = 0;
#pragma unroll
      for (int k = 0; k < kChainK; ++k) part += dec(r.w[k] - 1);
      sum += wave_sum_u64(part);
      base += 64 * kChainK;
      if (base >= hi) return sum;
      chain_issue(agg, base, hi, r);
    }
  }
  for (;;) {
    bool missing = false;
#pragma unroll
    for (int k = 0; k < kChainK; ++k) {
      if constexpr (CDMA_CHAIN_LAZY)
        if (base + (uint64_t)(k * 64) + lane >= hi) r.w[k] = 1u;
      missing |= r.w[k] == 0;
    }
    if (__ballot(missing)) {
      if (++spins > kChainSpinLimit) {
        *stuck = true;
        return 0;
      }
      __builtin_amdgcn_s_sleep(1);
#pragma unroll
      for (int k = 0; k < kChainK; ++k)
        if (r.w[k] == 0) r.w[k] = agg_load(agg, base + (uint64_t)(k * 64) + lane);
      continue;
    }
    using Part = decltype(dec(0u));
    if constexpr (sizeof(Part) == 4 && CDMA_CHAIN_SUM32) {
      // 32-bit decoded aggregates (nonzero counts): a round's sum fits in 32
      // bits, and a DPP scan reduces it without LDS round trips
      uint32_t part = 0;
#pragma unroll
      for (int k = 0; k < kChainK; ++k) part += dec(r.w[k] - 1);
      sum += read_lane(wave_incl_scan(part), 63);
    } else {
      uint64_t part = 0;
#pragma unroll
      for (int k = 0; k < kChainK; ++k) part += dec(r.w[k] - 1);
      sum += wave_sum_u64(part);
    }
    base += 64 * kChainK;
    if (base >= hi) return sum;
    chain_issue(agg, base, hi, r);
  }
}

}  // namespace cdma
