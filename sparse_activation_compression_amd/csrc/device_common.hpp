// device_common.hpp -- wave-level primitives and the decoupled-lookback scan
// shared by the gfx950 codec kernels.
//
// The codec is stream compaction (compress) and expansion (decompress): the
// only arithmetic is integer compares, popcounts and prefix sums, which is
// what "Compressing DMA Engine: Leveraging Activation Sparsity for Training
// Deep Neural Networks" (§V.A Compression Algorithm, §V.B Compressing DMA
// Engine Architecture) names as the cost of its hardware units.  Here the
// prefix sums run at three levels: DPP scans inside a 64-lane wavefront, an
// LDS pass across the 4 waves of a workgroup, and a decoupled lookback across
// workgroups through one 64-bit status word per tile in device memory.
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

template <typename T>
__device__ __forceinline__ T ld_stream(const T* p) {
  if constexpr (CDMA_NT_LOAD) return __builtin_nontemporal_load(p);
  else return *p;
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

// ---- decoupled lookback ----------------------------------------------------
//
// status[t] holds flag (2 bits) | value (62 bits) in one 64-bit word that is
// written and read with single-copy-atomic agent-scope accesses, so no fence
// is needed: the value travels inside the word that carries the flag.  The
// "value" is a sum that composes by 64-bit addition (a count, or two packed
// 31-bit counts).

constexpr uint64_t kFlagAggregate = 1ull << 62;  // tile's own total is known
constexpr uint64_t kFlagPrefix = 2ull << 62;     // inclusive prefix is known
constexpr uint64_t kValueMask = (1ull << 62) - 1;
constexpr uint64_t kSizeInternalError = CDMA_SIZE_INTERNAL_ERROR;

__device__ __forceinline__ void status_store(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t status_load(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Upper bound on polling rounds of one lookback.  A predecessor publishes its
// aggregate a few microseconds after it starts, so a healthy wait is a few
// rounds; the bound only turns an impossible wait into a reported error
// instead of a wave that never finishes.
constexpr uint32_t kLookbackSpinLimit = 1u << 21;

// Predecessors examined per lookback round: kLookbackK status words per lane.
// One round covers 64*kLookbackK tiles, so tiles can enter the pipeline at up
// to 64*kLookbackK per round-trip latency of a status read.
#ifndef CDMA_LOOKBACK_K
#define CDMA_LOOKBACK_K 4
#endif
constexpr int kLookbackK = CDMA_LOOKBACK_K;

// Called by all 64 lanes of one wavefront of tile t with the tile's own
// aggregate.  Publishes the aggregate, looks back over predecessors
// 64*kLookbackK at a time until one with a known inclusive prefix closes the
// window, publishes this tile's inclusive prefix and returns the exclusive
// prefix (uniform).  Every predecessor belongs to a workgroup that is resident
// and publishes its aggregate without waiting, so the loop ends; *stuck is
// set if the spin bound was hit anyway (the result is then meaningless).
//
// `after_issue` runs once, right after the first round's status loads are
// issued.  Vector-memory counters retire in order on this GPU, so loads the
// caller issues there (e.g. a prefetch) do not delay that first round.
struct NoOp {
  __device__ void operator()() const {}
};

template <typename F = NoOp>
__device__ __forceinline__ uint64_t lookback_exclusive(uint64_t* status, uint32_t t, uint64_t agg,
                                                       bool* stuck, F after_issue = F()) {
  const uint32_t lane = lane_id();
  *stuck = false;
  if (t == 0) {
    if (lane == 0) status_store(&status[0], kFlagPrefix | agg);
    after_issue();
    return 0;
  }
  if (lane == 0) status_store(&status[t], kFlagAggregate | agg);
  uint64_t excl = 0;
  int64_t base = (int64_t)t - 1;
  uint32_t spins = 0;
  bool first = true;
  for (;;) {
    // slot k*64 + lane looks at tile base - (k*64 + lane): nearest first
    uint64_t s[kLookbackK];
#pragma unroll
    for (int k = 0; k < kLookbackK; ++k) {
      const int64_t idx = base - (int64_t)(k * 64 + lane);
      s[k] = idx >= 0 ? status_load(&status[idx]) : kFlagPrefix;
    }
    if (first) {
      after_issue();
      first = false;
    }
    bool wait = false, closed = false;
    uint64_t sum = 0;
#pragma unroll
    for (int k = 0; k < kLookbackK; ++k) {
      if (wait || closed) break;
      const uint32_t flag = (uint32_t)(s[k] >> 62);
      const uint64_t pmask = __ballot(flag == 2);
      const uint64_t zmask = __ballot(flag == 0);
      const int p = pmask ? __ffsll((unsigned long long)pmask) - 1 : 64;  // nearest prefix
      const uint64_t need = p >= 63 ? ~0ull : ((2ull << p) - 1);          // lanes 0..p
      if (zmask & need) {
        wait = true;
      } else {
        sum += (int)lane <= p ? (s[k] & kValueMask) : 0;
        closed = p < 64;
      }
    }
    if (wait && !closed) {
      // partial progress is discarded: the next round re-reads the same window
      if (++spins > kLookbackSpinLimit) {
        *stuck = true;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
      continue;
    }
    excl += wave_sum_u64(sum);
    if (closed) break;
    base -= 64 * kLookbackK;
  }
  if (lane == 0) status_store(&status[t], kFlagPrefix | (excl + agg));
  return excl;
}

// ---- split lookback: issue a round early, resolve later ---------------------
//
// The pipelined compressor issues the first round for a tile before doing
// other work and resolves it afterwards, so the round trip of the status
// reads overlaps that work.  Publishing the tile's own flags is left to the
// caller.

struct LookbackRound {
  uint64_t s[kLookbackK];
};

// Issue the status reads of predecessors base, base-1, ..., base-64K+1.
__device__ __forceinline__ void lookback_issue(const uint64_t* status, int64_t base, LookbackRound& r) {
  const uint32_t lane = lane_id();
#pragma unroll
  for (int k = 0; k < kLookbackK; ++k) {
    const int64_t idx = base - (int64_t)(k * 64 + lane);
    r.s[k] = idx >= 0 ? status_load(&status[idx]) : kFlagPrefix;
  }
}

// Exclusive prefix of tile t >= 1 whose first round (base t-1) is already in
// r; further rounds are issued as needed.  Uniform result; *stuck as above.
__device__ __forceinline__ uint64_t lookback_resolve(const uint64_t* status, uint32_t t, LookbackRound& r,
                                                     bool* stuck) {
  const uint32_t lane = lane_id();
  *stuck = false;
  uint64_t excl = 0;
  int64_t base = (int64_t)t - 1;
  uint32_t spins = 0;
  for (;;) {
    bool wait = false, closed = false;
    uint64_t sum = 0;
#pragma unroll
    for (int k = 0; k < kLookbackK; ++k) {
      if (wait || closed) break;
      const uint32_t flag = (uint32_t)(r.s[k] >> 62);
      const uint64_t pmask = __ballot(flag == 2);
      const uint64_t zmask = __ballot(flag == 0);
      const int p = pmask ? __ffsll((unsigned long long)pmask) - 1 : 64;
      const uint64_t need = p >= 63 ? ~0ull : ((2ull << p) - 1);
      if (zmask & need) {
        wait = true;
      } else {
        sum += (int)lane <= p ? (r.s[k] & kValueMask) : 0;
        closed = p < 64;
      }
    }
    if (wait && !closed) {
      if (++spins > kLookbackSpinLimit) {
        *stuck = true;
        return excl;
      }
      __builtin_amdgcn_s_sleep(1);
      lookback_issue(status, base, r);
      continue;
    }
    excl += wave_sum_u64(sum);
    if (closed) return excl;
    base -= 64 * kLookbackK;
    lookback_issue(status, base, r);
  }
}

}  // namespace cdma
