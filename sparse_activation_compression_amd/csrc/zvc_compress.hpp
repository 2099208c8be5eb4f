// zvc_compress.hpp -- ZVC compression for gfx950 (stream format in
// zvc_common.hpp): load -> per-lane nonzero bits -> window masks (DPP OR) and
// per-lane counts (DPP wave scan) -> LDS pass over the wave segments -> masks
// stored at their fixed place -> nonzeros compacted into LDS -> the tile's
// value offset from a per-workgroup chain sum over published tile aggregates
// -> realigned 16-byte stores.
#pragma once

#include "zvc_common.hpp"

namespace cdma {

// ---------------------------------------------------------------------------
// compress: persistent workgroups of data wavefronts plus one control wavefront
// ---------------------------------------------------------------------------
//
// A persistent grid of (about) one workgroup per CU takes its tiles in
// increasing order: static tiles (workgroup b takes b, b+G, b+2G, ...) when
// every workgroup of the grid is known to have started, else tiles drawn from
// a ticket counter (start_mode decides once per launch).  Waves 0..kDWaves-1
// move data; the last wave, the control wave, hands out tiles and computes
// tile offsets by chaining over published aggregates (see chain_sum).
// Vector-memory counters retire in order on this GPU, so a wave that had both
// prefetched a tile and issued status reads could not use the tile before the
// status reads came back; with the status traffic in a wave of its own, the
// data waves wait only for their own loads.  Iteration i of a workgroup holds
// tile t (loaded), tn (to prefetch) and the previous tile tp (nonzeros staged
// in LDS):
//   data waves:   classify t (window masks, nonzero counts) -> B1 -> store
//                 t's masks, compact t's nonzeros into LDS buffer i%2, issue
//                 tn's loads -> B2 -> store tp's staged values at the offset
//                 the control wave resolved;
//   control wave: B1 -> publish t's aggregate (static tiles) -> hand the data
//                 waves the next tile and, with tickets, draw the one after it
//                 and publish -> finish tp's chain sum (aggregates of the tiles
//                 between this workgroup's previous tile and tp, read one
//                 iteration earlier) -> B2 -> issue the first round of t's
//                 chain sum.
// The ticket counter is one word hit by every workgroup, so its atomic comes
// back slower than a load; drawing right after the hand-over gives it a whole
// iteration, and static tiles need none.
// The size is reported with 64-bit atomic max operations on a word cleared
// before the launch: the last tile writes the stream size and a control wave
// whose chain sum hit the spin bound writes the all-ones error value, which
// wins whatever the order.  (Such a sum returns an under-estimate, so every
// store still lands inside the stream's bounds.)
// Progress: every workgroup takes its tiles in increasing order and publishes
// a tile's aggregate in the iteration that classifies it, before that
// iteration waits on any other workgroup.  With tickets, a ticket is drawn only by a
// running workgroup, so the smallest tile whose aggregate is unpublished is
// held by a running workgroup that waits only for aggregates of smaller tiles,
// all published: no co-residency is assumed and every chain sum ends.  Static
// tiles are used only once every workgroup has started, so the owner of that
// smallest tile is running too.

#ifndef CDMA_CBLOCK
#define CDMA_CBLOCK 1024
#endif
constexpr int kCBlock = CDMA_CBLOCK;
constexpr int kCWaves = kCBlock / 64;
constexpr int kDWaves = kCWaves - 1;  // data wavefronts; the last one is the control wave
constexpr int kDThreads = kDWaves * 64;

template <int ESZ>
struct ZvcCShape {
  static constexpr int V = 4;                      // 16-byte vectors per lane
  static constexpr int EPL = 16 / ESZ;
  static constexpr int TE = kDThreads * V * EPL;   // elements per tile (60 KB)
  static constexpr int LPW = 32 / EPL;
  static constexpr int WPT = TE / 32;              // windows per tile
  static constexpr int SEG = kDWaves * V;          // wave segments per tile
  static constexpr int STAGE = TE * ESZ + 16;
  static_assert(SEG <= 64, "one lane per wave segment in the tile scan");
  static_assert(WPT <= kDThreads, "one mask store per data thread");
};

template <int ESZ>
struct ZvcCLds {
  using S = ZvcCShape<ESZ>;
  uint64_t excl;         // exclusive prefix of the tile being stored
  uint32_t total[2];     // nonzeros held in stage[b]
  uint32_t next;         // ticket handed from the control wave to the data waves
  uint32_t mode;         // kModeStatic or kModeTickets (start_mode)
  uint32_t init[3];      // the first three tickets
  uint32_t tot[S::SEG];
  uint32_t mask[S::WPT];
  __attribute__((aligned(16))) uint8_t stage[2][S::STAGE];
};

template <int ESZ>
__device__ __forceinline__ void zvc_c_load_full(u32x4 (&v)[ZvcCShape<ESZ>::V], const uint8_t* __restrict__ src,
                                                uint32_t t, int wave, int lane) {
  using S = ZvcCShape<ESZ>;
  const uint8_t* p = src + (uint64_t)t * (S::TE * ESZ);  // uniform tile base
  uint32_t o = (uint32_t)((wave * S::V * 64 + lane) * 16);
  asm volatile("" : "+v"(o));  // keep base + o from being hoisted into a 64-bit register pair
#pragma unroll
  for (int j = 0; j < S::V; ++j) v[j] = ld_stream(reinterpret_cast<const u32x4*>(p + o + j * 1024));
}

template <int ESZ>
__device__ __forceinline__ void zvc_c_load_bounded(u32x4 (&v)[ZvcCShape<ESZ>::V], const uint8_t* __restrict__ src,
                                                   uint64_t n, uint32_t t, int wave, int lane) {
  using S = ZvcCShape<ESZ>;
  const uint64_t e_tile = (uint64_t)t * S::TE;
#pragma unroll
  for (int j = 0; j < S::V; ++j) {
    const uint32_t c = (uint32_t)((wave * S::V + j) * 64 + lane);
    v[j] = load_vec<ESZ>(src, e_tile + (uint64_t)c * S::EPL, n);
  }
}

// Apply the epilogue OP to a classified tile's vectors in place and, if act is
// given, store them densely at the places they were loaded from.
template <int ESZ, int OP>
__device__ __forceinline__ void zvc_c_epilogue(u32x4 (&v)[ZvcCShape<ESZ>::V], uint8_t* __restrict__ act,
                                               uint64_t n, uint32_t t, bool full_tile, int wave, int lane) {
  using S = ZvcCShape<ESZ>;
#pragma unroll
  for (int j = 0; j < S::V; ++j) v[j] = apply_op<OP>(v[j]);
  if (!act) return;
  if (full_tile) {
    uint8_t* p = act + (uint64_t)t * (S::TE * ESZ);
    uint32_t o = (uint32_t)((wave * S::V * 64 + lane) * 16);
    asm volatile("" : "+v"(o));
#pragma unroll
    for (int j = 0; j < S::V; ++j) st_stream(reinterpret_cast<u32x4*>(p + o + j * 1024), v[j]);
  } else {
    const uint64_t e_tile = (uint64_t)t * S::TE;
#pragma unroll
    for (int j = 0; j < S::V; ++j) {
      const uint32_t c = (uint32_t)((wave * S::V + j) * 64 + lane);
      store_vec<ESZ>(act, e_tile + (uint64_t)c * S::EPL, n, v[j]);
    }
  }
}

// One pipeline iteration (see above).  Returns the ticket the data waves
// prefetch in the next iteration, with the workgroup synchronised.
template <int ESZ, int OP>
__device__ __forceinline__ uint32_t zvc_c_iteration(ZvcCLds<ESZ>& L, u32x4 (&cur)[ZvcCShape<ESZ>::V],
                                                    u32x4 (&nxt)[ZvcCShape<ESZ>::V], ChainRound& cr,
                                                    uint64_t& chain_lo, uint64_t& P, uint32_t& pend, uint32_t t,
                                                    uint32_t tn, uint32_t tp, int buf,
                                                    uint32_t full, uint64_t W, const uint8_t* __restrict__ src,
                                                    uint64_t n, uint8_t* __restrict__ dst,
                                                    uint64_t* __restrict__ out_bytes, uint32_t* __restrict__ agg,
                                                    uint32_t* __restrict__ counter, uint32_t num_tiles,
                                                    uint8_t* __restrict__ act, int tid, int wave, int lane,
                                                    bool stat) {
  using S = ZvcCShape<ESZ>;
  constexpr int V = S::V;
  const bool have_cur = t < num_tiles;
  const bool have_prev = tp < num_tiles;
  const bool data = wave < kDWaves;

  uint32_t bits[V], ex[V];
  if (data && have_cur) {
    if (t >= full) {  // the one partial tile: load bounded, drain so nothing stays pending on cur
      zvc_c_load_bounded<ESZ>(cur, src, n, t, wave, lane);
      __builtin_amdgcn_s_waitcnt(0);
    }
    if constexpr (OP != kOpNone) zvc_c_epilogue<ESZ, OP>(cur, act, n, t, t < full, wave, lane);
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const uint32_t c = (uint32_t)((wave * V + j) * 64 + lane);
      bits[j] = vec_nz_bits<ESZ>(cur[j]);
      const uint32_t m = group_or<S::LPW>(bits[j] << ((lane % S::LPW) * S::EPL));
      if (lane % S::LPW == 0) L.mask[c / S::LPW] = m;
      const uint32_t cnt = (uint32_t)__builtin_popcount(bits[j]);
      const uint32_t inc = wave_incl_scan(cnt);
      ex[j] = inc - cnt;
      if (lane == 63) L.tot[wave * V + j] = inc;
    }
  }
  __syncthreads();

  if (data) {
    if (have_cur) {
      // segment bases: lane l of every data wave scans the segment totals
      const uint32_t x = lane < S::SEG ? L.tot[lane] : 0u;
      const uint32_t inc = wave_incl_scan(x);
      if (tid < S::WPT) {
        const uint64_t g = (uint64_t)t * S::WPT + tid;
        if (g < W) reinterpret_cast<uint32_t*>(dst)[g] = L.mask[tid];
      }
      uint8_t* st = L.stage[buf];
#pragma unroll
      for (int j = 0; j < V; ++j) {
        uint32_t pos = ESZ * (read_lane(inc - x, wave * V + j) + ex[j]);
#pragma unroll
        for (int k = 0; k < S::EPL; ++k) {
          if ((bits[j] >> k) & 1u) {
            store_elem<ESZ>(st + pos, vec_elem<ESZ>(cur[j], k));
            pos += ESZ;
          }
        }
      }
      if (tn < full) zvc_c_load_full<ESZ>(nxt, src, tn, wave, lane);
    }
  } else {
    // control wave
    // publish t's aggregate: every other workgroup's chain sum may be waiting
    // for it.  Static tiles publish before anything else; with tickets the
    // hand-over below has to wait for the ticket anyway, and the aggregate
    // follows it (waiting there would also wait for this store).
    const uint32_t T = read_lane(wave_incl_scan(lane < S::SEG ? L.tot[lane] : 0u), 63);
    if (stat && have_cur && lane == 0) {
      L.total[buf] = T;
      agg_publish(agg, t, T);
    }
    // what this wave issued last iteration (chain round, ticket) must be back
    // before the hand-over; waiting here on every path keeps the compiler from
    // waiting again after the ticket drawn next
    __builtin_amdgcn_s_waitcnt(0);
    if (lane == 0) L.next = pend;
    if (have_cur) {
      if (stat) {
        pend += gridDim.x;
      } else if (lane == 0) {
        // the next ticket goes out now and has a whole iteration to come back
        pend = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        L.total[buf] = T;
        agg_publish(agg, t, T);
      }
    }
    if (have_prev) {
      bool stuck = false;
      const uint64_t X = P + chain_sum(agg, chain_lo, tp, cr, &stuck, [](uint32_t v) { return (uint64_t)v; });
      if (lane == 0) {
        L.excl = X;
        if (stuck) atomicMax(reinterpret_cast<unsigned long long*>(out_bytes), kSizeInternalError);
      }
      P = X + L.total[buf ^ 1];  // tp's inclusive prefix
    }
  }
  __syncthreads();

  if (data) {
    if (have_prev) {
      const uint32_t T = L.total[buf ^ 1];
      const uint64_t A = 4 * W + (uint64_t)ESZ * L.excl;
      store_staged<ESZ, kDThreads>(L.stage[buf ^ 1], ESZ * T, A, dst, tid);
      if (tp == num_tiles - 1 && tid == 0)
        atomicMax(reinterpret_cast<unsigned long long*>(out_bytes), A + (uint64_t)ESZ * T);
    }
  } else if (have_cur) {
    // the first round of t's chain sum goes out while the data waves store,
    // late enough that the tiles drawn just before t are mostly classified
    chain_lo = have_prev ? (uint64_t)tp + 1 : 0;
    chain_issue(agg, chain_lo, t, cr);
  }
  return __builtin_amdgcn_readfirstlane(L.next);  // uniform: keeps tile bases in SGPRs
}

// OP: epilogue applied to the input before it is coded (kOpNone = plain
// compression); act: optional dense output of the epilogue (OP != kOpNone).
template <int ESZ, int OP>
__global__ __launch_bounds__(kCBlock) void zvc_compress_kernel(
    const uint8_t* __restrict__ src, uint64_t n, uint8_t* __restrict__ dst,
    uint64_t* __restrict__ out_bytes, uint32_t* __restrict__ counter, uint32_t* __restrict__ agg,
    uint32_t num_tiles, uint8_t* __restrict__ act) {
  using S = ZvcCShape<ESZ>;
  __shared__ ZvcCLds<ESZ> L;
  const int tid = threadIdx.x;
  const int lane = (int)lane_id();
  const int wave = tid >> 6;
  const uint64_t W = (n + 31) / 32;
  const uint32_t full = (uint32_t)(n / S::TE);  // tiles with no element past n
  // the fused epilogue also streams the dense activation out, which makes its
  // tiles bandwidth-bound; tickets balance them better (static was 2-5 % slower)
  if (tid == 0) L.mode = OP == kOpNone ? start_mode(counter) : kModeTickets;
  __syncthreads();
  const bool stat = OP == kOpNone && __builtin_amdgcn_readfirstlane(L.mode) == kModeStatic;
  if (tid < 3 * 64 && lane == 0)
    L.init[wave] = stat ? blockIdx.x + wave * gridDim.x
                        : __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  // the first three tickets in increasing order: classify, prefetch, hand over
  const uint32_t a = __builtin_amdgcn_readfirstlane(L.init[0]);
  const uint32_t b = __builtin_amdgcn_readfirstlane(L.init[1]);
  const uint32_t c = __builtin_amdgcn_readfirstlane(L.init[2]);
  const uint32_t lo = min(a, min(b, c)), hi = max(a, max(b, c));
  uint32_t t = lo;
  uint32_t tn = a + b + c - lo - hi;
  uint32_t pend = hi;        // meaningful in the control wave only
  uint32_t tp = num_tiles;   // tile to store (none yet)
  u32x4 ra[S::V], rb[S::V];
  ChainRound cr;           // control wave: chain sum in flight
  uint64_t chain_lo = 0;   // control wave: first tile of that sum
  uint64_t P = 0;          // control wave: inclusive prefix of the last resolved tile
  if (wave < kDWaves && t < full) zvc_c_load_full<ESZ>(ra, src, t, wave, lane);
  // two iterations per trip so the register sets swap roles without copies;
  // an iteration with no tile left to classify only stores the last one
  for (;;) {
    uint32_t tnn = zvc_c_iteration<ESZ, OP>(L, ra, rb, cr, chain_lo, P, pend, t, tn, tp, 0, full, W, src, n, dst,
                                            out_bytes, agg, counter, num_tiles, act, tid, wave, lane, stat);
    if (t >= num_tiles) break;
    tp = t;
    t = tn;
    tn = tnn;
    tnn = zvc_c_iteration<ESZ, OP>(L, rb, ra, cr, chain_lo, P, pend, t, tn, tp, 1, full, W, src, n, dst,
                                   out_bytes, agg, counter, num_tiles, act, tid, wave, lane, stat);
    if (t >= num_tiles) break;
    tp = t;
    t = tn;
    tn = tnn;
  }
}

}  // namespace cdma
