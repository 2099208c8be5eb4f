// zvc_compress.hpp -- ZVC compression for gfx950 (stream format in
// zvc_common.hpp): load -> per-lane nonzero bits -> window masks (DPP OR) and
// per-lane counts (one packed DPP wave scan) -> LDS pass over the wave
// segments -> masks stored at their fixed place -> nonzeros compacted into LDS
// -> the tile's value offset from a per-workgroup chain sum over published
// tile aggregates -> realigned 16-byte stores.
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
// data waves wait only for their own loads.
//
// A tile passes through three iterations of its workgroup: iteration i
// classifies tile t_i, iteration i+1 compacts its nonzeros into LDS stage
// buffer i%2, iteration i+2 stores them.  Two stage buffers suffice, since the
// store of t_{i-2} precedes the compaction of t_i into the same buffer by a
// barrier.  The value offset of t_{i-2} needs the aggregates of every tile
// before it; those of the tiles classified alongside it by other workgroups
// are published in their iteration i-2, and this workgroup reads them in its
// iteration i-1 and sums them at the start of iteration i: a whole iteration
// of slack, so a workgroup that runs a little behind the others rarely makes
// another wait.  Iteration i (buffer b = i%2):
//   phase X  data waves:   compact t_{i-1} into stage[b^1]; issue the loads
//                          of t_{i+1} into the registers t_{i-1} held; wait
//                          for t_i (loaded one iteration earlier) and
//                          classify it (window masks, nonzero counts)
//            control wave: finish t_{i-2}'s chain sum -> its value offset
//   B1
//   phase Y  data waves:   segment bases of t_i; store t_{i-2}'s staged
//                          values from stage[b]
//            control wave: hand the data waves the tile they load next
//                          iteration (drawing a ticket when tiles are not
//                          static), issue the first round of t_{i-1}'s chain
//                          sum, publish t_i's aggregate, store t_i's masks
//                          (16-bit elements and the fused epilogue:
//                          publish and masks first)
//   B2
// The loads of t_{i+1} are issued by every wave on every path (the control
// wave's and a missing tile's cover no bytes), so the compiler sees the same
// loads after the other register set on every path and waits only for that
// set when it classifies.  For the same reason the control wave's aggregate
// and mask stores come after its chain loads and are a fixed number of buffer
// stores: memory operations retire in issue order, and a chain sum that
// waited for them as well (its round's loads behind the stores) took a store's
// latency every iteration (fp32, 4 GiB: 71.3 against 68.0 % of 8 TB/s at
// s = 0.99, 74.8 against 69.7 % at s = 1).  With 16-bit elements the
// masks' four quads per lane would not fit in registers beside the chain
// words, so that order is kept for 32-bit elements.
// The size is reported with 64-bit atomic max operations on a word cleared
// before the launch: the last tile writes the stream size and a control wave
// whose chain sum hit the spin bound writes the all-ones error value, which
// wins whatever the order.  (Such a sum returns an under-estimate, so every
// store still lands inside the stream's bounds.)
// Progress: every workgroup takes its tiles in increasing order and publishes
// a tile's aggregate in the iteration that classifies it.  The only wait on
// other workgroups, in phase X of iteration i, is for aggregates of tiles
// before t_{i-2}; by then the workgroup has published every tile up to
// t_{i-1}.  So the smallest unpublished tile u is held by a workgroup that
// waits only for tiles below u, all published, and publishes u one phase
// later.  With tickets, a ticket is drawn only by a running workgroup, so no
// co-residency is assumed; static tiles are used only once every workgroup
// has started, so the owner of u is running too.

constexpr int kCBlock = 1024;
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
  uint64_t excl;         // value offset of the tile stored this iteration
  uint32_t next;         // tile handed from the control wave to the data waves
  uint32_t mode;         // kModeStatic or kModeTickets (start_mode)
  uint32_t init[3];      // the first tickets
  uint32_t tot[S::SEG];
  uint32_t dump[64];     // one word per lane for the 32-bit compaction's discarded writes
  __attribute__((aligned(16))) uint32_t mask[S::WPT];
  __attribute__((aligned(16))) uint8_t stage[2][S::STAGE];
};

// What a data lane keeps of a classified tile until it is compacted, packed
// into bit fields to leave registers for the two tiles in flight: per row j
// (16-byte vector) the element nonzero bits (EPL bits at EPL*j of bits), the
// nonzeros of the row before this lane (F bits at F*(j%PER) of ex[j/PER])
// and the nonzeros of the tile before the row (16 bits at 16*(j%2) of
// base[j/2]; a tile holds fewer than 2^16 elements).
template <int EPL, int V>
struct ZvcRows {
  static constexpr int F = EPL <= 4 ? 8 : 16;
  static constexpr int PER = 32 / F;
  static_assert(EPL * V <= 32 && V % PER == 0 && V % 2 == 0, "row fields must fit");
  uint32_t bits;
  uint32_t ex[V / PER];
  uint32_t base[V / 2];
  __device__ __forceinline__ uint32_t bits_of(int j) const { return __builtin_amdgcn_ubfe(bits, EPL * j, EPL); }
  __device__ __forceinline__ uint32_t ex_of(int j) const { return __builtin_amdgcn_ubfe(ex[j / PER], F * (j % PER), F); }
  __device__ __forceinline__ uint32_t base_of(int j) const { return __builtin_amdgcn_ubfe(base[j / 2], 16 * (j % 2), 16); }
};

// Load tile t into v.  A buffer resource covers exactly the tile when it is
// full (valid) and nothing otherwise, so an invalid tile's loads return zeros
// without touching memory.  The loads are therefore issued on every path,
// which lets the compiler count precisely which loads are still in flight
// when the registers are next read (a load skipped on some path makes it wait
// for everything).  valid must be wave-uniform.
template <int ESZ>
__device__ __forceinline__ void zvc_c_load_full(u32x4 (&v)[ZvcCShape<ESZ>::V], const uint8_t* __restrict__ src,
                                                uint32_t t, bool valid, int wave, int lane) {
  using S = ZvcCShape<ESZ>;
  const uint8_t* p = src + (uint64_t)t * (S::TE * ESZ);  // uniform tile base
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p), (short)0, valid ? S::TE * ESZ : 0, kBufferFlags);
  const uint32_t o = (uint32_t)((wave * S::V * 64 + lane) * 16);
#pragma unroll
  for (int j = 0; j < S::V; ++j) v[j] = __builtin_amdgcn_raw_buffer_load_b128(r, o + j * 1024, 0, kLoadAux);
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

// Classify the tile held in v (data waves): its window masks go to L.mask,
// each wave row's nonzero count to L.tot, and the lane's per-row bits and
// in-row prefixes to R.
template <int ESZ>
__device__ __forceinline__ void zvc_c_classify(ZvcCLds<ESZ>& L, const u32x4 (&v)[ZvcCShape<ESZ>::V],
                                               ZvcRows<ZvcCShape<ESZ>::EPL, ZvcCShape<ESZ>::V>& R, int wave, int lane) {
  using S = ZvcCShape<ESZ>;
  constexpr int V = S::V;
  if constexpr (ESZ == 4) {
    // each lane's bits land at their window-mask position directly, and the
    // V rows' counts are scanned as one packed word
    const uint32_t sh = (uint32_t)((lane % S::LPW) * S::EPL);
    uint32_t cnt[V], ex[V], tot[V];
    R.bits = 0;
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const uint32_t c = (uint32_t)((wave * V + j) * 64 + lane);
      const uint32_t m = vec_nz_at<ESZ>(v[j], sh);
      const uint32_t win = group_or<S::LPW>(m);
      if (lane % S::LPW == 0) L.mask[c / S::LPW] = win;
      R.bits |= (m >> sh) << (S::EPL * j);
      cnt[j] = (uint32_t)__builtin_popcount(m);
    }
    packed_row_scan<S::EPL, V>(cnt, ex, tot);
#pragma unroll
    for (int g = 0; g < V / R.PER; ++g) {
      R.ex[g] = 0;
#pragma unroll
      for (int i = 0; i < R.PER; ++i) R.ex[g] |= ex[g * R.PER + i] << (R.F * i);
    }
    if (lane == 63) {
#pragma unroll
      for (int j = 0; j < V; ++j) L.tot[wave * V + j] = tot[j];
    }
  } else {
    uint32_t cnt[V], ex[V], tot[V];
    R.bits = 0;
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const uint32_t c = (uint32_t)((wave * V + j) * 64 + lane);
      const uint32_t b = vec_nz_bits<ESZ>(v[j]);
      R.bits |= b << (S::EPL * j);
      const uint32_t m = group_or<S::LPW>(b << ((lane % S::LPW) * S::EPL));
      if (lane % S::LPW == 0) L.mask[c / S::LPW] = m;
      cnt[j] = (uint32_t)__builtin_popcount(b);
    }
    packed_row_scan<S::EPL, V>(cnt, ex, tot);
#pragma unroll
    for (int g = 0; g < V / R.PER; ++g) {
      R.ex[g] = 0;
#pragma unroll
      for (int i = 0; i < R.PER; ++i) R.ex[g] |= ex[g * R.PER + i] << (R.F * i);
    }
    if (lane == 63) {
#pragma unroll
      for (int j = 0; j < V; ++j) L.tot[wave * V + j] = tot[j];
    }
  }
}

// Write the nonzeros of the tile held in v into stage, in index order, at the
// places R gives (data waves).  32-bit elements are written without a branch:
// in increasing element order every element is stored at its nonzero rank, so
// a zero writes the slot that the lane's next nonzero overwrites right after
// (a wave's LDS writes complete in order); zeros after the row's last nonzero
// go to the lane's dump word instead of the next lane's first slot.  16-bit
// elements keep a branch per element: the branch-free form spilled there.
template <int ESZ>
__device__ __forceinline__ void zvc_c_compact(uint8_t* __restrict__ st, const u32x4 (&v)[ZvcCShape<ESZ>::V],
                                              const ZvcRows<ZvcCShape<ESZ>::EPL, ZvcCShape<ESZ>::V>& R,
                                              uint8_t* __restrict__ dump) {
  using S = ZvcCShape<ESZ>;
#pragma unroll
  for (int j = 0; j < S::V; ++j) {
    uint32_t pos = ESZ * (R.base_of(j) + R.ex_of(j));
    const uint32_t bits = R.bits_of(j);
#pragma unroll
    for (int k = 0; k < S::EPL; ++k) {
      if constexpr (ESZ == 4) {
        uint8_t* a = (bits >> k) ? st + pos : dump;
        store_elem<ESZ>(a, vec_elem<ESZ>(v[j], k));
        pos += ESZ * ((bits >> k) & 1u);
      } else if ((bits >> k) & 1u) {
        store_elem<ESZ>(st + pos, vec_elem<ESZ>(v[j], k));
        pos += ESZ;
      }
    }
  }
}

// Store tile t's window masks from L.mask to the stream with 16-byte stores
// (the control wave; words at or past W are not written).  Issued by the
// control wave so that no data wave has a store in flight, of a number the
// compiler cannot count, ahead of the loads it waits for next (its memory
// operations retire in order).
template <int ESZ>
__device__ __forceinline__ void zvc_c_store_masks(const ZvcCLds<ESZ>& L, uint8_t* __restrict__ dst, uint32_t t,
                                                  uint64_t W, int lane) {
  using S = ZvcCShape<ESZ>;
  static_assert(S::WPT % 4 == 0, "whole mask quads per tile");
  const uint64_t w0 = (uint64_t)t * S::WPT;
  uint32_t* out = reinterpret_cast<uint32_t*>(dst) + w0;
#pragma unroll
  for (int k = 0; k < (S::WPT / 4 + 63) / 64; ++k) {
    const int q = k * 64 + lane;
    if (q < S::WPT / 4) {
      const u32x4 m = *reinterpret_cast<const u32x4*>(&L.mask[4 * q]);
      if (w0 + 4 * q + 4 <= W) {
        *reinterpret_cast<u32x4*>(out + 4 * q) = m;
      } else {
        for (int i = 0; i < 4; ++i)
          if (w0 + 4 * q + i < W) out[4 * q + i] = m[i];
      }
    }
  }
}

// The same for a full tile (every mask word below W), with a fixed number of
// 16-byte buffer stores per lane whatever the tile: lanes past the tile's
// quads, and every lane when !valid, store out of range (dropped).  A fixed
// count lets the compiler wait for loads issued before these stores without
// waiting for the stores.
template <int ESZ>
__device__ __forceinline__ void zvc_c_store_masks_full(const ZvcCLds<ESZ>& L, uint8_t* __restrict__ dst, uint32_t t,
                                                       bool valid, int lane) {
  using S = ZvcCShape<ESZ>;
  constexpr int KQ = (S::WPT / 4 + 63) / 64;  // mask quads per lane
  uint8_t* out = dst + (uint64_t)t * S::WPT * 4;
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(out, (short)0, valid ? S::WPT * 4 : 0, kBufferFlags);
#pragma unroll
  for (int k = 0; k < KQ; ++k) {
    const int q = k * 64 + lane;
    const int qc = q < S::WPT / 4 ? q : 0;
    const u32x4 m = *reinterpret_cast<const u32x4*>(&L.mask[4 * qc]);
    __builtin_amdgcn_raw_buffer_store_b128(m, r, q < S::WPT / 4 ? (uint32_t)(16 * q) : (uint32_t)(S::WPT * 4), 0,
                                           CDMA_NT_STORE ? 2 : 0);
  }
}

// Per-iteration state of the control wave.
struct ZvcCtl {
  ChainRound cr;      // first round of the pending chain sum (issued last iteration)
  uint64_t chain_lo;  // first tile of that sum
  uint64_t P;         // inclusive value prefix of the last tile resolved
  uint32_t pend;      // next tile to hand over (drawn ticket, or static successor)
};

// One iteration (see the description above).  t: tile to classify (its
// loads were issued last iteration into cur); tp1, tp2: the two tiles before
// it (compacted / stored now); tl: tile whose loads go into prev now.  T1, T2:
// nonzeros of tp1, tp2; updated for the next iteration.  Returns the tile the
// data waves load next iteration, with the workgroup synchronised.
template <int ESZ, int OP>
__device__ __forceinline__ uint32_t zvc_c_iteration(
    ZvcCLds<ESZ>& L, u32x4 (&cur)[ZvcCShape<ESZ>::V], u32x4 (&prev)[ZvcCShape<ESZ>::V],
    ZvcRows<ZvcCShape<ESZ>::EPL, ZvcCShape<ESZ>::V>& rc, const ZvcRows<ZvcCShape<ESZ>::EPL, ZvcCShape<ESZ>::V>& rp, ZvcCtl& C, uint32_t& T1, uint32_t& T2,
    uint32_t t, uint32_t tp1, uint32_t tp2, uint32_t tl, int buf, uint32_t full, uint64_t W,
    const uint8_t* __restrict__ src, uint64_t n, uint8_t* __restrict__ dst, uint64_t* __restrict__ out_bytes,
    uint32_t* __restrict__ agg, uint32_t* __restrict__ counter, uint32_t num_tiles, uint8_t* __restrict__ act,
    int tid, int wave, int lane, bool stat) {
  using S = ZvcCShape<ESZ>;
  constexpr int V = S::V;
  // The control wave's stores after its chain loads (see the top of this
  // file): the plain 32-bit compressor only.  The 16-bit kernel has no
  // registers for it, and the fused epilogue (ticket tiles, whose draw comes
  // before the chain loads anyway) measured 2 % slower with it.
  constexpr bool kLateStores = ESZ == 4 && OP == kOpNone;
  const bool have_t = t < num_tiles;
  const bool have_p1 = tp1 < num_tiles;
  const bool have_p2 = tp2 < num_tiles;
  const bool data = wave < kDWaves;

  // ---- phase X ----
  if (data && have_p1) zvc_c_compact<ESZ>(L.stage[buf ^ 1], prev, rp, reinterpret_cast<uint8_t*>(&L.dump[lane]));
  {
    const bool load = __builtin_amdgcn_readfirstlane(wave) < kDWaves && tl < full;
    zvc_c_load_full<ESZ>(prev, src, tl, load, wave, lane);
  }
  if (data) {
    if (have_t) {
      if (t >= full) {  // the one partial tile: load bounded, drain so nothing stays pending on cur
        zvc_c_load_bounded<ESZ>(cur, src, n, t, wave, lane);
        __builtin_amdgcn_s_waitcnt(0);
      }
      if constexpr (OP != kOpNone) zvc_c_epilogue<ESZ, OP>(cur, act, n, t, t < full, wave, lane);
      zvc_c_classify<ESZ>(L, cur, rc, wave, lane);
    }
  } else if (have_p2) {
    bool stuck = false;
    const uint64_t X = C.P + chain_sum<kLateStores>(agg, C.chain_lo, tp2, C.cr, &stuck, [](uint32_t v) { return v; });
    if (lane == 0) {
      L.excl = X;
      if (stuck) atomicMax(reinterpret_cast<unsigned long long*>(out_bytes), kSizeInternalError);
    }
    C.P = X + T2;  // tp2's inclusive prefix
  }
  __syncthreads();

  // ---- phase Y ----
  uint32_t Tn = 0;  // nonzeros of t
  if (data) {
    if (have_t) {
      // segment bases: lane l of every data wave scans the segment totals
      const uint32_t x = lane < S::SEG ? L.tot[lane] : 0u;
      const uint32_t inc = wave_incl_scan(x);
#pragma unroll
      for (int j = 0; j < V; j += 2)
        rc.base[j / 2] = read_lane(inc - x, wave * V + j) | (read_lane(inc - x, wave * V + j + 1) << 16);
      Tn = read_lane(inc, 63);
    }
    if (have_p2) {
      const uint64_t A = 4 * W + (uint64_t)ESZ * L.excl;
      store_staged<ESZ, kDThreads>(L.stage[buf], ESZ * T2, A, dst, tid);
      if (tp2 == num_tiles - 1 && tid == 0)
        atomicMax(reinterpret_cast<unsigned long long*>(out_bytes), A + (uint64_t)ESZ * T2);
    }
  } else {
    // control wave
    if (have_t) Tn = read_lane(wave_incl_scan(lane < S::SEG ? L.tot[lane] : 0u), 63);
    if (stat) {
      if constexpr (!kLateStores) {
        // every other workgroup's chain sums may be waiting for t's aggregate
        if (have_t && lane == 0) agg_publish(agg, t, Tn);
      }
      if (lane == 0) L.next = C.pend;
      if (have_t) C.pend += gridDim.x;
    } else {
      // the ticket drawn last iteration must be back before the hand-over;
      // waiting here on every path keeps the compiler from waiting again
      // after the ticket drawn next
      __builtin_amdgcn_s_waitcnt(0);
      if (lane == 0) L.next = C.pend;
      // the next ticket goes out now and has a whole iteration to come back
      if (have_t && lane == 0) {
        C.pend = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if constexpr (!kLateStores) agg_publish(agg, t, Tn);
      }
    }
    if constexpr (kLateStores) {
      // The chain loads go out before t's aggregate and masks, which are a
      // fixed count of stores, so the chain sum of the next iteration waits
      // only for its loads (memory operations retire in order).  The
      // partial tile's masks go out before the chain loads.
      if (have_t && t >= full) zvc_c_store_masks<ESZ>(L, dst, t, W, lane);
      if (have_p1) {
        // tp1's chain sum: the tiles between this workgroup's tile before it
        // (tp2) and tp1; summed at the start of the next iteration
        C.chain_lo = have_p2 ? (uint64_t)tp2 + 1 : 0;
        chain_issue(agg, C.chain_lo, tp1, C.cr);
      }
      // t's aggregate (lane 0; other workgroups' chain sums may be waiting
      // for it): a buffer store with the agent-scope policy of agg_publish,
      // out of range on the other lanes and when there is no t
      const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(agg, (short)0, num_tiles * 4, kBufferFlags);
      __builtin_amdgcn_raw_buffer_store_b32(Tn + 1, ra, lane == 0 ? 4 * t : 4 * num_tiles, 0, 16 /* sc1 */);
      zvc_c_store_masks_full<ESZ>(L, dst, t, have_t && t < full, lane);
    } else {
      // the order before: aggregate (above) and masks, then the chain loads
      if (have_t) zvc_c_store_masks<ESZ>(L, dst, t, W, lane);
      if (have_p1) {
        C.chain_lo = have_p2 ? (uint64_t)tp2 + 1 : 0;
        chain_issue(agg, C.chain_lo, tp1, C.cr);
      }
    }
  }
  T2 = T1;
  T1 = Tn;
  __syncthreads();
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
  // the first three tickets in increasing order: classify, load, hand over
  const uint32_t a = __builtin_amdgcn_readfirstlane(L.init[0]);
  const uint32_t b = __builtin_amdgcn_readfirstlane(L.init[1]);
  const uint32_t c = __builtin_amdgcn_readfirstlane(L.init[2]);
  const uint32_t lo = min(a, min(b, c)), hi = max(a, max(b, c));
  uint32_t t = lo;                     // classified this iteration
  uint32_t tl = a + b + c - lo - hi;   // loaded this iteration
  uint32_t tp1 = num_tiles, tp2 = num_tiles;  // compacted / stored this iteration (none yet)
  ZvcCtl C;                            // control wave
  C.chain_lo = 0;
  C.P = 0;
  C.pend = hi;
  uint32_t T1 = 0, T2 = 0;
  u32x4 ra[S::V], rb[S::V];
  ZvcRows<S::EPL, S::V> qa, qb;
  zvc_c_load_full<ESZ>(ra, src, t, __builtin_amdgcn_readfirstlane(wave) < kDWaves && t < full, wave, lane);
  // Two iterations per trip so the register sets swap roles without copies.
  // One exit, after the second iteration of a trip: an iteration with no tile
  // to classify, compact or store only passes its barriers, and a single path
  // back to the loop head keeps the compiler's count of loads in flight exact.
  for (;;) {
    uint32_t r = zvc_c_iteration<ESZ, OP>(L, ra, rb, qa, qb, C, T1, T2, t, tp1, tp2, tl, 0, full, W, src, n, dst,
                                          out_bytes, agg, counter, num_tiles, act, tid, wave, lane, stat);
    tp2 = tp1;
    tp1 = t;
    t = tl;
    tl = r;
    r = zvc_c_iteration<ESZ, OP>(L, rb, ra, qb, qa, C, T1, T2, t, tp1, tp2, tl, 1, full, W, src, n, dst, out_bytes,
                                 agg, counter, num_tiles, act, tid, wave, lane, stat);
    tp2 = tp1;
    tp1 = t;
    t = tl;
    tl = r;
    if (t >= num_tiles && tp1 >= num_tiles && tp2 >= num_tiles) break;
  }
}

// ---------------------------------------------------------------------------
// single pass: maps of at most one tile per resident workgroup
// ---------------------------------------------------------------------------
//
// Such a map would give every workgroup of the persistent grid at most one
// tile, which the pipeline above takes through three iterations (load;
// classify and compact; chain sum and store) before storing it.  Here each
// workgroup draws one tile and runs the same steps back to back: load,
// classify, publish the tile's aggregate and store its masks (their place
// depends only on the tile), compact the values, sum the aggregates of all
// tiles before it, store the values.  A workgroup only waits for tiles drawn
// before its own, by workgroups that have started and publish without
// waiting, so every wait ends (the chain sum's spin bound still applies).
template <int ESZ>
__global__ __launch_bounds__(kCBlock) void zvc_compress_single_kernel(
    const uint8_t* __restrict__ src, uint64_t n, uint8_t* __restrict__ dst, uint64_t* __restrict__ out_bytes,
    uint32_t* __restrict__ counter, uint32_t* __restrict__ agg, uint32_t num_tiles) {
  using S = ZvcCShape<ESZ>;
  constexpr int V = S::V;
  __shared__ ZvcCLds<ESZ> L;
  const int tid = threadIdx.x;
  const int lane = (int)lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool data = wave < kDWaves;
  const uint64_t W = (n + 31) / 32;
  const uint32_t full = (uint32_t)(n / S::TE);  // tiles with no element past n
  if (tid == 0) L.next = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  // One workgroup per tile, so every ticket names a tile below num_tiles when
  // the counter starts cleared.  A call that overlaps another on the same
  // workspace breaks that: report it instead of reading past the input.
  const uint32_t t = __builtin_amdgcn_readfirstlane(L.next);
  if (t >= num_tiles) {
    if (tid == 0) atomicMax(reinterpret_cast<unsigned long long*>(out_bytes), kSizeInternalError);
    return;
  }
  ZvcRows<S::EPL, V> R;
  u32x4 v[V];
  if (data) {
    if (t < full) zvc_c_load_full<ESZ>(v, src, t, true, wave, lane);
    else zvc_c_load_bounded<ESZ>(v, src, n, t, wave, lane);
    zvc_c_classify<ESZ>(L, v, R, wave, lane);
  }
  __syncthreads();
  // segment bases and the tile's nonzeros (every wave scans the segment totals)
  const uint32_t x = lane < S::SEG ? L.tot[lane] : 0u;
  const uint32_t inc = wave_incl_scan(x);
  const uint32_t Tn = read_lane(inc, 63);
  if (data) {
#pragma unroll
    for (int j = 0; j < V; j += 2)
      R.base[j / 2] = read_lane(inc - x, wave * V + j) | (read_lane(inc - x, wave * V + j + 1) << 16);
    zvc_c_compact<ESZ>(L.stage[0], v, R, reinterpret_cast<uint8_t*>(&L.dump[lane]));
  } else {
    if (lane == 0) agg_publish(agg, t, Tn);
    zvc_c_store_masks<ESZ>(L, dst, t, W, lane);
    ChainRound cr;
    chain_issue(agg, 0, t, cr);
    bool stuck = false;
    const uint64_t X = chain_sum(agg, 0, t, cr, &stuck, [](uint32_t a) { return a; });
    if (lane == 0) {
      L.excl = X;
      if (stuck) atomicMax(reinterpret_cast<unsigned long long*>(out_bytes), kSizeInternalError);
    }
  }
  __syncthreads();
  if (data) {
    const uint64_t A = 4 * W + (uint64_t)ESZ * L.excl;
    store_staged<ESZ, kDThreads>(L.stage[0], ESZ * Tn, A, dst, tid);
    if (t == num_tiles - 1 && tid == 0)
      atomicMax(reinterpret_cast<unsigned long long*>(out_bytes), A + (uint64_t)ESZ * Tn);
  }
}

}  // namespace cdma
