// zvc_kernels.hpp -- zero-value compression and decompression for gfx950.
//
// Format ("Compressing DMA Engine: Leveraging Activation Sparsity for Training
// Deep Neural Networks", §V.A Compression Algorithm): per window of 32
// consecutive elements a 32-bit mask (bit i = element i is nonzero), then the
// nonzero elements.  All W = ceil(n/32) masks come first, then all values in
// index order, so every mask sits at a fixed offset and a single prefix sum
// over nonzero counts places every value.
//
// One workgroup handles one tile of TE elements (V 16-byte vectors per lane,
// 256 lanes).  Vector j of wave w covers bytes [(w*V + j) * 1024, +1024) of the
// tile, so every global load and store instruction moves 1 KB of contiguous
// memory per wavefront.  A 32-element window spans LPW = 32/EPL lanes (8 for
// fp32, 4 for fp16), so its mask is an OR across a DPP lane group.
//
// compress:   load -> per-lane nonzero bits -> window masks (DPP OR) and
//             per-lane counts (DPP wave scan) -> LDS pass over the 4*V wave
//             segments -> masks stored -> decoupled lookback gives the tile's
//             value offset -> nonzeros compacted into LDS at their final byte
//             alignment -> aligned 16-byte stores (element stores only for the
//             two partial 16-byte quads at the ends of the tile's span).
// decompress: masks -> counts -> same scan and lookback -> the tile's value
//             span is read into LDS with aligned 16-byte loads -> each lane
//             expands its vector from LDS -> aligned 16-byte stores.
#pragma once

#include "device_common.hpp"

namespace cdma {

template <int ESZ, int V>
struct ZvcShape {
  static constexpr int EPL = 16 / ESZ;              // elements per 16-byte vector
  static constexpr int TE = kBlock * V * EPL;       // elements per tile
  static constexpr int LPW = 32 / EPL;              // lanes per 32-element window
  static constexpr int WPT = TE / 32;               // windows per tile
  static constexpr int SEG = kWaves * V;            // wave segments per tile
  static constexpr int STAGE = TE * ESZ + 32;       // LDS staging bytes
};

// Per-element nonzero bits of one 16-byte vector (bit k = element k).
template <int ESZ>
__device__ __forceinline__ uint32_t vec_nz_bits(u32x4 v) {
  if constexpr (ESZ == 4) {
    return (uint32_t)(v.x != 0) | ((uint32_t)(v.y != 0) << 1) | ((uint32_t)(v.z != 0) << 2) |
           ((uint32_t)(v.w != 0) << 3);
  } else {
    uint32_t r = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t w = v[k];
      r |= ((uint32_t)((w & 0xFFFFu) != 0) << (2 * k)) | ((uint32_t)((w >> 16) != 0) << (2 * k + 1));
    }
    return r;
  }
}

template <int ESZ>
__device__ __forceinline__ uint32_t vec_elem(u32x4 v, int k) {
  if constexpr (ESZ == 4) return v[k];
  else return (v[k >> 1] >> ((k & 1) * 16)) & 0xFFFFu;
}

template <int ESZ>
__device__ __forceinline__ void vec_set(u32x4& v, int k, uint32_t e) {
  if constexpr (ESZ == 4) v[k] = e;
  else v[k >> 1] |= e << ((k & 1) * 16);
}

template <int ESZ>
__device__ __forceinline__ uint32_t load_elem(const uint8_t* p) {
  if constexpr (ESZ == 4) return *reinterpret_cast<const uint32_t*>(p);
  else return *reinterpret_cast<const uint16_t*>(p);
}

template <int ESZ>
__device__ __forceinline__ void store_elem(uint8_t* p, uint32_t e) {
  if constexpr (ESZ == 4) *reinterpret_cast<uint32_t*>(p) = e;
  else *reinterpret_cast<uint16_t*>(p) = (uint16_t)e;
}

// Load the 16-byte vector of elements [e0, e0 + EPL); elements >= n read as 0.
template <int ESZ>
__device__ __forceinline__ u32x4 load_vec(const uint8_t* __restrict__ src, uint64_t e0, uint64_t n) {
  constexpr int EPL = 16 / ESZ;
  if (e0 + EPL <= n) return ld_stream(reinterpret_cast<const u32x4*>(src + e0 * ESZ));
  u32x4 v = {0u, 0u, 0u, 0u};
  for (int k = 0; k < EPL; ++k)
    if (e0 + k < n) vec_set<ESZ>(v, k, load_elem<ESZ>(src + (e0 + k) * ESZ));
  return v;
}

// Store the vector of elements [e0, e0 + EPL); elements >= n are not stored.
template <int ESZ>
__device__ __forceinline__ void store_vec(uint8_t* __restrict__ dst, uint64_t e0, uint64_t n, u32x4 v) {
  constexpr int EPL = 16 / ESZ;
  if (e0 + EPL <= n) {
    st_stream(reinterpret_cast<u32x4*>(dst + e0 * ESZ), v);
    return;
  }
  for (int k = 0; k < EPL; ++k)
    if (e0 + k < n) store_elem<ESZ>(dst + (e0 + k) * ESZ, vec_elem<ESZ>(v, k));
}

// Tile-local bases of this wave's V segments and the tile total, from the
// per-segment totals in LDS (segment order = element order).
template <int V>
__device__ __forceinline__ uint32_t segment_bases(const uint32_t* s_tot, int wave, uint32_t (&base)[V]) {
  uint32_t acc = 0, total = 0;
  for (int k = 0; k < wave * V; ++k) acc += s_tot[k];
#pragma unroll
  for (int j = 0; j < V; ++j) {
    base[j] = acc;
    acc += s_tot[wave * V + j];
  }
  for (int k = 0; k < kWaves * V; ++k) total += s_tot[k];
  return total;
}

// ---------------------------------------------------------------------------
// compress: persistent workgroups of data wavefronts plus one control wavefront
// ---------------------------------------------------------------------------
//
// A persistent grid of (about) one workgroup per CU takes tiles from a ticket
// counter.  Waves 0..kDWaves-1 move data; the last wave, the control wave,
// draws tickets and computes tile offsets by chaining over published
// aggregates (see chain_sum).  Vector-memory counters
// retire in order on this GPU, so a wave that had both prefetched a tile and
// issued status reads could not use the tile before the status reads came
// back; with the status traffic in a wave of its own, the data waves wait only
// for their own loads.  Iteration i of a workgroup holds tile t (loaded), tn
// (to prefetch) and the previous tile tp (nonzeros staged in LDS):
//   data waves:   classify t (window masks, nonzero counts) -> B1 -> store
//                 t's masks, compact t's nonzeros into LDS buffer i%2, issue
//                 tn's loads -> B2 -> store tp's staged values at the offset
//                 the control wave resolved;
//   control wave: B1 -> hand the data waves the ticket drawn one iteration
//                 earlier -> publish t's aggregate -> finish tp's chain sum
//                 (aggregates of the tiles between this workgroup's previous
//                 tile and tp, read one iteration earlier) -> B2 -> issue the
//                 first round of t's chain sum and draw a ticket.
// The size is reported with 64-bit atomic max operations on a word cleared
// before the launch: the last tile writes the stream size and a control wave
// whose chain sum hit the spin bound writes the all-ones error value, which
// wins whatever the order.  (Such a sum returns an under-estimate, so every
// store still lands inside the stream's bounds.)
// Progress: a ticket is drawn only by a running workgroup, which classifies
// its tickets in increasing order, and a tile's aggregate is published in the
// iteration that classifies it, before that iteration waits for anything.
// The smallest ticket whose aggregate is unpublished is therefore held by a
// running workgroup that waits only for aggregates of smaller tickets, all
// published: no co-residency is assumed and every chain sum ends.

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

// Store `bytes` staged bytes (staged from offset 0) to stream bytes
// [A, A + bytes) with NT threads: aligned 16-byte stores, the staged bytes
// shifted into place on the way.  A and bytes are multiples of G (2 or 4);
// the two partial quads at the ends are written G bytes at a time.  Reads up
// to 4 bytes past the staged span, which the stage buffer must hold.
template <int G, int NT>
__device__ __forceinline__ void store_staged(const uint8_t* __restrict__ st, uint32_t bytes, uint64_t A,
                                             uint8_t* __restrict__ dst, int tid) {
  static_assert(G == 2 || G == 4, "store granularity");
  const uint64_t end = A + bytes;
  const uint64_t q0 = A >> 4, q1 = (end + 15) >> 4;
  const uint32_t d = (uint32_t)(A & 15);
  const uint32_t* sw = reinterpret_cast<const uint32_t*>(st);
  for (uint64_t q = q0 + tid; q < q1; q += NT) {
    const uint64_t qb = q << 4;
    if (qb >= A && qb + 16 <= end) {
      const uint32_t o = (uint32_t)(qb - A);  // staged byte of the quad's first byte
      u32x4 out;
      if (d == 0) {
        out = *reinterpret_cast<const u32x4*>(st + o);
      } else if (G == 4 || (d & 3) == 0) {
        const uint32_t i = o >> 2;
        out = u32x4{sw[i], sw[i + 1], sw[i + 2], sw[i + 3]};
      } else {  // 2 bytes off a word boundary
        const uint32_t i = o >> 2;
        const uint32_t w0 = sw[i], w1 = sw[i + 1], w2 = sw[i + 2], w3 = sw[i + 3], w4 = sw[i + 4];
        out = u32x4{__builtin_amdgcn_alignbyte(w1, w0, 2), __builtin_amdgcn_alignbyte(w2, w1, 2),
                    __builtin_amdgcn_alignbyte(w3, w2, 2), __builtin_amdgcn_alignbyte(w4, w3, 2)};
      }
      st_stream(reinterpret_cast<u32x4*>(dst + qb), out);
    } else {
      for (int k = 0; k < 16; k += G) {
        const uint64_t b = qb + k;
        if (b >= A && b < end) store_elem<G>(dst + b, load_elem<G>(st + (b - A)));
      }
    }
  }
}

// One pipeline iteration (see above).  Returns the ticket the data waves
// prefetch in the next iteration, with the workgroup synchronised.
template <int ESZ>
__device__ __forceinline__ uint32_t zvc_c_iteration(ZvcCLds<ESZ>& L, u32x4 (&cur)[ZvcCShape<ESZ>::V],
                                                    u32x4 (&nxt)[ZvcCShape<ESZ>::V], ChainRound& cr,
                                                    uint64_t& chain_lo, uint64_t& P, uint32_t& pend, uint32_t t,
                                                    uint32_t tn, uint32_t tp, int buf,
                                                    uint32_t full, uint64_t W, const uint8_t* __restrict__ src,
                                                    uint64_t n, uint8_t* __restrict__ dst,
                                                    uint64_t* __restrict__ out_bytes, uint32_t* __restrict__ agg,
                                                    uint32_t* __restrict__ counter, uint32_t num_tiles, int tid,
                                                    int wave, int lane) {
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
    // control wave.  The ticket drawn last iteration goes out first: waiting
    // for it also covers the status reads issued before it, which the resolve
    // below needs anyway.
    if (lane == 0) L.next = pend;
    if (have_cur) {
      const uint32_t x = lane < S::SEG ? L.tot[lane] : 0u;
      const uint32_t T = read_lane(wave_incl_scan(x), 63);
      if (lane == 0) {
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
    if (lane == 0) pend = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  return __builtin_amdgcn_readfirstlane(L.next);  // uniform: keeps tile bases in SGPRs
}

template <int ESZ>
__global__ __launch_bounds__(kCBlock) void zvc_compress_kernel(
    const uint8_t* __restrict__ src, uint64_t n, uint8_t* __restrict__ dst,
    uint64_t* __restrict__ out_bytes, uint32_t* __restrict__ counter, uint32_t* __restrict__ agg,
    uint32_t num_tiles) {
  using S = ZvcCShape<ESZ>;
  __shared__ ZvcCLds<ESZ> L;
  const int tid = threadIdx.x;
  const int lane = (int)lane_id();
  const int wave = tid >> 6;
  const uint64_t W = (n + 31) / 32;
  const uint32_t full = (uint32_t)(n / S::TE);  // tiles with no element past n
  if (tid < 3 * 64 && lane == 0)
    L.init[wave] = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
    uint32_t tnn = zvc_c_iteration<ESZ>(L, ra, rb, cr, chain_lo, P, pend, t, tn, tp, 0, full, W, src, n, dst,
                                        out_bytes, agg, counter, num_tiles, tid, wave, lane);
    if (t >= num_tiles) break;
    tp = t;
    t = tn;
    tn = tnn;
    tnn = zvc_c_iteration<ESZ>(L, rb, ra, cr, chain_lo, P, pend, t, tn, tp, 1, full, W, src, n, dst, out_bytes,
                               agg, counter, num_tiles, tid, wave, lane);
    if (t >= num_tiles) break;
    tp = t;
    t = tn;
    tn = tnn;
  }
}

// ---------------------------------------------------------------------------
// decompress, passes 1 and 2: value offset of every tile from the masks alone
// ---------------------------------------------------------------------------
//
// Pass 1 (zvc_count_kernel): a super tile is SUPER consecutive ZVC tiles
// (32 KB of masks).  Each workgroup popcounts its masks and writes, for every
// tile, the number of nonzeros before it inside the super tile (local[t]),
// and the super tile's total (sup[u]).  Mask bytes at or past the readable
// size count as 0; mask bits for indices >= n are not counted but reported.
// Pass 2 (zvc_scan_kernel): one workgroup turns sup[] into exclusive prefixes
// in place, with the grand total in sup[num_super].  The value offset of tile
// t is then sup[t / SUPER] + local[t].  Neither pass waits on another
// workgroup.

template <int ESZ, int V>
struct ZvcScanShape {
  using S = ZvcShape<ESZ, V>;
  static constexpr int WORDS = 8192;                 // mask words per super tile
  static constexpr int SUPER = WORDS / S::WPT;       // ZVC tiles per super tile
  static constexpr int WPTH = WORDS / kBlock;        // mask words per thread (32)
  static constexpr int TPT = S::WPT / WPTH;          // threads per ZVC tile
  static_assert(SUPER <= 64 && TPT >= 1 && S::WPT % WPTH == 0, "super tile shape");
};

template <int ESZ, int V>
__global__ __launch_bounds__(kBlock) void zvc_count_kernel(
    const uint8_t* __restrict__ src, uint64_t src_capacity, const uint64_t* __restrict__ src_bytes,
    uint64_t n, uint32_t* __restrict__ local, uint32_t* __restrict__ sup, uint32_t* __restrict__ error,
    uint32_t num_tiles) {
  using C = ZvcScanShape<ESZ, V>;
  __shared__ uint32_t s_cnt[C::SUPER];
  const int tid = threadIdx.x;
  const int lane = (int)lane_id();
  const int wave = tid >> 6;
  const uint32_t u = blockIdx.x;
  for (int i = tid; i < C::SUPER; i += kBlock) s_cnt[i] = 0;
  const uint64_t W = (n + 31) / 32;
  const uint64_t claimed = src_bytes ? *src_bytes : src_capacity;
  const uint64_t eff = claimed < src_capacity ? claimed : src_capacity;
  const uint64_t g0 = (uint64_t)u * C::WORDS + (uint64_t)tid * C::WPTH;  // first mask word of this thread
  u32x4 m[C::WPTH / 4];
#pragma unroll
  for (int k = 0; k < C::WPTH / 4; ++k) {
    const uint64_t g = g0 + 4 * k;
    if (g + 4 <= W && 4 * (g + 4) <= eff) {
      m[k] = ld_stream(reinterpret_cast<const u32x4*>(src + 4 * g));
    } else {
      m[k] = u32x4{0u, 0u, 0u, 0u};
      for (int i = 0; i < 4; ++i) {
        if (g + i >= W) break;
        uint32_t w = 0;
        for (int b = 0; b < 4; ++b)
          if (4 * (g + i) + b < eff) w |= (uint32_t)src[4 * (g + i) + b] << (8 * b);
        m[k][i] = w;
      }
    }
  }
  __syncthreads();
  uint32_t cnt = 0, err = 0;
#pragma unroll
  for (int k = 0; k < C::WPTH / 4; ++k) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t w = m[k][i];
      if (g0 + 4 * k + i == W - 1 && (n & 31)) {
        const uint32_t valid = (1u << (n & 31)) - 1;
        if (w & ~valid) err |= CDMA_E_MASK_PAST_N;
        w &= valid;
      }
      cnt += (uint32_t)__builtin_popcount(w);
    }
  }
  if (cnt) atomicAdd(&s_cnt[tid / C::TPT], cnt);
  __syncthreads();
  if (wave == 0) {
    const uint32_t c = lane < C::SUPER ? s_cnt[lane] : 0u;
    const uint32_t inc = wave_incl_scan(c);
    const uint64_t t = (uint64_t)u * C::SUPER + lane;
    if (lane < C::SUPER && t < num_tiles) local[t] = inc - c;
    if (lane == 63) sup[u] = inc;
  }
  if (err && error) atomicOr(error, err);
}

// Exclusive prefix sums of sup[0..count) in place, total in sup[count]; one
// workgroup of kScanBlock threads.
constexpr int kScanBlock = 1024;

__global__ __launch_bounds__(kScanBlock) void zvc_scan_kernel(uint32_t* __restrict__ sup, uint32_t count) {
  __shared__ uint32_t s_wave[kScanBlock / 64];
  __shared__ uint32_t s_carry;
  const int tid = threadIdx.x;
  const int lane = (int)lane_id();
  const int wave = tid >> 6;
  if (tid == 0) s_carry = 0;
  __syncthreads();
  for (uint32_t base = 0; base < count; base += kScanBlock) {
    const uint32_t i = base + tid;
    const uint32_t v = i < count ? sup[i] : 0u;
    const uint32_t inc = wave_incl_scan(v);
    if (lane == 63) s_wave[wave] = inc;
    __syncthreads();
    uint32_t before = s_carry, all = 0;
    for (int w = 0; w < kScanBlock / 64; ++w) {
      if (w < wave) before += s_wave[w];
      all += s_wave[w];
    }
    if (i < count) sup[i] = before + inc - v;
    __syncthreads();
    if (tid == 0) s_carry += all;
    __syncthreads();
  }
  if (tid == 0) sup[count] = s_carry;
}

// ---------------------------------------------------------------------------
// decompress, pass 2: expand, persistent grid-stride with prefetch
// ---------------------------------------------------------------------------
//
// With the offsets known, tiles are independent.  Each workgroup walks tiles
// t, t+G, t+2G, ...; while it expands tile a from LDS it already has the
// masks and value quads of tile b = a+G in flight in registers, and the
// offsets of tile b+G on their way.

template <int ESZ, int V>
struct ZvcExpandShape {
  using S = ZvcShape<ESZ, V>;
  static constexpr int QPT = (S::TE * ESZ / 16 + 2 + kBlock - 1) / kBlock;  // value quads per thread
  static constexpr int MPT = (S::WPT + kBlock - 1) / kBlock;                // mask words per thread
};

template <int ESZ, int V>
struct ZvcTileIn {
  using X = ZvcExpandShape<ESZ, V>;
  u32x4 q[X::QPT];
  uint32_t m[X::MPT];
  uint64_t beg, end;  // value span in the stream
  bool short_read;
};

template <int ESZ, int V>
__device__ __forceinline__ void zvc_fetch_tile(ZvcTileIn<ESZ, V>& in, const uint8_t* __restrict__ src, uint64_t eff,
                                               uint64_t W, uint32_t t, uint32_t o0, uint32_t o1, int tid) {
  using S = ZvcShape<ESZ, V>;
  using X = ZvcExpandShape<ESZ, V>;
#pragma unroll
  for (int k = 0; k < X::MPT; ++k) {
    const int i = tid + k * kBlock;
    const uint64_t g = (uint64_t)t * S::WPT + i;
    uint32_t w = 0;
    if (i < S::WPT && g < W) {
      if (4 * g + 4 <= eff) {
        w = reinterpret_cast<const uint32_t*>(src)[g];
      } else {
        for (int b = 0; b < 4; ++b)
          if (4 * g + b < eff) w |= (uint32_t)src[4 * g + b] << (8 * b);
      }
    }
    in.m[k] = w;
  }
  in.beg = 4 * W + (uint64_t)ESZ * o0;
  in.end = 4 * W + (uint64_t)ESZ * (o1 > o0 ? o1 : o0);
  in.short_read = false;
  const uint64_t q0 = in.beg >> 4, q1 = (in.end + 15) >> 4;
#pragma unroll
  for (int k = 0; k < X::QPT; ++k) {
    const uint64_t q = q0 + tid + (uint64_t)k * kBlock;
    u32x4 d = {0u, 0u, 0u, 0u};
    if (q < q1) {
      const uint64_t qb = q << 4;
      if (qb + 16 <= eff) {
        d = ld_stream(reinterpret_cast<const u32x4*>(src + qb));
      } else {
        for (int b = 0; b < 16; b += ESZ) {
          if (qb + b + ESZ <= eff) vec_set<ESZ>(d, b / ESZ, load_elem<ESZ>(src + qb + b));
          else if (qb + b >= in.beg && qb + b < in.end) in.short_read = true;
        }
      }
    }
    in.q[k] = d;
  }
}

template <int ESZ, int V>
struct ZvcExpandLds {
  using S = ZvcShape<ESZ, V>;
  uint32_t tot[S::SEG];
  uint32_t mask[S::WPT];
  __attribute__((aligned(16))) uint8_t stage[S::STAGE];
};

template <int ESZ, int V>
__device__ __forceinline__ uint32_t zvc_expand_tile(ZvcExpandLds<ESZ, V>& L, const ZvcTileIn<ESZ, V>& in, uint32_t t,
                                                    uint64_t n, uint8_t* __restrict__ dst, int tid, int wave,
                                                    int lane) {
  using S = ZvcShape<ESZ, V>;
  using X = ZvcExpandShape<ESZ, V>;
  const uint64_t W = (n + 31) / 32;
  const uint64_t q0 = in.beg >> 4, q1 = (in.end + 15) >> 4;
#pragma unroll
  for (int k = 0; k < X::MPT; ++k) {
    const int i = tid + k * kBlock;
    if (i < S::WPT) {
      uint32_t w = in.m[k];
      const uint64_t g = (uint64_t)t * S::WPT + i;
      if (g == W - 1 && (n & 31)) w &= (1u << (n & 31)) - 1;
      L.mask[i] = w;
    }
  }
#pragma unroll
  for (int k = 0; k < X::QPT; ++k) {
    const uint64_t q = q0 + tid + (uint64_t)k * kBlock;
    if (q < q1 && 16 * (q - q0) + 16 <= (uint64_t)S::STAGE) *reinterpret_cast<u32x4*>(L.stage + 16 * (q - q0)) = in.q[k];
  }
  __syncthreads();
  uint32_t bits[V], ex[V];
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const uint32_t c = (uint32_t)((wave * V + j) * 64 + lane);
    bits[j] = (L.mask[c / S::LPW] >> ((c % S::LPW) * S::EPL)) & ((1u << S::EPL) - 1);
    const uint32_t cnt = (uint32_t)__builtin_popcount(bits[j]);
    const uint32_t inc = wave_incl_scan(cnt);
    ex[j] = inc - cnt;
    if (lane == 63) L.tot[wave * V + j] = inc;
  }
  __syncthreads();
  uint32_t base[V];
  const uint32_t total = segment_bases<V>(L.tot, wave, base);
  // values the offsets give this tile (never more than a tile holds)
  const uint64_t span = (in.end - in.beg) / ESZ;
  const uint32_t avail = span < (uint64_t)S::TE ? (uint32_t)span : (uint32_t)S::TE;
  const uint32_t shift = (uint32_t)(in.beg & 15);
  const uint64_t e_tile = (uint64_t)t * S::TE;
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const uint32_t c = (uint32_t)((wave * V + j) * 64 + lane);
    uint32_t r = base[j] + ex[j];
    u32x4 o = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < S::EPL; ++k) {
      if ((bits[j] >> k) & 1u) {
        if (r < avail) vec_set<ESZ>(o, k, load_elem<ESZ>(L.stage + shift + ESZ * r));
        ++r;
      }
    }
    store_vec<ESZ>(dst, e_tile + (uint64_t)c * S::EPL, n, o);
  }
  __syncthreads();
  return total;
}

// Value offset of tile t (t <= num_tiles) from the two count passes.
template <int ESZ, int V>
__device__ __forceinline__ uint32_t zvc_tile_offset(const uint32_t* __restrict__ local,
                                                    const uint32_t* __restrict__ sup, uint32_t t,
                                                    uint32_t num_tiles) {
  using C = ZvcScanShape<ESZ, V>;
  if (t >= num_tiles) return sup[(num_tiles + C::SUPER - 1) / C::SUPER];  // the grand total
  return sup[t / C::SUPER] + local[t];
}

template <int ESZ, int V>
__global__ __launch_bounds__(kBlock) void zvc_expand_kernel(
    const uint8_t* __restrict__ src, uint64_t src_capacity, const uint64_t* __restrict__ src_bytes,
    uint64_t n, uint8_t* __restrict__ dst, uint32_t* __restrict__ error,
    const uint32_t* __restrict__ local, const uint32_t* __restrict__ sup, uint32_t num_tiles) {
  __shared__ ZvcExpandLds<ESZ, V> L;
  const int tid = threadIdx.x;
  const int lane = (int)lane_id();
  const int wave = tid >> 6;
  const uint32_t G = gridDim.x;
  const uint64_t W = (n + 31) / 32;
  const uint64_t claimed = src_bytes ? *src_bytes : src_capacity;
  const uint64_t eff = claimed < src_capacity ? claimed : src_capacity;
  uint32_t err = 0;
  uint32_t ta = blockIdx.x;
  if (ta >= num_tiles) return;
  ZvcTileIn<ESZ, V> A, B;
  zvc_fetch_tile<ESZ, V>(A, src, eff, W, ta, zvc_tile_offset<ESZ, V>(local, sup, ta, num_tiles),
                         zvc_tile_offset<ESZ, V>(local, sup, ta + 1, num_tiles), tid);
  uint32_t tb = ta + G;
  uint32_t ob0 = 0, ob1 = 0;
  if (tb < num_tiles) {
    ob0 = zvc_tile_offset<ESZ, V>(local, sup, tb, num_tiles);
    ob1 = zvc_tile_offset<ESZ, V>(local, sup, tb + 1, num_tiles);
  }
  for (;;) {
    // A holds tile ta; fetch tile tb into B; offsets of the tile after tb
    uint32_t tc = tb + G, oc0 = 0, oc1 = 0;
    if (tb < num_tiles) zvc_fetch_tile<ESZ, V>(B, src, eff, W, tb, ob0, ob1, tid);
    if (tc < num_tiles) {
      oc0 = zvc_tile_offset<ESZ, V>(local, sup, tc, num_tiles);
      oc1 = zvc_tile_offset<ESZ, V>(local, sup, tc + 1, num_tiles);
    }
    if (A.short_read) err |= CDMA_E_SIZE;
    zvc_expand_tile<ESZ, V>(L, A, ta, n, dst, tid, wave, lane);
    if (ta == num_tiles - 1 && tid == 0 && src_bytes && A.end != *src_bytes) err |= CDMA_E_SIZE;
    if (tb >= num_tiles) break;
    ta = tb;
    tb = tc;
    ob0 = oc0;
    ob1 = oc1;
    // same step with the roles of A and B swapped
    tc = tb + G;
    if (tb < num_tiles) zvc_fetch_tile<ESZ, V>(A, src, eff, W, tb, ob0, ob1, tid);
    if (tc < num_tiles) {
      oc0 = zvc_tile_offset<ESZ, V>(local, sup, tc, num_tiles);
      oc1 = zvc_tile_offset<ESZ, V>(local, sup, tc + 1, num_tiles);
    }
    if (B.short_read) err |= CDMA_E_SIZE;
    zvc_expand_tile<ESZ, V>(L, B, ta, n, dst, tid, wave, lane);
    if (ta == num_tiles - 1 && tid == 0 && src_bytes && B.end != *src_bytes) err |= CDMA_E_SIZE;
    if (tb >= num_tiles) break;
    ta = tb;
    tb = tc;
    ob0 = oc0;
    ob1 = oc1;
  }
  if (err && error) atomicOr(error, err);
}

}  // namespace cdma
