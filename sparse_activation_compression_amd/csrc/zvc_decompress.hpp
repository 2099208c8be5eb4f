// zvc_decompress.hpp -- ZVC decompression for gfx950 (stream format in
// zvc_common.hpp): per-tile value offsets from the masks alone (a count pass
// and a one-workgroup scan), then an expand pass, one workgroup per 16 KB
// tile, in which the tile's value span is read into LDS with aligned 16-byte
// loads and each lane expands its vector from LDS -> aligned 16-byte stores.
#pragma once

#include "zvc_common.hpp"

namespace cdma {

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
// workgroup.  The masks are read twice, here and in the expand pass; both
// reads leave out the non-temporal hint, so the second one is served by the
// memory-side cache while the masks fit in it (128 MB for 2^30 elements) and
// the expand pass's HBM traffic is then its values and its output alone.
// When the whole stream fits (CDMA_WARM_BYTES), pass 1 reads the values too,
// and the expand pass's HBM traffic is its output alone; a larger stream that
// is a small share of the output is read ahead chunk by chunk inside the
// expand pass (zvc_expand_kernel).

// Super tile of decode tiles with TWPT mask words each: KQ quads of mask
// words per thread, i.e. KQ * kBlock * 4 words (32 KB for KQ = 8: 64 fp32 or
// 32 fp16 tiles; 4 KB for KQ = 1: 8 fp32 or 4 fp16 tiles), at most 64 tiles.
// Small outputs take the small super tile, so the count pass has enough
// workgroups to fill the GPU (a 148 MB map has 4.6 MB of masks: 142
// workgroups of 32 KB); large ones the big one, so the one-workgroup scan
// stays short.  SHIFT = log2(SUPER) is how the other passes find a tile's
// super tile.
template <int TWPT, int KQ>
struct ZvcScanShape {
  static constexpr int WPT = TWPT;                // mask words per decode tile
  static constexpr int WORDS = KQ * kBlock * 4;   // mask words per super tile
  static constexpr int SUPER = WORDS / WPT;       // decode tiles per super tile
  static constexpr int SHIFT = __builtin_ctz(SUPER);
  static_assert(SUPER <= 64 && WORDS % WPT == 0 && (SUPER & (SUPER - 1)) == 0, "super tile shape");
};

template <int TWPT, int KQ_>
__global__ __launch_bounds__(kBlock) void zvc_count_kernel(
    const uint8_t* __restrict__ src, uint64_t src_capacity, const uint64_t* __restrict__ src_bytes,
    uint64_t n, uint32_t* __restrict__ local, uint32_t* __restrict__ sup, uint32_t* __restrict__ error,
    uint32_t num_tiles, bool warm) {
  using C = ZvcScanShape<TWPT, KQ_>;
  static_assert(512 % TWPT == 0, "a decode tile is 16 KB: 32 * TWPT elements of 512 / TWPT bytes");
  // Mask quad i of the super tile (16 bytes) is read by thread i % kBlock in
  // step i / kBlock, so each load instruction covers 1 KB of contiguous masks.
  // A decode tile's quads are then an aligned group of QT lanes of one step.
  constexpr int QT = C::WPT / 4;               // mask quads per decode tile
  constexpr int KQ = KQ_;                       // steps (quads per thread)
  static_assert(QT == 8 || QT == 16 || QT == 32 || QT == 64, "a decode tile's masks are a lane group of quads");
  static_assert(KQ * kBlock * 4 == C::WORDS, "super tile shape");
  __shared__ uint32_t s_cnt[C::SUPER];
  const int tid = threadIdx.x;
  const int lane = (int)lane_id();
  const int wave = tid >> 6;
  const uint32_t u = blockIdx.x;
  const uint64_t W = (n + 31) / 32;
  const uint64_t claimed = src_bytes ? *src_bytes : src_capacity;
  const uint64_t eff = claimed < src_capacity ? claimed : src_capacity;
  const uint64_t w0 = (uint64_t)u * C::WORDS;  // first mask word of the super tile
  u32x4 m[KQ];
  if (w0 + C::WORDS <= W && 4 * (w0 + C::WORDS) <= eff) {
#pragma unroll
    for (int k = 0; k < KQ; ++k)
      m[k] = ld_keep(reinterpret_cast<const u32x4*>(src + 4 * (w0 + 4 * (uint64_t)(k * kBlock + tid))));
  } else {  // the last super tile: words past W count as 0, bytes past the readable size read as 0
    for (int k = 0; k < KQ; ++k) {
      const uint64_t g = w0 + 4 * (uint64_t)(k * kBlock + tid);
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
  uint32_t err = 0;
#pragma unroll
  for (int k = 0; k < KQ; ++k) {
    const uint32_t qi = (uint32_t)(k * kBlock + tid);
    const uint64_t g = w0 + 4 * (uint64_t)qi;
    uint32_t cnt = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t w = m[k][i];
      if (g + i == W - 1 && (n & 31)) {
        const uint32_t valid = (1u << (n & 31)) - 1;
        if (w & ~valid) err |= CDMA_E_MASK_PAST_N;
        w &= valid;
      }
      cnt += (uint32_t)__builtin_popcount(w);
    }
    const uint32_t inc = wave_incl_scan(cnt);
    if constexpr (QT == 64) {
      if (lane == 63) s_cnt[qi / 64] = inc;
    } else {  // group total = inclusive prefix at its last lane minus that of the group before
      const uint32_t before = __shfl(inc, (lane - QT) & 63);
      if ((lane & (QT - 1)) == QT - 1) s_cnt[qi / QT] = inc - (lane >= QT ? before : 0u);
    }
  }
  __syncthreads();
  if (wave == 0) {
    const uint32_t c = lane < C::SUPER ? s_cnt[lane] : 0u;
    const uint32_t inc = wave_incl_scan(c);
    const uint64_t t = (uint64_t)u * C::SUPER + lane;
    if (lane < C::SUPER && t < num_tiles) local[t] = inc - c;
    if (lane == 63) sup[u] = inc;
  }
  if (err && error) atomicOr(error, err);
  // a stream to warm whole (warm_whole): every workgroup also reads its
  // share of the values (the masks it read are kept already), so the expand
  // pass reads the whole stream from the cache
  if (warm && eff > 4 * W && warm_whole(eff, (uint64_t)(512 / TWPT) * n)) {
    const uint64_t q0 = 4 * W / 16, q1 = eff / 16;
    const uint64_t per = (q1 - q0 + gridDim.x - 1) / gridDim.x;
    const uint64_t a = q0 + (uint64_t)u * per, b = a + per < q1 ? a + per : q1;
    if (a < b) warm_quads(src, a, b, (uint64_t)tid, kBlock);
  }
}

// Exclusive prefix sums of sup[0..count) in place, total in sup[count]; one
// workgroup of kScanBlock threads.
constexpr int kScanBlock = 1024;

// It also clears the expand pass's nsync read-ahead counters.
__global__ __launch_bounds__(kScanBlock) void zvc_scan_kernel(uint32_t* __restrict__ sup, uint32_t count,
                                                             uint32_t* __restrict__ sync, uint32_t nsync) {
  __shared__ uint32_t s_wave[kScanBlock / 64];
  __shared__ uint32_t s_carry;
  const int tid = threadIdx.x;
  const int lane = (int)lane_id();
  const int wave = tid >> 6;
  if (tid == 0) s_carry = 0;
  for (uint32_t i = tid; i < nsync; i += kScanBlock) sync[i] = 0;
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
// decompress, pass 3: expand
// ---------------------------------------------------------------------------
//
// With the offsets known, tiles are independent: a tile's masks and value
// quads are fetched into registers, staged in LDS and expanded (the kernel at
// the end of this file runs one tile per workgroup).

template <int ESZ, int V>
struct ZvcExpandShape {
  using S = ZvcShape<ESZ, V>;
  // A tile's values span at most TE * ESZ bytes, i.e. TE * ESZ / 16 quads
  // plus one when the span starts mid-quad: QPT per thread, and the one
  // extra quad (its address is uniform) by a scalar load.
  static constexpr int QPT = S::TE * ESZ / 16 / kBlock;  // value quads per thread
  static_assert(QPT * kBlock * 16 == S::TE * ESZ && S::STAGE >= S::TE * ESZ + 16, "expand staging shape");
  static constexpr int MPT = (S::WPT + kBlock - 1) / kBlock;                // mask words per thread
};

template <int ESZ, int V>
struct ZvcTileIn {
  using X = ZvcExpandShape<ESZ, V>;
  u32x4 q[X::QPT];
  u32x4 qx;  // the quad after the QPT * kBlock ones (uniform)
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
        w = ld_keep(reinterpret_cast<const uint32_t*>(src) + g);
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
  {
    const uint64_t q = q0 + (uint64_t)X::QPT * kBlock;
    u32x4 d = {0u, 0u, 0u, 0u};
    if (q < q1) {
      const uint64_t qb = q << 4;
      if (qb + 16 <= eff) {
        d = *reinterpret_cast<const u32x4*>(src + qb);
      } else {
        for (int b = 0; b < 16; b += ESZ) {
          if (qb + b + ESZ <= eff) vec_set<ESZ>(d, b / ESZ, load_elem<ESZ>(src + qb + b));
          else if (qb + b >= in.beg && qb + b < in.end) in.short_read = true;
        }
      }
    }
    in.qx = d;
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
    if (q < q1) *reinterpret_cast<u32x4*>(L.stage + 16 * (q - q0)) = in.q[k];
  }
  if (tid == 0 && q0 + (uint64_t)X::QPT * kBlock < q1)
    *reinterpret_cast<u32x4*>(L.stage + 16 * X::QPT * kBlock) = in.qx;
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
  // The offsets come from the same masks, so the tile's values are exactly
  // its set bits and every bit's value is staged.  Straight-line: every
  // element reads the value its bit would take (at most value index TE,
  // inside the stage) and keeps it only if the bit is set.
  const uint32_t shift = (uint32_t)(in.beg & 15);
  const uint64_t e_tile = (uint64_t)t * S::TE;
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const uint32_t c = (uint32_t)((wave * V + j) * 64 + lane);
    const uint8_t* pv = L.stage + shift + ESZ * (base[j] + ex[j]);
    u32x4 o = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < S::EPL; ++k) {
      const int32_t keep = __builtin_amdgcn_sbfe((int32_t)bits[j], k, 1);  // 0 or -1
      vec_set<ESZ>(o, k, load_elem<ESZ>(pv) & (uint32_t)keep);
      pv -= ESZ * keep;
    }
    store_vec<ESZ>(dst, e_tile + (uint64_t)c * S::EPL, n, o);
  }
  __syncthreads();
  return total;
}

// Value offset of tile t (t <= num_tiles) from the two count passes, whose
// super tiles hold 2^shift tiles.
__device__ __forceinline__ uint32_t zvc_tile_offset(const uint32_t* __restrict__ local,
                                                    const uint32_t* __restrict__ sup, uint32_t t,
                                                    uint32_t num_tiles, uint32_t shift) {
  if (t >= num_tiles) return sup[(num_tiles + (1u << shift) - 1) >> shift];  // the grand total
  return sup[t >> shift] + local[t];
}

// Pass 3: one tile per workgroup, no inter-workgroup dependency for
// correctness.  Workgroups are dispatched in block order, and each XCD takes
// one contiguous range of tiles (xcd_tile), so the tiles in flight stay a few
// narrow windows of the output and of the stream.  How many are in flight per
// CU is set by the launcher (see expand_lds_pad): more workgroups hide the
// latency of the mask and value reads when a tile has few values, fewer keep
// the mixed read/write traffic efficient when it has many.
//
// Read-ahead chunks.  When the stream is large but a small share of the
// output (high sparsity), its reads, scattered through the output's write
// stream, slow HBM far more than their bytes (s = 0.9, fp32: 66 % of peak
// against 75 % at s = 0.5).  The grid is then cut into chunks of chunk_tiles
// tiles, each preceded by warm_groups read-ahead workgroups that read the
// chunk's masks and values once with caching loads (a short pure-read burst
// that leaves them in the memory-side cache).  They count themselves done on
// two levels (sixteen sub-counters, then one top counter, so no word takes
// more than a few dozen atomics), and the last one raises kAheadFlags copies
// of a done flag, each on a cache line of its own.  The chunk's first expand
// workgroups (those that can be resident before the read-ahead ends: block
// index within the chunk below wait_window) poll one copy each, sleeping
// between polls, with a bounded spin; a thousand waiters polling one word
// slow the memory channel that holds it enough to stall the read-ahead
// itself.  The expand pass then reads from the cache, and its HBM traffic is
// its writes.  Whether a chunk is read ahead is decided on the device,
// identically by every workgroup, from the offsets: not when the whole
// stream fits in the cache (the count pass read it), when the stream is over
// CDMA_AHEAD_MAX_PCT percent of the output, or when the chunk's share
// exceeds CDMA_WARM_BYTES.  The waits only order memory traffic; the result
// does not depend on them.
#ifndef CDMA_AHEAD_SPIN
#define CDMA_AHEAD_SPIN 1000
#endif
#ifndef CDMA_AHEAD_SLEEP
#define CDMA_AHEAD_SLEEP 32
#endif
// Per chunk in sync[], one 128-byte line each: the top counter, kAheadSubs
// sub-counters of finished read-ahead workgroups, and kAheadFlags copies of
// the done flag.
constexpr uint32_t kAheadSubs = 16;
constexpr uint32_t kAheadFlags = 15;
constexpr uint32_t kAheadSyncWords = 32 * (1 + kAheadSubs + kAheadFlags);

template <int ESZ, int V>
__global__ __launch_bounds__(kBlock) void zvc_expand_kernel(
    const uint8_t* __restrict__ src, uint64_t src_capacity, const uint64_t* __restrict__ src_bytes,
    uint64_t n, uint8_t* __restrict__ dst, uint32_t* __restrict__ error,
    const uint32_t* __restrict__ local, const uint32_t* __restrict__ sup, uint32_t num_tiles, uint32_t super_shift,
    uint32_t chunk_tiles, uint32_t warm_groups, uint32_t wait_window, uint32_t lead, uint32_t* __restrict__ sync) {
  __shared__ ZvcExpandLds<ESZ, V> L;
  constexpr int WPT = ZvcShape<ESZ, V>::WPT;
  const int tid = threadIdx.x;
  const int lane = (int)lane_id();
  const int wave = tid >> 6;
  // Block order: chunk k's read-ahead group (warm_groups blocks) sits `lead`
  // expand blocks before chunk k's first expand block (chunk 0's first of
  // all), so it runs during the tail of chunk k - 1.  Decode this block into
  // (chunk c, read-ahead index r < warm_groups) or (chunk c, expand index
  // warm_groups + i within the chunk).
  uint32_t c = 0, r = blockIdx.x;
  if (warm_groups) {
    const uint32_t nch = (num_tiles + chunk_tiles - 1) / chunk_tiles;
    uint32_t nw = 0;  // read-ahead groups before this block
    bool warm_block = false;
    for (uint32_t k = 0; k < nch; ++k) {
      const uint32_t start = (k ? k * chunk_tiles - lead : 0u) + k * warm_groups;
      if (blockIdx.x < start) break;
      if (blockIdx.x < start + warm_groups) {
        c = k;
        r = blockIdx.x - start;
        warm_block = true;
        break;
      }
      nw = k + 1;
    }
    if (!warm_block) {
      const uint32_t e = blockIdx.x - nw * warm_groups;  // expand block in tile order
      c = e / chunk_tiles;
      r = warm_groups + e % chunk_tiles;
    }
  }
  const uint32_t t0 = c * chunk_tiles;
  const uint32_t t1 = num_tiles - t0 < chunk_tiles ? num_tiles : t0 + chunk_tiles;
  const uint64_t W = (n + 31) / 32;
  const uint64_t claimed = src_bytes ? *src_bytes : src_capacity;
  const uint64_t eff = claimed < src_capacity ? claimed : src_capacity;
  if (warm_groups && (r < warm_groups || r - warm_groups < wait_window)) {
    uint64_t m0 = 4ull * WPT * t0, m1 = 4ull * WPT * t1;
    if (m1 > 4 * W) m1 = 4 * W;
    uint64_t v0 = 4 * W + (uint64_t)ESZ * zvc_tile_offset(local, sup, t0, num_tiles, super_shift);
    uint64_t v1 = 4 * W + (uint64_t)ESZ * zvc_tile_offset(local, sup, t1, num_tiles, super_shift);
    const uint64_t stream = 4 * W + (uint64_t)ESZ * zvc_tile_offset(local, sup, num_tiles, num_tiles, super_shift);
    if (m1 > eff) m1 = eff;
    if (v1 > eff) v1 = eff;
    if (m0 > m1) m0 = m1;
    if (v0 > v1) v0 = v1;
    const bool ahead = !warm_whole(stream, (uint64_t)ESZ * n) && stream * 100 <= (uint64_t)ESZ * n * CDMA_WARM_MAX_PCT &&
                       (m1 - m0) + (v1 - v0) <= (uint64_t)CDMA_WARM_BYTES;
    if (r < warm_groups) {  // a read-ahead workgroup: its strided share of the chunk
      if (!ahead) return;
      const uint64_t start = (uint64_t)r * kBlock + tid, stride = (uint64_t)warm_groups * kBlock;
      warm_quads(src, m0 / 16, m1 / 16, start, stride);
      warm_quads(src, v0 / 16, v1 / 16, start, stride);
      __syncthreads();
      if (tid == 0) {
        // two-level count, so that no counter takes more than a few dozen
        // atomics: the last arrival at each sub-counter counts at the top,
        // and the last arrival at the top raises the flag copies
        uint32_t* cs = sync + (uint64_t)c * kAheadSyncWords;
        const uint32_t j = r % kAheadSubs;
        const uint32_t subs = warm_groups < kAheadSubs ? warm_groups : kAheadSubs;
        const uint32_t expect = warm_groups / kAheadSubs + (j < warm_groups % kAheadSubs ? 1u : 0u);
        if (__hip_atomic_fetch_add(cs + 32 * (1 + j), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                expect - 1 &&
            __hip_atomic_fetch_add(cs, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == subs - 1)
          for (uint32_t k = 0; k < kAheadFlags; ++k)
            __hip_atomic_store(cs + 32 * (1 + kAheadSubs + k), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      return;
    }
    if (ahead) {
      // waiters spread their polls over the flag copies (one cache line each)
      if (tid == 0) {
        const uint32_t* flag = sync + (uint64_t)c * kAheadSyncWords + 32 * (1 + kAheadSubs + blockIdx.x % kAheadFlags);
        for (uint32_t k = 0; k < CDMA_AHEAD_SPIN; ++k) {
          if (__hip_atomic_load(const_cast<uint32_t*>(flag), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) break;
          __builtin_amdgcn_s_sleep(CDMA_AHEAD_SLEEP);
        }
      }
      __syncthreads();
    }
  }
  const uint32_t t = t0 + xcd_tile(r - warm_groups, t1 - t0);  // this workgroup's tile
  ZvcTileIn<ESZ, V> in;
  zvc_fetch_tile<ESZ, V>(in, src, eff, W, t, zvc_tile_offset(local, sup, t, num_tiles, super_shift),
                         zvc_tile_offset(local, sup, t + 1, num_tiles, super_shift), tid);
  // E_SIZE with a size word: the masks describe another size, or the size
  // exceeds the readable capacity (bytes past the end read as 0); without
  // one: described values lie past the capacity
  uint32_t err = in.short_read && !src_bytes ? CDMA_E_SIZE : 0u;
  zvc_expand_tile<ESZ, V>(L, in, t, n, dst, tid, wave, lane);
  if (t == num_tiles - 1 && tid == 0 && src_bytes && (in.end != *src_bytes || *src_bytes > src_capacity))
    err |= CDMA_E_SIZE;
  if (err && error) atomicOr(error, err);
}

}  // namespace cdma
