// zvci_kernels.hpp -- ZVC in its per-window interleaved form, for gfx950.
//
// "Compressing DMA Engine: Leveraging Activation Sparsity for Training Deep
// Neural Networks", §V.A Compression Algorithm: each window of 32 values is
// coded as its 32-bit nonzero mask followed by its nonzero values.  Windows
// follow each other in order; in front sits an index u32 val_off[Wr+1], the
// nonzeros before each block of E = 4096/ESZ elements (the 4 KB window of
// §VII.A), so a block starts at 4(Wr+1) + 4*b*(E/32) + ESZ*val_off[b] and can be
// decoded without the blocks before it.  Same masks and values as the
// masks-then-values stream of zvc_common.hpp, in a different order.
//
// compress:   the run-length compressor's pipeline (persistent workgroups, one
//             data wavefront per block, a control wavefront drawing tickets
//             (ticket classes once the whole grid has started) and
//             chain-summing the tiles' nonzero counts), with the block built in
//             LDS as mask, values, mask, values, ...: the mask of window w goes
//             to 4w + ESZ*(nonzeros before w), a lane's values to
//             4(w+1) + ESZ*(nonzeros before the lane), both from the wave's
//             prefix sums of per-lane counts.
// decompress: one wavefront per block: the index gives the block's place, the
//             block is read into LDS, the masks are walked in order (each
//             window starts after the previous window's values, so this step is
//             sequential: by one wave per block, or for sparse workgroups by
//             one wave with a lane per block), and then every lane expands its
//             16-byte vector.
#pragma once

#include "rle_kernels.hpp"  // stream_u32
#include "zvc_common.hpp"

namespace cdma {

template <int ESZ>
struct ZviShape {
  static constexpr int V = 4;                   // 16-byte vectors per lane
  static constexpr int EPL = 16 / ESZ;          // elements per vector
  static constexpr int LPW = 32 / EPL;          // lanes per 32-element window
  static constexpr int E = 4096 / ESZ;          // elements per index block (one wavefront)
  static constexpr int WPB = E / 32;            // windows per block: 32 (fp32) / 64 (fp16)
  static constexpr int WPV = 64 / LPW;          // windows per 16-byte vector row of the wave
  static constexpr int BLKMAX = 4 * WPB + 4096;  // largest block in bytes
  static_assert(V * 64 * EPL == E, "a wavefront must cover one block");
};

template <int ESZ>
struct ZviCShape : ZviShape<ESZ> {
  static constexpr int BLOCK = 1024;                 // threads
  static constexpr int NW = BLOCK / 64 - 1;          // blocks per tile: one per data wave
  static constexpr int TE = NW * ZviShape<ESZ>::E;   // elements per tile
  static constexpr int STAGE = NW * ZviShape<ESZ>::BLKMAX + 16;
};

template <int ESZ>
struct ZviCLds {
  using S = ZviCShape<ESZ>;
  uint64_t excl;                          // exclusive nonzero prefix of the tile stored this iteration
  uint32_t total2, span2;                 // and its nonzeros and staged bytes
  uint32_t total[2], span[2];             // nonzeros / staged bytes of the tile classified in an iteration of parity b
  uint32_t vw[S::NW], bw[S::NW];          // per-block nonzeros and bytes of the tile being classified
  uint32_t next;                          // ticket handed from the control wave to the data waves
  uint32_t mode;                          // start_mode's choice (selects the ticket source)
  uint32_t init[3];                       // the first three tickets
  __attribute__((aligned(16))) uint8_t stage[2][S::STAGE];
};

// What a data lane keeps of its block from the classify to the compaction
// one iteration later: the element nonzero bits of its V rows (EPL bits at
// EPL*j of bits), the block's nonzeros before the lane's elements of each row
// (16 bits at 16*(j%2) of pre[j/2]), and the block's place in its tile (Bb
// staged bytes and Vb nonzeros before it; nwin windows; all the same on every
// lane).
template <int V>
struct ZviLane {
  uint32_t bits;
  uint32_t pre[V / 2];
  uint32_t nwin, Bb, Vb;
  __device__ __forceinline__ uint32_t pre_of(int j) const { return __builtin_amdgcn_ubfe(pre[j / 2], 16 * (j % 2), 16); }
};

// 32-bit LDS word at a 2-byte aligned address, as two halves.
__device__ __forceinline__ void lds_u32_at2(uint8_t* base, uint32_t byte, uint32_t v) {
  *reinterpret_cast<uint16_t*>(base + byte) = (uint16_t)v;
  *reinterpret_cast<uint16_t*>(base + byte + 2) = (uint16_t)(v >> 16);
}
__device__ __forceinline__ uint32_t lds_get_u32_at2(const uint8_t* base, uint32_t byte) {
  return (uint32_t)*reinterpret_cast<const uint16_t*>(base + byte) |
         ((uint32_t)*reinterpret_cast<const uint16_t*>(base + byte + 2) << 16);
}

// Load tile t's blocks, one per data wave, issued on every path (see
// rle_c_load_full).
template <int ESZ>
__device__ __forceinline__ void zvi_c_load_full(u32x4 (&v)[ZviShape<ESZ>::V], const uint8_t* __restrict__ src,
                                                uint32_t t, bool valid, int wave, int lane) {
  using S = ZviCShape<ESZ>;
  const uint8_t* p = src + (uint64_t)t * (S::NW * 4096);  // uniform tile base
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p), (short)0, valid ? S::NW * 4096 : 0, kBufferFlags);
  const uint32_t o = (uint32_t)(wave * 4096 + lane * 16);
#pragma unroll
  for (int j = 0; j < S::V; ++j) v[j] = __builtin_amdgcn_raw_buffer_load_b128(r, o + j * 1024, 0, kLoadAux);
}

// Classify tile t's block of this data wave (its vectors in cur): per-lane
// row bits and in-block prefixes to q, the block's nonzeros and staged bytes
// to L.vw / L.bw.
template <int ESZ>
__device__ __forceinline__ void zvi_c_classify(ZviCLds<ESZ>& L, u32x4 (&cur)[ZviShape<ESZ>::V],
                                               ZviLane<ZviShape<ESZ>::V>& q, uint32_t t, uint32_t full, uint64_t Wr,
                                               const uint8_t* __restrict__ src, uint64_t n, int wave, int lane) {
  using S = ZviCShape<ESZ>;
  constexpr int V = S::V;
  const uint64_t gw = (uint64_t)t * S::NW + wave;
  const uint64_t e_win = gw * S::E;
  const uint32_t Lw = gw < Wr ? (uint32_t)(n - e_win < (uint64_t)S::E ? n - e_win : S::E) : 0u;
  q.nwin = (Lw + 31) / 32;
  if (t >= full) {  // the one partial tile: load bounded, drain so nothing stays pending on cur
    uint32_t el = (uint32_t)lane * S::EPL;
    asm volatile("" : "+v"(el));
    for (int j = 0; j < V; ++j) cur[j] = load_vec<ESZ>(src, e_win + (el + (uint32_t)(j * 64 * S::EPL)), n);
    __builtin_amdgcn_s_waitcnt(0);
  }
  uint32_t v_w = 0;
  q.bits = 0;
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const uint32_t bits = vec_nz_bits<ESZ>(cur[j]);
    const uint32_t cnt = (uint32_t)__builtin_popcount(bits);
    const uint32_t inc = wave_incl_scan(cnt);
    const uint32_t pre = v_w + inc - cnt;  // nonzeros of the block before this lane's elements of row j
    q.bits |= bits << (S::EPL * j);
    if (j % 2 == 0) q.pre[j / 2] = pre;
    else q.pre[j / 2] |= pre << 16;
    v_w += read_lane(inc, 63);
  }
  if (lane == 0) {
    L.vw[wave] = v_w;
    L.bw[wave] = 4 * q.nwin + ESZ * v_w;
  }
}

// Write the block (mask, values, mask, values, ...) into stage st at the
// block's place in its tile (data waves).
template <int ESZ>
__device__ __forceinline__ void zvi_c_compact(uint8_t* __restrict__ stage, const u32x4 (&v)[ZviShape<ESZ>::V],
                                              const ZviLane<ZviShape<ESZ>::V>& q, int lane) {
  using S = ZviCShape<ESZ>;
  uint8_t* st = stage + q.Bb;
#pragma unroll
  for (int j = 0; j < S::V; ++j) {
    const uint32_t bits = __builtin_amdgcn_ubfe(q.bits, S::EPL * j, S::EPL);
    const uint32_t msk = group_or<S::LPW>(bits << ((lane % S::LPW) * S::EPL));
    const uint32_t pre = q.pre_of(j);
    const uint32_t wl = (uint32_t)(j * S::WPV + lane / S::LPW);  // window of this lane in the block
    if (wl < q.nwin) {
      // the window's mask sits after the masks and values of the windows before it
      if (lane % S::LPW == 0) {  // the window's first lane: nothing of the window before it
        if constexpr (ESZ == 4) *reinterpret_cast<uint32_t*>(st + 4 * wl + ESZ * pre) = msk;
        else lds_u32_at2(st, 4 * wl + ESZ * pre, msk);
      }
      uint32_t pos = 4 * (wl + 1) + ESZ * pre;
#pragma unroll
      for (int k = 0; k < S::EPL; ++k) {
        if ((bits >> k) & 1u) {
          store_elem<ESZ>(st + pos, vec_elem<ESZ>(v[j], k));
          pos += ESZ;
        }
      }
    }
  }
}

// One iteration of the two-deep pipeline (see rle_c_iteration): t is
// classified, tp1 compacted into stage[b ^ 1] from prev (whose registers then
// take tl's loads), tp2 stored from stage[b].  V2b: the nonzero base of tp2's
// block of this wave (read, then set to tp1's).
template <int ESZ>
__device__ __forceinline__ uint32_t zvi_c_iteration(ZviCLds<ESZ>& L, u32x4 (&cur)[ZviShape<ESZ>::V],
                                                    u32x4 (&prev)[ZviShape<ESZ>::V], ZviLane<ZviShape<ESZ>::V>& q,
                                                    const ZviLane<ZviShape<ESZ>::V>& qp, uint32_t& V2b, RleCtl& C,
                                                    uint32_t t, uint32_t tp1, uint32_t tp2, uint32_t tl, int b,
                                                    uint32_t full, uint64_t Wr, const uint8_t* __restrict__ src,
                                                    uint64_t n, uint8_t* __restrict__ dst,
                                                    uint64_t* __restrict__ out_bytes, uint32_t* __restrict__ agg,
                                                    const Tickets& tk, uint32_t num_tiles, int tid, int wave,
                                                    int lane) {
  using S = ZviCShape<ESZ>;
  const bool have_t = t < num_tiles;
  const bool have_p1 = tp1 < num_tiles;
  const bool have_p2 = tp2 < num_tiles;
  const bool data = wave < S::NW;
  const uint64_t H = 4 * (Wr + 1);

  // ---- phase X ----
  if (data && have_p1 && qp.nwin) zvi_c_compact<ESZ>(L.stage[b ^ 1], prev, qp, lane);
  {
    const bool load = __builtin_amdgcn_readfirstlane(wave) < S::NW && tl < full;
    zvi_c_load_full<ESZ>(prev, src, tl, load, wave, lane);
  }
  if (data) {
    if (have_t) zvi_c_classify<ESZ>(L, cur, q, t, full, Wr, src, n, wave, lane);
  } else if (have_p2) {
    bool stuck = false;
    const uint64_t X = C.pfx + chain_sum(agg, C.chain_lo, tp2, C.cr, &stuck, [](uint32_t v) { return v; });
    const uint32_t T2 = L.total[b];  // tp2 was classified two iterations ago
    if (lane == 0) {
      L.excl = X;
      L.total2 = T2;
      L.span2 = L.span[b];
      if (stuck) atomicMax(reinterpret_cast<unsigned long long*>(out_bytes), kSizeInternalError);
    }
    C.pfx = X + T2;  // tp2's inclusive prefix
  }
  __syncthreads();

  // ---- phase Y ----
  if (data) {
    if (have_t) {  // t's block bases inside its tile
      const uint32_t bl = lane < S::NW ? L.bw[lane] : 0u;
      const uint32_t vl = lane < S::NW ? L.vw[lane] : 0u;
      const uint32_t bi = wave_incl_scan(bl), vi = wave_incl_scan(vl);
      q.Bb = read_lane(bi - bl, wave);
      q.Vb = read_lane(vi - vl, wave);
    }
    if (have_p2) {
      const uint64_t X = L.excl;
      // full tiles only precede tp2, so the windows before it are tp2 * NW * WPB
      const uint64_t O = H + 4 * ((uint64_t)tp2 * S::NW * S::WPB) + (uint64_t)ESZ * X;
      const uint32_t span = L.span2;
      store_staged<ESZ == 4 ? 4 : 2, S::NW * 64>(L.stage[b], span, O, dst, tid);
      const uint64_t w = (uint64_t)tp2 * S::NW + wave;
      if (lane == 0 && w < Wr) reinterpret_cast<uint32_t*>(dst)[w] = (uint32_t)(X + V2b);
      if (tp2 == num_tiles - 1 && tid == 0) {
        reinterpret_cast<uint32_t*>(dst)[Wr] = (uint32_t)(X + L.total2);
        atomicMax(reinterpret_cast<unsigned long long*>(out_bytes), O + span);
      }
    }
  } else {
    // control wave (see rle_c_iteration)
    __builtin_amdgcn_s_waitcnt(0);
    if (lane == 0) L.next = tk.tile(C.pend);
    if (lane == 0 && have_t) C.pend = tk.raw();
    if (have_t) {
      const uint32_t vl = lane < S::NW ? L.vw[lane] : 0u;
      const uint32_t bl = lane < S::NW ? L.bw[lane] : 0u;
      const uint32_t T = read_lane(wave_incl_scan(vl), 63), B = read_lane(wave_incl_scan(bl), 63);
      if (lane == 0) {
        L.total[b] = T;
        L.span[b] = B;
        agg_publish(agg, t, T);
      }
    }
    if (have_p1) {
      C.chain_lo = have_p2 ? (uint64_t)tp2 + 1 : 0;
      chain_issue(agg, C.chain_lo, tp1, C.cr);
    }
  }
  V2b = qp.Vb;
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(L.next);  // uniform: keeps tile bases in SGPRs
}

template <int ESZ>
__global__ __launch_bounds__(ZviCShape<ESZ>::BLOCK) void zvci_compress_kernel(
    const uint8_t* __restrict__ src, uint64_t n, uint8_t* __restrict__ dst,
    uint64_t* __restrict__ out_bytes, uint32_t* __restrict__ counter,
    uint32_t* __restrict__ agg, uint32_t num_tiles) {
  using S = ZviCShape<ESZ>;
  __shared__ ZviCLds<ESZ> L;
  const int tid = threadIdx.x;
  const int lane = (int)lane_id();
  const int wave = tid >> 6;
  const uint64_t Wr = (n + S::E - 1) / S::E;
  const uint32_t full = (uint32_t)(n / S::TE);  // tiles with no element past n
  if (tid == 0) L.mode = start_mode(counter);
  __syncthreads();
  const Tickets tk = ticket_source(counter, __builtin_amdgcn_readfirstlane(L.mode));
  if (tid < 3 * 64 && lane == 0) L.init[wave] = tk.raw();
  __syncthreads();
  // raw counter values of the first three tickets in increasing order (a
  // class's tiles increase with them): classify, load, hand over
  const uint32_t a = __builtin_amdgcn_readfirstlane(L.init[0]);
  const uint32_t b = __builtin_amdgcn_readfirstlane(L.init[1]);
  const uint32_t c = __builtin_amdgcn_readfirstlane(L.init[2]);
  const uint32_t lo = min(a, min(b, c)), hi = max(a, max(b, c));
  uint32_t t = tk.tile(lo);
  uint32_t tl = tk.tile(a + b + c - lo - hi);
  uint32_t tp1 = num_tiles, tp2 = num_tiles;
  RleCtl C;
  C.chain_lo = 0;
  C.pfx = 0;
  C.pend = hi;
  ZviLane<S::V> qa, qb;
  qa.nwin = qb.nwin = 0;
  qa.Bb = qa.Vb = qb.Bb = qb.Vb = 0;
  uint32_t V2b = 0;
  u32x4 ra[S::V], rb[S::V];
  zvi_c_load_full<ESZ>(ra, src, t, __builtin_amdgcn_readfirstlane(wave) < S::NW && t < full, wave, lane);
  for (;;) {
    uint32_t r = zvi_c_iteration<ESZ>(L, ra, rb, qa, qb, V2b, C, t, tp1, tp2, tl, 0, full, Wr, src, n, dst,
                                      out_bytes, agg, tk, num_tiles, tid, wave, lane);
    tp2 = tp1;
    tp1 = t;
    t = tl;
    tl = r;
    r = zvi_c_iteration<ESZ>(L, rb, ra, qb, qa, V2b, C, t, tp1, tp2, tl, 1, full, Wr, src, n, dst, out_bytes, agg,
                             tk, num_tiles, tid, wave, lane);
    tp2 = tp1;
    tp1 = t;
    t = tl;
    tl = r;
    if (t >= num_tiles && tp1 >= num_tiles && tp2 >= num_tiles) break;
  }
}

// ---------------------------------------------------------------------------
// decompress: one wavefront per block
// ---------------------------------------------------------------------------

// Percent of values below which a workgroup walks its blocks' masks in one
// wave, a lane per block (see the walk below).  A 16-bit block has twice the
// mask words of a 32-bit one, so its per-block walks cost more and the shared
// walk pays at every density (above 100: always taken).
#ifndef CDMA_ZVCI_SHARED_PCT
#define CDMA_ZVCI_SHARED_PCT 90
#endif
#ifndef CDMA_ZVCI_SHARED_PCT16
#define CDMA_ZVCI_SHARED_PCT16 101
#endif

template <int ESZ>
__global__ __launch_bounds__(kBlock) void zvci_decompress_kernel(
    const uint8_t* __restrict__ src, uint64_t src_capacity, const uint64_t* __restrict__ src_bytes,
    uint64_t n, uint8_t* __restrict__ dst, uint32_t* __restrict__ error, uint32_t num_tiles) {
  using S = ZviShape<ESZ>;
  constexpr int V = S::V;
  constexpr int WSTAGE = S::BLKMAX + 32;
  __shared__ uint32_t s_err;
  __shared__ uint32_t s_mask[kWaves][S::WPB];  // each window's mask (bits past n cleared)
  __shared__ uint32_t s_vpos[kWaves][S::WPB];  // staged byte of each window's mask
  __shared__ __attribute__((aligned(16))) uint8_t s_blk[kWaves][WSTAGE];
  __shared__ uint32_t s_span[kWaves], s_shift[kWaves], s_nv[kWaves], s_valid[kWaves];  // for the walk
  __shared__ uint32_t s_zero[kWaves];  // block known to hold only zero masks: no walk

  const int tid = threadIdx.x;
  const int lane = (int)lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: block math stays scalar
  const uint32_t t = blockIdx.x;  // (the XCD-aware order measured slower here at s = 0.5)
  if (tid == 0) s_err = 0;
  const uint64_t claimed = src_bytes ? *src_bytes : src_capacity;
  const uint64_t eff = claimed < src_capacity ? claimed : src_capacity;
  const uint64_t Wr = (n + S::E - 1) / S::E;
  const uint64_t W = (n + 31) / 32;
  const uint64_t H = 4 * (Wr + 1);
  const uint64_t gw = (uint64_t)t * kWaves + wave;
  const uint64_t e_win = gw * S::E;
  const uint32_t Lw = gw < Wr ? (uint32_t)(n - e_win < (uint64_t)S::E ? n - e_win : S::E) : 0u;
  const uint32_t nwin = (Lw + 31) / 32;
  uint32_t err = 0;
  if (t == 0 && tid == 0 && stream_u32(src, eff, 0) != 0) err |= CDMA_E_INDEX;
  // E_SIZE with a size word: the index total describes another size, or the
  // size exceeds the readable capacity (bytes past the end read as 0)
  if (t == num_tiles - 1 && tid == 0 && src_bytes) {
    const uint64_t vt = stream_u32(src, eff, 4 * Wr);
    if (H + 4 * W + (uint64_t)ESZ * vt != *src_bytes || *src_bytes > src_capacity) err |= CDMA_E_SIZE;
  }
  __syncthreads();

  // this wave's block
  bool valid = false;
  uint32_t nv = 0;
  uint64_t B = 0, span = 0;
  if (Lw) {
    uint32_t iw = 0;  // lanes 0 and 1: val_off[gw], val_off[gw + 1]
    if (lane < 2) iw = stream_u32(src, eff, 4 * (gw + (uint64_t)lane));
    const uint32_t v0 = read_lane(iw, 0), v1 = read_lane(iw, 1);
    if (v1 < v0) {
      err |= CDMA_E_INDEX;
    } else {
      valid = true;
      nv = v1 - v0;
      B = H + 4 * gw * S::WPB + (uint64_t)ESZ * v0;
      // never stage more than a block of this many windows can hold
      const uint64_t most = 4 * (uint64_t)nwin + (uint64_t)ESZ * 32 * nwin;
      span = 4 * (uint64_t)nwin + (uint64_t)ESZ * nv;
      if (span > most) span = most;
    }
  }
  uint8_t* blk = s_blk[wave];
  uint32_t shift = 0;
  if (valid) {
    const uint64_t beg = B, end = B + span;
    shift = (uint32_t)(beg & 15);
    const uint64_t base = beg - shift;                          // 16-byte aligned
    const uint32_t nq = (uint32_t)((end - base + 15) >> 4);     // 16-byte pieces to stage
    const uint64_t whole = eff > base ? (eff - base) >> 4 : 0;  // pieces that end by eff
    const uint32_t nfull = whole < nq ? (uint32_t)whole : nq;
    const u32x4* g = reinterpret_cast<const u32x4*>(src + base);
    // pieces per lane at most: nq * 16 <= WSTAGE
    stage_pieces<(WSTAGE + 1023) / 1024>(blk, g, nfull, (uint32_t)lane);
    if (nfull < nq) {  // the readable stream ends inside the block: bytes past it read as 0
      bool short_read = false;
      for (uint32_t i = nfull + (uint32_t)lane; i < nq; i += 64) {
        const uint64_t qb = base + 16 * (uint64_t)i;
        for (int k = 0; k < 16; k += 2) {
          const uint64_t b = qb + k;
          uint32_t e = 0;
          if (b + 2 <= eff) {
            e = *reinterpret_cast<const uint16_t*>(src + b);
          } else {
            if (b < eff) e = src[b];  // the last readable byte; the one after it reads as 0
            if (b >= beg && b < end) short_read = true;
          }
          *reinterpret_cast<uint16_t*>(blk + 16 * i + k) = (uint16_t)e;
        }
      }
      if (!src_bytes && __ballot(short_read)) err |= CDMA_E_SIZE;  // no size word: data past capacity
    }
  }
  // A block whose index claims no values is, if valid, nwin zero masks at 4w:
  // that is checked with one read per lane, and such a block skips the walk
  // (any nonzero word sends it through the walk, which reports the errors).
  bool zero_blk = false;
  if (valid && nv == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");  // this wave's own staged block
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const uint32_t q = 4 * (uint32_t)lane;  // span = 4 * nwin here
    uint32_t m = 0;
    if ((uint32_t)lane < nwin)
      m = ESZ == 4 ? *reinterpret_cast<const uint32_t*>(blk + shift + q) : lds_get_u32_at2(blk + shift, q);
    zero_blk = __ballot(m != 0) == 0;
    if (zero_blk && (uint32_t)lane < nwin) {
      s_mask[wave][lane] = 0;
      s_vpos[wave][lane] = q;
    }
  }
  if (lane == 0) {
    s_zero[wave] = zero_blk;
    s_valid[wave] = valid;
    s_span[wave] = (uint32_t)span;
    s_shift[wave] = shift;
    s_nv[wave] = nv;
  }
  __syncthreads();

  // walk the masks: window w starts after window w-1's mask and values, a
  // chain of dependent reads.  Unless the workgroup's blocks are nearly dense
  // (the percentage above, or more, of values) one wave walks them all, lane
  // b taking block b: the instruction stream, not the chain's latency, is the
  // cost, so one stream per workgroup beats one per block.  Dense blocks keep
  // one walk per wave.
  uint32_t tot = 0;
#pragma unroll
  for (int b = 0; b < kWaves; ++b) tot += s_nv[b];
  constexpr uint64_t kPct = ESZ == 4 ? CDMA_ZVCI_SHARED_PCT : CDMA_ZVCI_SHARED_PCT16;
  const bool shared_walk = (uint64_t)tot * 100 < kPct * kWaves * S::E;
  const int b = shared_walk ? lane : wave;
  // every block of the tile holds E elements (all tiles but the last)
  const bool full_tile = (uint64_t)(t + 1) * kWaves * S::E <= n;
  if (full_tile) {
    // Straight-line steps, two dependent ALU operations each: the value
    // count is read off the final position.  Masks are read where the chain
    // puts them, also past the span: the first mask that starts past it
    // follows more values than the index claims (4(w + 1) + ESZ C > span
    // = 4 WPB + ESZ nv gives C > nv), so the count check fails then, as it
    // does when such masks read as 0.  Each step adds at most 4 + 32 ESZ
    // bytes, so window w's mask lies below w (4 + 32 ESZ) + 4 <= BLKMAX:
    // every read stays in the stage.
    if (shared_walk ? (wave == 0 && lane < kWaves) : lane == 0) {
      if (s_valid[b] && !s_zero[b]) {
        const uint8_t* base = s_blk[b] + s_shift[b];
        const uint8_t* q = base;  // the chain runs on the LDS address itself
#pragma unroll 4
        for (uint32_t w = 0; w < (uint32_t)S::WPB; ++w) {
          const uint32_t m = ESZ == 4 ? *reinterpret_cast<const uint32_t*>(q) : lds_get_u32_at2(q, 0);
          s_mask[b][w] = m;
          s_vpos[b][w] = (uint32_t)(q - base);
          q += ESZ * ((uint32_t)__builtin_popcount(m) + 4 / ESZ);
        }
        if (((uint32_t)(q - base) - 4 * (uint32_t)S::WPB) / ESZ != s_nv[b]) err |= CDMA_E_VAL_COUNT;
      }
    }
  } else if (shared_walk ? (wave == 0 && lane < kWaves) : true) {
    if (s_valid[b] && !s_zero[b]) {
      const bool writer = shared_walk || lane == 0;
      const uint64_t gb = (uint64_t)t * kWaves + b;
      const uint64_t eb = gb * S::E;
      const uint32_t nwb = ((uint32_t)(n - eb < (uint64_t)S::E ? n - eb : S::E) + 31) / 32;
      const uint32_t spb = s_span[b];
      const uint8_t* base = s_blk[b] + s_shift[b];
      // the window holding element n - 1 when n is not a multiple of 32 (only
      // the last block has it; ~0 elsewhere)
      const uint32_t wtail = (n & 31) && gb * S::WPB + nwb == W ? nwb - 1 : ~0u;
      const uint32_t ok = (1u << (n & 31)) - 1;
      uint32_t p = 0, count = 0;
      for (uint32_t w = 0; w < nwb; ++w) {
        // 32-bit elements keep every mask 4-byte aligned (the block starts so)
        uint32_t m = 0;
        if (p + 4 <= spb)
          m = ESZ == 4 ? *reinterpret_cast<const uint32_t*>(base + p) : lds_get_u32_at2(base, p);
        count += (uint32_t)__builtin_popcount(m);
        if (w == wtail) {
          if (m & ~ok) err |= CDMA_E_MASK_PAST_N;
          m &= ok;
        }
        if (writer) {
          s_mask[b][w] = m;
          s_vpos[b][w] = p;
        }
        p += 4 + ESZ * (uint32_t)__builtin_popcount(m);
      }
      if (count != s_nv[b]) err |= CDMA_E_VAL_COUNT;
    }
  }
  __syncthreads();

  // expand
  if (full_tile && valid) {
    // Straight-line: every element reads the value its bit would take and
    // keeps it only if the bit is set.  Without an error, every set bit's
    // value lies in the span; with one, the output is unspecified, and the
    // reads stay below the window's mask position + 4 + 32 ESZ <= BLKMAX.
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const uint32_t wl = (uint32_t)(j * S::WPV + lane / S::LPW);
      const uint32_t c = (uint32_t)(j * 64 + lane);
      const uint32_t m = s_mask[wave][wl];
      const uint32_t sub = (lane % S::LPW) * S::EPL;
      const uint32_t bits = __builtin_amdgcn_ubfe(m, sub, S::EPL);
      const uint8_t* q =
          blk + shift + s_vpos[wave][wl] + 4 + ESZ * (uint32_t)__builtin_popcount(__builtin_amdgcn_ubfe(m, 0, sub));
      u32x4 o = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < S::EPL; ++e) {
        const int32_t keep = __builtin_amdgcn_sbfe((int32_t)bits, e, 1);  // 0 or -1
        vec_set<ESZ>(o, e, load_elem<ESZ>(q) & (uint32_t)keep);
        q -= ESZ * keep;
      }
      st_stream(reinterpret_cast<u32x4*>(dst + (e_win + (uint64_t)c * S::EPL) * ESZ), o);
    }
  } else {
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const uint32_t wl = (uint32_t)(j * S::WPV + lane / S::LPW);
    const uint32_t c = (uint32_t)(j * 64 + lane);
    u32x4 o = {0u, 0u, 0u, 0u};
    if (valid && wl < nwin) {
      const uint32_t m = s_mask[wave][wl];
      const uint32_t sub = (lane % S::LPW) * S::EPL;
      const uint32_t b = (m >> sub) & ((1u << S::EPL) - 1u);
      uint32_t at = s_vpos[wave][wl] + 4 + ESZ * (uint32_t)__builtin_popcount(m & ((1u << sub) - 1u));
#pragma unroll
      for (int k = 0; k < S::EPL; ++k) {
        if ((b >> k) & 1u) {
          if (at + ESZ <= (uint32_t)span) vec_set<ESZ>(o, k, load_elem<ESZ>(blk + shift + at));
          at += ESZ;
        }
      }
    }
    if (Lw == (uint32_t)S::E) st_stream(reinterpret_cast<u32x4*>(dst + (e_win + (uint64_t)c * S::EPL) * ESZ), o);
    else if (Lw) store_vec<ESZ>(dst, e_win + (uint64_t)c * S::EPL, n, o);
  }
  }

  if (err) atomicOr(&s_err, err);
  __syncthreads();
  if (tid == 0 && s_err && error) atomicOr(error, s_err);
}

}  // namespace cdma
