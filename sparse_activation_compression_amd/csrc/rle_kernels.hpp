// rle_kernels.hpp -- run-length variant of the activation codec for gfx950.
//
// "Compressing DMA Engine: Leveraging Activation Sparsity for Training Deep
// Neural Networks", §V.A Compression Algorithm: run-length coding exploits
// clustered zeros and nonzeros; §VII.A Compression Efficiency: 4 KB window.
//
// Stream: u32 run_off[Wr+1], u32 val_off[Wr+1], then per window of
// E = 4096/ESZ elements a block of p_w u16 run lengths (alternating zero and
// nonzero runs, zero run first; for ESZ == 4 an odd list gets one 0 pad
// entry) followed by its v_w nonzero elements.  run_off / val_off are the
// exclusive prefix sums of p_w / v_w.
//
// One wavefront owns one window: 4 vectors of 16 bytes per lane cover exactly
// E elements, so each window's bitmap (E/32 mask words), runs and values are
// produced by one wave.
//
// compress:   persistent workgroups of NW waves take tiles of NW windows from
//             tickets (ticket classes once the whole grid has started, see
//             ticket_source): load -> nonzero bits -> window masks in LDS (DPP
//             OR) -> run boundaries = mask XOR (mask shifted by one element) ->
//             per-window entry and nonzero counts -> run lengths (gaps between
//             boundaries) and values staged in LDS -> a chain sum over the
//             packed (entries, nonzeros) aggregates of the tiles since the
//             workgroup's previous tile, overlapped with the next tile, gives
//             the tile's byte offset -> realigned 16-byte
//             stores of the staged blocks and the tile's index entries.
// decompress: the index gives each window's block offset directly (no scan)
//             -> block read into LDS -> run starts by a wave prefix sum ->
//             boundary bitmap (LDS XOR) -> prefix-XOR turns boundaries back
//             into the nonzero bitmap, with each mask word's nonzero prefix ->
//             the same expansion as ZVC.
#pragma once

#include <type_traits>

#include "zvc_common.hpp"

namespace cdma {

template <int ESZ>
struct RleShape {
  static constexpr int V = 4;                      // 16-byte vectors per lane
  static constexpr int EPL = 16 / ESZ;             // elements per vector
  static constexpr int LPW = 32 / EPL;             // lanes per 32-element mask word
  static constexpr int E = 4096 / ESZ;             // window = one wavefront's elements
  static constexpr int WPW = E / 32;               // mask words per window (32 or 64)
  // largest block of a window that passes every decode check (bound derived
  // below, at the compressor)
  static constexpr int BLKMAX = ESZ == 4 ? 4 * E + 8 : 3 * E + 6;
  // decompress: the staged part of one window's block, plus alignment.  A
  // 32-bit block always fits.  16-bit staging stops at 4448 bytes, so that a
  // decoder wavefront's LDS stays under 5 KB and 8 wavefronts per SIMD fit;
  // only blocks of many short runs are longer (random data at half density
  // averages about 4.1 KB), and their remaining values are read from memory.
  static constexpr int WSTAGE = ESZ == 4 ? BLKMAX + 32 : 4480;
  static_assert(V * 64 * EPL == E, "a wavefront must cover one window");
};

constexpr uint32_t kLow31 = (1u << 31) - 1;

__device__ __forceinline__ uint32_t wave_incl_max(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true));   // row_shr:1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true));   // row_shr:2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true));   // row_shr:4
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true));   // row_shr:8
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));  // row_bcast:15
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));  // row_bcast:31
  return v;
}

__device__ __forceinline__ void lds_u16(uint8_t* base, uint32_t byte, uint32_t v) {
  *reinterpret_cast<uint16_t*>(base + byte) = (uint16_t)v;
}

// ---------------------------------------------------------------------------
// compress: persistent workgroups, one data wavefront per window
// ---------------------------------------------------------------------------
//
// The same pipeline as the ZVC compressor: a tile is NW windows, one per data
// wavefront, and the last wavefront is the control wave (tickets and offset
// chain sums).  A published aggregate packs the tile's run-entry and nonzero
// counts (each below 2^15) as (entries << 15) | nonzeros; offsets are summed
// as (entries << 31) | nonzeros, and the stream limit keeps both sums below
// 2^31, so the packed sums never carry between the fields.
//
// A window of L elements with v nonzeros has k <= min(v, L - v + 1) nonzero
// runs and at most 2k + 1 runs, so its block is at most 4L + 8 bytes for
// 32-bit and 3L + 6 bytes for 16-bit elements; BLKMAX bounds the staging.
// The decoder's checks (runs alternate from a zero run, none but the first is
// empty, they sum to L, the nonzero runs sum to v, padding only after an odd
// list) fix the same structure, so a block that passes them obeys the bound.

// Threads of a 16-bit compressor workgroup: its blocks stage up to 1.5x the
// window, so two stage buffers of 15 windows would not fit in LDS.
#ifndef CDMA_RLE_C16_BLOCK
#define CDMA_RLE_C16_BLOCK 832
#endif

template <int ESZ>
struct RleCShape {
  static constexpr int BLOCK = ESZ == 4 ? 1024 : CDMA_RLE_C16_BLOCK;  // threads
  static constexpr int NW = BLOCK / 64 - 1;             // windows per tile: one per data wave
  static constexpr int V = 4;
  static constexpr int EPL = 16 / ESZ;
  static constexpr int LPW = 32 / EPL;
  static constexpr int E = 4096 / ESZ;
  static constexpr int TE = NW * E;
  static constexpr int WPW = E / 32;
  static constexpr int BLKMAX = RleShape<ESZ>::BLKMAX;
  static constexpr int STAGE = NW * BLKMAX + 16;
  static_assert(V * 64 * EPL == E, "a wavefront must cover one window");
  static_assert(NW * (E + 2) < (1 << 15), "a tile's entries and nonzeros fit 15-bit fields");
};

template <int ESZ>
struct RleCLds {
  using S = RleCShape<ESZ>;
  uint64_t excl;                        // packed exclusive prefix of the tile stored this iteration
  uint64_t agg2;                        // and its packed aggregate
  uint64_t agg[2];                      // packed aggregate of the tile classified in an iteration of parity b
  uint32_t pv[S::NW];                   // per-window entries | nonzeros << 16 of the tile being classified
  uint32_t next;                        // ticket handed from the control wave to the data waves
  uint32_t mode;                        // start_mode's choice (selects the ticket source)
  uint32_t init[3];                     // the first three tickets
  uint32_t mask[2][S::NW * S::WPW];     // window masks of the tiles classified in iterations of parity b
  uint32_t pre[2][S::NW * S::WPW];      // nonzeros of the window before each mask word
  __attribute__((aligned(16))) uint8_t stage[2][S::STAGE];
};

// What a data lane keeps of its window from the classify to the compaction
// one iteration later.  Lw, r_w, p_w, Pb and Vb are the same on every lane.
struct RleLane {
  uint32_t T;      // run-boundary bits of this lane's window positions
  uint32_t texcl;  // boundaries before this lane in the window
  uint32_t Lw;     // window length (0: no window)
  uint32_t r_w;    // runs in the window
  uint32_t p_w;    // run entries (runs plus the 32-bit pad)
  uint32_t Pb, Vb; // entries / nonzeros of the tile's windows before this one
};

// Load tile t's windows, one per data wave.  As in the ZVC compressor, a
// buffer resource covers exactly the tile when it is full and valid, and
// nothing otherwise, so the loads are issued on every path (an invalid
// tile's, the control wave's and the partial tile's return zeros without
// touching memory) and the compiler counts exactly which are in flight.
template <int ESZ>
__device__ __forceinline__ void rle_c_load_full(u32x4 (&v)[RleCShape<ESZ>::V], const uint8_t* __restrict__ src,
                                                uint32_t t, bool valid, int wave, int lane) {
  using S = RleCShape<ESZ>;
  const uint8_t* p = src + (uint64_t)t * (S::NW * 4096);  // uniform tile base
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p), (short)0, valid ? S::NW * 4096 : 0, kBufferFlags);
  const uint32_t o = (uint32_t)(wave * 4096 + lane * 16);
#pragma unroll
  for (int j = 0; j < S::V; ++j) v[j] = __builtin_amdgcn_raw_buffer_load_b128(r, o + j * 1024, 0, kLoadAux);
}

// Apply the epilogue OP to a window's vectors in place and, if act is given,
// store them densely where they were loaded from.
template <int ESZ, int OP>
__device__ __forceinline__ void rle_c_epilogue(u32x4 (&v)[RleCShape<ESZ>::V], uint8_t* __restrict__ act,
                                               uint64_t n, uint32_t t, uint64_t e_win, bool full_tile, int wave,
                                               int lane) {
  using S = RleCShape<ESZ>;
#pragma unroll
  for (int j = 0; j < S::V; ++j) v[j] = apply_op<OP>(v[j]);
  if (!act) return;
  if (full_tile) {
    uint8_t* p = act + (uint64_t)t * (S::NW * 4096);
    uint32_t o = (uint32_t)(wave * 4096 + lane * 16);
    asm volatile("" : "+v"(o));
#pragma unroll
    for (int j = 0; j < S::V; ++j) st_stream(reinterpret_cast<u32x4*>(p + o + j * 1024), v[j]);
  } else {
#pragma unroll
    for (int j = 0; j < S::V; ++j)
      store_vec<ESZ>(act, e_win + (uint64_t)(lane * S::EPL + j * 64 * S::EPL), n, v[j]);
  }
}

// Packed (entries << 15 | nonzeros) aggregate word -> (entries << 31 | nonzeros).
struct RleAggDec {
  __device__ uint64_t operator()(uint32_t v) const { return ((uint64_t)(v >> 15) << 31) | (v & 0x7FFFu); }
};

// Classify tile t's window of this data wave (its vectors in cur): window
// masks and per-word nonzero prefixes to L.mask[b] / L.pre[b], the lane's
// run boundaries and counts to q, and the window's entry and nonzero counts
// to L.pv.  The window's mask words are written and read by this wave
// only, so a wave-level fence orders them.
template <int ESZ, int OP>
__device__ __forceinline__ void rle_c_classify(RleCLds<ESZ>& L, u32x4 (&cur)[RleCShape<ESZ>::V], RleLane& q, int b,
                                               uint32_t t, uint32_t full, uint64_t Wr, const uint8_t* __restrict__ src,
                                               uint64_t n, uint8_t* __restrict__ act, int wave, int lane) {
  using S = RleCShape<ESZ>;
  constexpr int V = S::V;
  const uint64_t gw = (uint64_t)t * S::NW + wave;
  const uint64_t e_win = gw * S::E;
  q.Lw = gw < Wr ? (uint32_t)(n - e_win < (uint64_t)S::E ? n - e_win : S::E) : 0u;
  // lane l takes SB = E/64 consecutive window positions starting at p0 (16 for
  // 4-byte elements, 32 for 2-byte), so every lane has a share of the runs
  constexpr uint32_t SB = (uint32_t)S::E / 64;
  const uint32_t p0 = SB * (uint32_t)lane;
  if (t >= full) {  // the one partial tile: load bounded, drain so nothing stays pending on cur
    uint32_t el = (uint32_t)lane * S::EPL;
    asm volatile("" : "+v"(el));
    for (int j = 0; j < V; ++j) cur[j] = load_vec<ESZ>(src, e_win + (el + (uint32_t)(j * 64 * S::EPL)), n);
    __builtin_amdgcn_s_waitcnt(0);
  }
  if constexpr (OP != kOpNone) rle_c_epilogue<ESZ, OP>(cur, act, n, t, e_win, t < full, wave, lane);
  uint32_t* wm = L.mask[b] + wave * S::WPW;
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const uint32_t bits = vec_nz_bits<ESZ>(cur[j]);
    const uint32_t m = group_or<S::LPW>(bits << ((lane % S::LPW) * S::EPL));
    if (lane % S::LPW == 0) wm[j * (64 / S::LPW) + lane / S::LPW] = m;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // nonzeros of the mask word this lane reads (lanes below WPW)
  const uint32_t c = (uint32_t)__builtin_popcount(lane < S::WPW ? wm[lane] : 0u);
  // boundary bits of this lane's positions: element i starts a run when it
  // differs from element i-1 (the element before the window counts as zero)
  uint32_t T = 0;
  if (p0 < q.Lw) {
    const uint32_t w0 = p0 / 32, sh = p0 % 32;
    const uint32_t m = wm[w0];
    const uint32_t before = sh ? (m >> (sh - 1)) & 1u : (w0 ? wm[w0 - 1] >> 31 : 0u);
    if constexpr (SB == 32) {
      T = m ^ ((m << 1) | before);
    } else {
      const uint32_t seg = (m >> sh) & ((1u << SB) - 1);
      T = (seg ^ ((seg << 1) | before)) & ((1u << SB) - 1);
    }
    const uint32_t rem = q.Lw - p0;
    if (rem < SB) T &= (1u << rem) - 1;
  }
  const uint32_t tc = (uint32_t)__builtin_popcount(T);
  // One scan for both counts: the word's nonzeros in the low half, the
  // lane's boundaries in the high half (each totals at most E < 2^16, so the
  // halves never carry).  It gives the window's nonzeros and, for the value
  // placement, the nonzeros before every word; the window's runs and the
  // boundaries before this lane.
  static_assert(S::E < (1 << 16), "16-bit count fields");
  const uint32_t x = c | (tc << 16);
  const uint32_t inc = wave_incl_scan(x);
  const uint32_t ex = inc - x, tot = read_lane(inc, 63);
  if (lane < S::WPW) L.pre[b][wave * S::WPW + lane] = ex & 0xFFFFu;
  const uint32_t v_w = tot & 0xFFFFu;
  q.T = T;
  q.texcl = ex >> 16;
  q.r_w = q.Lw ? 1 + (tot >> 16) : 0u;
  q.p_w = ESZ == 4 ? q.r_w + (q.r_w & 1) : q.r_w;
  if (lane == 0) L.pv[wave] = q.Lw ? q.p_w | (v_w << 16) : 0u;
}

// Write the window's block (run lengths, then its nonzeros in index order)
// into the stage buffer st at the window's place in its tile (data waves).
template <int ESZ>
__device__ __forceinline__ void rle_c_compact(uint8_t* __restrict__ st, const uint32_t* __restrict__ wm,
                                              const uint32_t* __restrict__ wp, const u32x4 (&v)[RleCShape<ESZ>::V],
                                              const RleLane& q, int lane) {
  using S = RleCShape<ESZ>;
  constexpr uint32_t SB = (uint32_t)S::E / 64;
  const uint32_t p0 = SB * (uint32_t)lane;
  uint8_t* blk = st + 2 * q.Pb + ESZ * q.Vb;
  // run lengths: the gap from the previous boundary (0 at the window start)
  const uint32_t lastpos = q.T ? p0 + 31 - (uint32_t)__builtin_clz(q.T) : 0u;
  const uint32_t imax = wave_incl_max(lastpos);
  const uint32_t before = __shfl_up(imax, 1, 64);
  uint32_t prev = lane ? before : 0u;
  const uint32_t tau_last = read_lane(imax, 63);
  uint32_t x = q.T, k = q.texcl;
  while (x) {
    const uint32_t bt = (uint32_t)__builtin_ctz(x);
    x &= x - 1;
    const uint32_t pos = p0 + bt;
    lds_u16(blk, 2 * k, pos - prev);
    prev = pos;
    ++k;
  }
  if (lane == 0) {
    lds_u16(blk, 2 * (q.r_w - 1), q.Lw - tau_last);
    if (q.p_w > q.r_w) lds_u16(blk, 2 * q.r_w, 0);
  }
  // values follow the runs: a lane's first value of vector j comes after the
  // nonzeros before its mask word and those below its bits there.  A window
  // without run boundaries holds no nonzero: its per-element tests are skipped.
  if (!__ballot(q.T != 0)) return;
#pragma unroll
  for (int j = 0; j < S::V; ++j) {
    const uint32_t c = (uint32_t)(j * 64 + lane);
    const uint32_t mw = wm[c / S::LPW];
    const uint32_t sh = (c % S::LPW) * S::EPL;
    const uint32_t bits = (mw >> sh) & ((1u << S::EPL) - 1);
    uint32_t pos = 2 * q.p_w + ESZ * (wp[c / S::LPW] + (uint32_t)__builtin_popcount(mw & ((1u << sh) - 1)));
#pragma unroll
    for (int k2 = 0; k2 < S::EPL; ++k2) {
      if ((bits >> k2) & 1u) {
        store_elem<ESZ>(blk + pos, vec_elem<ESZ>(v[j], k2));
        pos += ESZ;
      }
    }
  }
}

// Per-iteration state of the control wave.
struct RleCtl {
  ChainRound cr;      // first round of the pending chain sum (issued last iteration)
  uint64_t chain_lo;  // first tile of that sum
  uint64_t pfx;       // packed inclusive prefix of the last tile resolved
  uint32_t pend;      // raw counter value of the ticket to hand over next
};

// One iteration of the two-deep pipeline (the ZVC compressor's structure):
// t is classified (its loads were issued last iteration into cur), tp1 is
// compacted into stage[b ^ 1] from prev, whose registers then take the loads
// of tl, and tp2 is stored from stage[b].  The control wave finishes tp2's
// chain sum in phase X; in phase Y it hands over the next tile, publishes t's
// aggregate and issues the first round of tp1's chain sum.  q: lane state of
// t (written); qp: of tp1 (read); P2b / V2b: the window bases of tp2 (read,
// then set to tp1's).  Returns the tile the data waves load next iteration,
// with the workgroup synchronised.
template <int ESZ, int OP>
__device__ __forceinline__ uint32_t rle_c_iteration(RleCLds<ESZ>& L, u32x4 (&cur)[RleCShape<ESZ>::V],
                                                    u32x4 (&prev)[RleCShape<ESZ>::V], RleLane& q, const RleLane& qp,
                                                    uint32_t& P2b, uint32_t& V2b, RleCtl& C, uint32_t t, uint32_t tp1,
                                                    uint32_t tp2, uint32_t tl, int b, uint32_t full, uint64_t Wr,
                                                    const uint8_t* __restrict__ src, uint64_t n,
                                                    uint8_t* __restrict__ dst, uint64_t* __restrict__ out_bytes,
                                                    uint32_t* __restrict__ aggw, const Tickets& tk,
                                                    uint32_t num_tiles, uint8_t* __restrict__ act, int tid,
                                                    int wave, int lane) {
  using S = RleCShape<ESZ>;
  const bool have_t = t < num_tiles;
  const bool have_p1 = tp1 < num_tiles;
  const bool have_p2 = tp2 < num_tiles;
  const bool data = wave < S::NW;
  const uint64_t H = 8 * (Wr + 1);

  // ---- phase X ----
  if (data && have_p1 && qp.Lw)
    rle_c_compact<ESZ>(L.stage[b ^ 1], L.mask[b ^ 1] + wave * S::WPW, L.pre[b ^ 1] + wave * S::WPW, prev, qp, lane);
  {
    const bool load = __builtin_amdgcn_readfirstlane(wave) < S::NW && tl < full;
    rle_c_load_full<ESZ>(prev, src, tl, load, wave, lane);
  }
  if (data) {
    if (have_t) rle_c_classify<ESZ, OP>(L, cur, q, b, t, full, Wr, src, n, act, wave, lane);
  } else if (have_p2) {
    bool stuck = false;
    const uint64_t X = C.pfx + chain_sum(aggw, C.chain_lo, tp2, C.cr, &stuck, RleAggDec());
    const uint64_t a2 = L.agg[b];  // tp2 was classified two iterations ago
    if (lane == 0) {
      L.excl = X;
      L.agg2 = a2;
      if (stuck) atomicMax(reinterpret_cast<unsigned long long*>(out_bytes), kSizeInternalError);
    }
    C.pfx = X + a2;  // tp2's inclusive prefix
  }
  __syncthreads();

  // ---- phase Y ----
  if (data) {
    if (have_t) {  // t's window bases inside its tile: one scan of the packed counts
      const uint32_t x = lane < S::NW ? L.pv[lane] : 0u;
      const uint32_t ex = read_lane(wave_incl_scan(x) - x, wave);
      q.Pb = ex & 0xFFFFu;
      q.Vb = ex >> 16;
    }
    if (have_p2) {
      const uint64_t a2 = L.agg2;
      const uint32_t P = (uint32_t)(a2 >> 31), Vs = (uint32_t)(a2 & kLow31);
      const uint64_t RX = L.excl >> 31, VX = L.excl & kLow31;
      const uint64_t O = H + 2 * RX + (uint64_t)ESZ * VX;  // first byte of the tile's blocks
      const uint32_t span = 2 * P + ESZ * Vs;
      store_staged<2, S::NW * 64>(L.stage[b], span, O, dst, tid);
      const uint64_t w = (uint64_t)tp2 * S::NW + wave;
      if (lane == 0 && w < Wr) {
        reinterpret_cast<uint32_t*>(dst)[w] = (uint32_t)(RX + P2b);
        reinterpret_cast<uint32_t*>(dst + 4 * (Wr + 1))[w] = (uint32_t)(VX + V2b);
      }
      if (tp2 == num_tiles - 1 && tid == 0) {
        reinterpret_cast<uint32_t*>(dst)[Wr] = (uint32_t)(RX + P);
        reinterpret_cast<uint32_t*>(dst + 4 * (Wr + 1))[Wr] = (uint32_t)(VX + Vs);
        atomicMax(reinterpret_cast<unsigned long long*>(out_bytes), O + span);
      }
    }
  } else {
    // control wave: what it issued last iteration (chain round, ticket) must
    // be back before the hand-over; waiting here on every path keeps the
    // compiler from waiting again after the ticket drawn next
    __builtin_amdgcn_s_waitcnt(0);
    if (lane == 0) L.next = tk.tile(C.pend);
    // the next ticket goes out now and has a whole iteration to come back
    if (lane == 0 && have_t) C.pend = tk.raw();
    if (have_t) {
      const uint32_t tot = read_lane(wave_incl_scan(lane < S::NW ? L.pv[lane] : 0u), 63);
      const uint32_t P = tot & 0xFFFFu, Vs = tot >> 16;
      if (lane == 0) {
        L.agg[b] = ((uint64_t)P << 31) | Vs;
        agg_publish(aggw, t, (P << 15) | Vs);
      }
    }
    if (have_p1) {
      // tp1's chain sum: the tiles between this workgroup's tile before it
      // (tp2) and tp1; summed at the start of the next iteration
      C.chain_lo = have_p2 ? (uint64_t)tp2 + 1 : 0;
      chain_issue(aggw, C.chain_lo, tp1, C.cr);
    }
  }
  P2b = qp.Pb;
  V2b = qp.Vb;
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(L.next);  // uniform: keeps tile bases in SGPRs
}

// OP / act: the epilogue and its optional dense output, as for zvc_compress_kernel.
template <int ESZ, int OP>
__global__ __launch_bounds__(RleCShape<ESZ>::BLOCK) void rle_compress_kernel(
    const uint8_t* __restrict__ src, uint64_t n, uint8_t* __restrict__ dst,
    uint64_t* __restrict__ out_bytes, uint32_t* __restrict__ counter,
    uint32_t* __restrict__ aggw, uint32_t num_tiles, uint8_t* __restrict__ act) {
  using S = RleCShape<ESZ>;
  __shared__ RleCLds<ESZ> L;
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
  uint32_t t = tk.tile(lo);                  // classified this iteration
  uint32_t tl = tk.tile(a + b + c - lo - hi);  // loaded this iteration
  uint32_t tp1 = num_tiles, tp2 = num_tiles;   // compacted / stored this iteration (none yet)
  RleCtl C;                                    // control wave
  C.chain_lo = 0;
  C.pfx = 0;
  C.pend = hi;
  RleLane qa, qb;
  qa.Lw = qb.Lw = 0;
  qa.Pb = qa.Vb = qb.Pb = qb.Vb = 0;
  uint32_t P2b = 0, V2b = 0;
  u32x4 ra[S::V], rb[S::V];
  rle_c_load_full<ESZ>(ra, src, t, __builtin_amdgcn_readfirstlane(wave) < S::NW && t < full, wave, lane);
  // Two iterations per trip so the register sets swap roles without copies,
  // and one exit after the second (see the ZVC compressor).
  for (;;) {
    uint32_t r = rle_c_iteration<ESZ, OP>(L, ra, rb, qa, qb, P2b, V2b, C, t, tp1, tp2, tl, 0, full, Wr, src, n, dst,
                                          out_bytes, aggw, tk, num_tiles, act, tid, wave, lane);
    tp2 = tp1;
    tp1 = t;
    t = tl;
    tl = r;
    r = rle_c_iteration<ESZ, OP>(L, rb, ra, qb, qa, P2b, V2b, C, t, tp1, tp2, tl, 1, full, Wr, src, n, dst,
                                 out_bytes, aggw, tk, num_tiles, act, tid, wave, lane);
    tp2 = tp1;
    tp1 = t;
    t = tl;
    tl = r;
    if (t >= num_tiles && tp1 >= num_tiles && tp2 >= num_tiles) break;
  }
}

// ---------------------------------------------------------------------------
// decompress
// ---------------------------------------------------------------------------

// Stage pieces [0, nfull) of a block (16 bytes each, piece i of lane i % 64)
// into LDS: every load goes out before the first LDS write, so the block
// costs one memory round trip.  K = load rounds per lane (64 * (K - 1) <
// nfull <= 64 * K): the rounds before the last are whole, only the last one
// has lanes past nfull, which stay idle.
template <int K>
__device__ __forceinline__ void stage_rounds(uint8_t* blk, const u32x4* __restrict__ g, uint32_t nfull,
                                             uint32_t lane) {
  u32x4 q[K];
#pragma unroll
  for (int j = 0; j < K - 1; ++j) q[j] = ld_stream(g + lane + 64 * j);
  const uint32_t il = lane + 64 * (K - 1);
  if (il < nfull) q[K - 1] = ld_stream(g + il);
#pragma unroll
  for (int j = 0; j < K - 1; ++j) *reinterpret_cast<u32x4*>(blk + 16 * (lane + 64 * j)) = q[j];
  if (il < nfull) *reinterpret_cast<u32x4*>(blk + 16 * il) = q[K - 1];
}

// The same for any nfull up to 64 * KMAX pieces (uniform across the wave).
template <int KMAX>
__device__ __forceinline__ void stage_pieces(uint8_t* blk, const u32x4* __restrict__ g, uint32_t nfull,
                                             uint32_t lane) {
  static_assert(KMAX >= 1 && KMAX <= 8, "rounds per lane");
  switch ((nfull + 63) / 64) {
    case 0: break;
    case 1: stage_rounds<1>(blk, g, nfull, lane); break;
    case 2: stage_rounds<2>(blk, g, nfull, lane); break;
    case 3: stage_rounds<3>(blk, g, nfull, lane); break;
    case 4: stage_rounds<4>(blk, g, nfull, lane); break;
    case 5: if constexpr (KMAX >= 5) stage_rounds<5>(blk, g, nfull, lane); break;
    case 6: if constexpr (KMAX >= 6) stage_rounds<6>(blk, g, nfull, lane); break;
    case 7: if constexpr (KMAX >= 7) stage_rounds<7>(blk, g, nfull, lane); break;
    default: if constexpr (KMAX >= 8) stage_rounds<8>(blk, g, nfull, lane); break;
  }
}

// Stage stream bytes [beg, end) into blk from the 16-byte piece that holds
// beg, so that byte beg lands at blk + (beg & 15); bytes at or past eff read
// as 0.  Returns beg & 15.
template <int KMAX>
__device__ __forceinline__ uint32_t stage_span(uint8_t* blk, const uint8_t* __restrict__ src, uint64_t eff,
                                               uint64_t beg, uint64_t end, uint32_t lane) {
  const uint32_t shift = (uint32_t)(beg & 15);
  const uint64_t base = beg - shift;                          // 16-byte aligned
  const uint32_t nq = (uint32_t)((end - base + 15) >> 4);     // 16-byte pieces to stage
  const uint64_t whole = eff > base ? (eff - base) >> 4 : 0;  // pieces that end by eff
  const uint32_t nfull = whole < nq ? (uint32_t)whole : nq;
  stage_pieces<KMAX>(blk, reinterpret_cast<const u32x4*>(src + base), nfull, lane);
  for (uint32_t i = nfull + lane; i < nq; i += 64) {  // the readable stream ends inside the span
    const uint64_t qb = base + 16 * (uint64_t)i;
    for (int k = 0; k < 16; k += 2) {
      const uint64_t b = qb + k;
      uint32_t e = 0;
      if (b + 2 <= eff) e = *reinterpret_cast<const uint16_t*>(src + b);
      else if (b < eff) e = src[b];  // the last readable byte; the one after it reads as 0
      lds_u16(blk, 16 * i + k, e);
    }
  }
  return shift;
}

// Read a little-endian u32 at stream byte off; bytes at or past eff read as 0.
__device__ __forceinline__ uint32_t stream_u32(const uint8_t* __restrict__ src, uint64_t eff, uint64_t off) {
  if (off + 4 <= eff && (off & 3) == 0) return *reinterpret_cast<const uint32_t*>(src + off);
  uint32_t v = 0;
  for (int b = 0; b < 4; ++b)
    if (off + b < eff) v |= (uint32_t)src[off + b] << (8 * b);
  return v;
}

// Waves (windows) per decoder workgroup.  The windows are independent; a
// workgroup keeps its LDS until its slowest window is done, but half as many
// workgroups start per byte.  Two per workgroup: 59.6 against 55.7 % of HBM
// peak at s = 0.99 (fp32, 4 GiB; fp16 56.6 against 53.2), within a point
// elsewhere except s = 1 (79.0 against 81.0); four: no better at s = 0.99 and
// 76.6 % at s = 1.
#ifndef CDMA_RLE_DEC_WAVES
#define CDMA_RLE_DEC_WAVES 2
#endif
constexpr int kRleDecWaves = CDMA_RLE_DEC_WAVES;
constexpr int kRleDecBlock = 64 * kRleDecWaves;

template <int ESZ>
__global__ __launch_bounds__(kRleDecBlock) void rle_decompress_kernel(
    const uint8_t* __restrict__ src, uint64_t src_capacity, const uint64_t* __restrict__ src_bytes,
    uint64_t n, uint8_t* __restrict__ dst, uint32_t* __restrict__ error, uint32_t num_tiles) {
  using S = RleShape<ESZ>;
  constexpr int V = S::V;
  // largest number of u32 run-entry pairs per lane (32-bit elements: at most
  // E + 2 entries)
  constexpr int kMaxPer = ((S::E + 2) / 2 + 63) / 64;
  __shared__ uint32_t s_err;
  // per mask word of each wave's window: .x the boundary bitmap, then the
  // nonzero bitmap; .y the window's nonzeros before that word
  __shared__ uint2 s_map[kRleDecWaves * S::WPW];
  __shared__ __attribute__((aligned(16))) uint8_t s_blk[kRleDecWaves][S::WSTAGE];

  const int tid = threadIdx.x;
  const int lane = (int)lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: window math stays scalar
  const uint32_t t = xcd_tile(blockIdx.x, gridDim.x);  // this workgroup's tile
  uint2* map = s_map + wave * S::WPW;
  if (tid == 0) s_err = 0;
  for (int i = lane; i < S::WPW; i += 64) map[i].x = 0;  // this wave's part only
  const uint64_t claimed = src_bytes ? *src_bytes : src_capacity;
  const uint64_t eff = claimed < src_capacity ? claimed : src_capacity;
  const uint64_t Wr = (n + S::E - 1) / S::E;
  const uint64_t H = 8 * (Wr + 1);
  const uint64_t gw = (uint64_t)t * kRleDecWaves + wave;
  const uint64_t e_win = gw * S::E;
  const uint32_t Lw = gw < Wr ? (uint32_t)(n - e_win < (uint64_t)S::E ? n - e_win : S::E) : 0;
  uint32_t err = 0;
  if (t == 0 && tid == 0 && (stream_u32(src, eff, 0) | stream_u32(src, eff, 4 * (Wr + 1))))
    err |= CDMA_E_INDEX;
  // E_SIZE with a size word: the index totals describe another size, or the
  // size exceeds the readable capacity (bytes past the end read as 0)
  if (t == num_tiles - 1 && tid == 0 && src_bytes) {
    const uint64_t rt = stream_u32(src, eff, 4 * Wr), vt = stream_u32(src, eff, 4 * (Wr + 1) + 4 * Wr);
    if (H + 2 * rt + (uint64_t)ESZ * vt != *src_bytes || *src_bytes > src_capacity) err |= CDMA_E_SIZE;
  }
  __syncthreads();

  // this wave's block: lanes 0-3 read run_off[gw], run_off[gw+1], val_off[gw]
  // and val_off[gw+1]
  bool valid = false;
  uint32_t p = 0, nv = 0, nvb = 0, nvs = 0;
  uint64_t B = 0;
  if (Lw) {
    uint32_t iw = 0;
    if (lane < 4) iw = stream_u32(src, eff, 4 * ((uint64_t)(lane >> 1) * (Wr + 1) + gw + (lane & 1)));
    const uint32_t r0 = read_lane(iw, 0), r1 = read_lane(iw, 1);
    const uint32_t v0 = read_lane(iw, 2), v1 = read_lane(iw, 3);
    if (r1 < r0 || v1 < v0) {
      err |= CDMA_E_INDEX;
    } else {
      p = r1 - r0;
      nv = v1 - v0;
      if (p == 0 || p > Lw + 2) {
        err |= CDMA_E_RUN_FORM;
      } else {
        valid = true;
        // The block's values are the first min(nv, Lw, (BLKMAX - 2p) / ESZ):
        // a block that passes every check is at most BLKMAX bytes, so a
        // longer one is corrupt and reported through the checks, which read
        // run entries only; its output is unspecified anyway.  Every run
        // entry is staged (2p <= 2E + 4 < WSTAGE - 32) and as many of the
        // values as fit in WSTAGE - 32 bytes; the rest are read from memory.
        const uint32_t room = ((uint32_t)S::BLKMAX - 2 * p) / ESZ;
        nvb = nv < Lw ? nv : Lw;
        nvb = nvb < room ? nvb : room;
        const uint32_t sroom = ((uint32_t)S::WSTAGE - 32 - 2 * p) / ESZ;
        nvs = ESZ == 4 || nvb < sroom ? nvb : sroom;
        B = H + 2 * (uint64_t)r0 + (uint64_t)ESZ * v0;
        // no size word: the block runs past the readable capacity
        if (!src_bytes && B + 2 * (uint64_t)p + (uint64_t)ESZ * nvb > eff) err |= CDMA_E_SIZE;
      }
    }
  }
  uint8_t* blk = s_blk[wave];
  constexpr int KST = (S::WSTAGE + 1023) / 1024;  // pieces per lane at most: a span is < WSTAGE bytes
  uint32_t shift = 0;
  if (valid) shift = stage_span<KST>(blk, src, eff, B, B + 2 * (uint64_t)p + (uint64_t)ESZ * nvs, (uint32_t)lane);
  // each wave only touches its own block and its own part of the bitmap
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // A window whose index claims no values and whose run list is one zero run
  // of Lw elements (then the pad, for 32-bit elements) passes every check and
  // expands to zeros: it is written directly.
  bool zero_win = false;
  if (valid && nv == 0 && p == (ESZ == 4 ? 2u : 1u)) {
    const uint32_t e0 = __builtin_amdgcn_readfirstlane(*reinterpret_cast<const uint16_t*>(blk + shift));
    const uint32_t e1 =
        ESZ == 4 ? __builtin_amdgcn_readfirstlane(*reinterpret_cast<const uint16_t*>(blk + shift + 2)) : 0u;
    zero_win = e0 == Lw && e1 == 0;
  }

  // run starts -> boundary bitmap; checks
  if (valid && !zero_win) {
    auto entry = [&](uint32_t k) -> uint32_t { return *reinterpret_cast<const uint16_t*>(blk + shift + 2 * k); };
    auto toggle = [&](uint32_t pos) { atomicXor(&map[pos / 32].x, 1u << (pos % 32)); };
    uint32_t r = p;
    if (ESZ == 4) {
      if (p & 1) err |= CDMA_E_RUN_FORM;
      else if (entry(p - 1) == 0) r = p - 1;
    }
    uint32_t sum = 0, odd = 0, inc;
    bool zero_len = false;
    if (ESZ == 4 && !(p & 1) && !(shift & 3)) {
      // (zero run, nonzero run) pairs as aligned u32 words, each lane a
      // contiguous range of pairs held in registers; the pad, if any, is the
      // nonzero half of the last pair
      const uint32_t np = p / 2;
      const uint32_t per = __builtin_amdgcn_readfirstlane((np + 63) / 64);
      const uint32_t j0 = (uint32_t)lane * per < np ? (uint32_t)lane * per : np;
      const uint32_t j1 = j0 + per < np ? j0 + per : np;
      const uint32_t jpad = r < p ? np - 1 : ~0u;
      const uint32_t* pw = reinterpret_cast<const uint32_t*>(blk + shift);
      // words past j1 (at most per - 1 of them) still lie in the stage buffer
      // and are read, then ignored.  K bounds per at compile time: 1 (at most
      // 64 pairs, the sparse windows) or the largest a window can have.
      auto pairs = [&](auto kc) {
        constexpr int K = decltype(kc)::value;
        uint32_t w[K];
#pragma unroll
        for (int i = 0; i < K; ++i)
          if ((uint32_t)i < per) w[i] = pw[j0 + i];
        uint32_t bad = 0;
#pragma unroll
        for (int i = 0; i < K; ++i) {
          if ((uint32_t)i < per) {
            const uint32_t j = j0 + i;
            const uint32_t x = j < j1 ? w[i] : 0u;
            const uint32_t z = x & 0xFFFFu, nz = x >> 16;
            sum += z + nz;
            odd += nz;
            bad |= (uint32_t)(j < j1) & (((uint32_t)(z == 0) & (uint32_t)(j != 0)) |
                                         ((uint32_t)(nz == 0) & (uint32_t)(j != jpad)));
          }
        }
        zero_len = bad != 0;
        inc = wave_incl_scan(sum);
        uint32_t start = inc - sum;
#pragma unroll
        for (int i = 0; i < K; ++i) {
          if ((uint32_t)i < per) {
            const uint32_t j = j0 + i;
            const bool in = j < j1;
            const uint32_t z = w[i] & 0xFFFFu, nz = w[i] >> 16;
            if (in && j > 0 && start < Lw) toggle(start);
            const uint32_t s2 = start + z;
            if (in && j != jpad && s2 < Lw) toggle(s2);
            start = s2 + nz;
          }
        }
      };
      if (per == 1) pairs(std::integral_constant<int, 1>{});
      else pairs(std::integral_constant<int, kMaxPer>{});
    } else {
      // one u16 entry at a time, each lane a contiguous range of entries
      const uint32_t per = (r + 63) / 64;
      const uint32_t k0 = (uint32_t)lane * per < r ? (uint32_t)lane * per : r;
      const uint32_t k1 = k0 + per < r ? k0 + per : r;
      for (uint32_t k = k0; k < k1; ++k) {
        const uint32_t len = entry(k);
        sum += len;
        if (k & 1) odd += len;
        if (len == 0 && k != 0) zero_len = true;
      }
      inc = wave_incl_scan(sum);
      uint32_t start = inc - sum;
      for (uint32_t k = k0; k < k1; ++k) {
        if (k > 0 && start < Lw) toggle(start);
        start += entry(k);
      }
    }
    const uint32_t total = read_lane(inc, 63);
    const uint32_t odd_total = read_lane(wave_incl_scan(odd), 63);
    if (total != Lw) err |= CDMA_E_RUN_SUM;
    if (odd_total != nv) err |= CDMA_E_VAL_COUNT;
    if (__ballot(zero_len)) err |= CDMA_E_RUN_FORM;
  }
  // each wave only touches its own block and its own part of the bitmap
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // A 16-bit block longer than the stage: once the run entries are read, its
  // remaining values are staged from the start of the buffer.  They are
  // ESZ * (nvb - nvs) < E * ESZ - (WSTAGE - 32) + 2p + ESZ bytes, which with
  // their alignment end before the first staged value at shift + 2p.
  uint32_t tshift = 0;
  if constexpr (ESZ == 2) {
    static_assert(S::WSTAGE - 32 >= S::E * ESZ + 32, "the tail must end before the staged values");
    if (nvb > nvs) {
      const uint64_t tb = B + 2 * (uint64_t)p + (uint64_t)ESZ * nvs;
      tshift = stage_span<KST>(blk, src, eff, tb, tb + (uint64_t)ESZ * (nvb - nvs), (uint32_t)lane);
    }
  }
  // boundaries -> nonzero bitmap (prefix XOR across the window), and the
  // nonzeros before each mask word (wave prefix sum of its popcounts)
  if (!zero_win) {
    const uint32_t g = (uint32_t)lane;
    uint32_t x = 0;
    if (g < (uint32_t)S::WPW) x = map[g].x;
    const uint32_t pc = (uint32_t)__builtin_popcount(x) & 1u;
    const uint32_t par = wave_incl_scan(pc) - pc;
    x ^= x << 1;
    x ^= x << 2;
    x ^= x << 4;
    x ^= x << 8;
    x ^= x << 16;
    if (par & 1u) x = ~x;
    if (!valid || 32 * g >= Lw) x = 0;
    else if (Lw - 32 * g < 32) x &= (1u << (Lw - 32 * g)) - 1;
    const uint32_t c = (uint32_t)__builtin_popcount(x);
    const uint32_t before = wave_incl_scan(c) - c;
    if (g < (uint32_t)S::WPW) map[g] = make_uint2(x, before);
  }
  // each wave only touches its own block and its own part of the bitmap
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // expand: a lane's first value is the nonzeros before its mask word plus
  // those below its bits in the word
  const uint32_t vals = shift + 2 * p;
  const bool full = Lw == (uint32_t)S::E;
  if (zero_win) {
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const uint32_t c = (uint32_t)(j * 64 + lane);
      if (full) st_stream(reinterpret_cast<u32x4*>(dst + (e_win + (uint64_t)c * S::EPL) * ESZ), z);
      else store_vec<ESZ>(dst, e_win + (uint64_t)c * S::EPL, n, z);
    }
  } else {
    // tail: the window's values are in two staged pieces (uniform per wave)
    auto expand = [&](auto tail) {
#pragma unroll
      for (int j = 0; j < V; ++j) {
        const uint32_t c = (uint32_t)(j * 64 + lane);
        const uint2 m = map[c / S::LPW];
        const uint32_t sh = (c % S::LPW) * S::EPL;
        const uint32_t b = (m.x >> sh) & ((1u << S::EPL) - 1);
        uint32_t q = m.y + (uint32_t)__builtin_popcount(m.x & ((1u << sh) - 1));
        u32x4 o = {0u, 0u, 0u, 0u};
        if constexpr (decltype(tail)::value) {
#pragma unroll
          for (int k = 0; k < S::EPL; ++k) {
            if ((b >> k) & 1u) {
              const uint32_t a = q < nvs ? vals + ESZ * q : tshift + ESZ * (q - nvs);
              if (q < nvb) vec_set<ESZ>(o, k, load_elem<ESZ>(blk + a));
              ++q;
            }
          }
        } else {
          // Straight-line: every element reads the value its bit would take
          // and keeps it only if the bit is set.  In a window without an
          // error every set bit's value is staged (the bitmap holds nv
          // bits); otherwise the output is unspecified and the base is
          // clamped so that the reads stay in the stage.
          uint32_t off = vals + ESZ * q;
          off = off < (uint32_t)(S::WSTAGE - ESZ * S::EPL) ? off : (uint32_t)(S::WSTAGE - ESZ * S::EPL);
          const uint8_t* pv = blk + off;
#pragma unroll
          for (int k = 0; k < S::EPL; ++k) {
            const int32_t keep = __builtin_amdgcn_sbfe((int32_t)b, k, 1);  // 0 or -1
            vec_set<ESZ>(o, k, load_elem<ESZ>(pv) & (uint32_t)keep);
            pv -= ESZ * keep;
          }
        }
        if (full) st_stream(reinterpret_cast<u32x4*>(dst + (e_win + (uint64_t)c * S::EPL) * ESZ), o);
        else if (Lw) store_vec<ESZ>(dst, e_win + (uint64_t)c * S::EPL, n, o);
      }
    };
    if (ESZ == 2 && nvb > nvs) expand(std::true_type{});
    else expand(std::false_type{});
  }

  if (err) atomicOr(&s_err, err);
  __syncthreads();
  if (tid == 0 && s_err && error) atomicOr(error, s_err);
}

}  // namespace cdma
