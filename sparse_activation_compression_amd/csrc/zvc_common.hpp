// zvc_common.hpp -- stream format and shared device helpers of the gfx950
// zero-value codec (also used by the run-length variant).
//
// Format ("Compressing DMA Engine: Leveraging Activation Sparsity for Training
// Deep Neural Networks", §V.A Compression Algorithm): per window of 32
// consecutive elements a 32-bit mask (bit i = element i is nonzero), then the
// nonzero elements.  All W = ceil(n/32) masks come first, then all values in
// index order, so every mask sits at a fixed offset and a single prefix sum
// over nonzero counts places every value.
//
// Tiles: V 16-byte vectors per lane; vector j of wave w covers bytes
// [(w*V + j) * 1024, +1024) of the tile, so every global load and store
// instruction moves 1 KB of contiguous memory per wavefront.  A 32-element
// window spans LPW = 32/EPL lanes (8 for fp32, 4 for fp16), so its mask is an
// OR across a DPP lane group.
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

// Activation epilogue applied to every loaded vector before it is coded (the
// fused producer: the compressor reads the layer's pre-activation output and
// codes its ReLU).  ReLU is max(x, 0) on the raw pattern: a value whose sign
// bit is set and that is not a NaN (-0.0, negative denormals and normals,
// -inf) becomes +0; NaNs and everything else pass unchanged.  A NaN is an
// all-ones exponent with a nonzero mantissa, i.e. |bits| > the +inf pattern.
enum { kOpNone = 0, kOpReluF32 = 1, kOpReluF16 = 2, kOpReluBF16 = 3 };

__device__ __forceinline__ uint32_t relu16(uint32_t h, uint32_t inf) {
  return ((h & 0x8000u) && (h & 0x7FFFu) <= inf) ? 0u : h;
}

template <int OP>
__device__ __forceinline__ u32x4 apply_op(u32x4 v) {
  if constexpr (OP == kOpReluF32) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t w = v[k];
      v[k] = ((w >> 31) && (w & 0x7FFFFFFFu) <= 0x7F800000u) ? 0u : w;
    }
  } else if constexpr (OP == kOpReluF16 || OP == kOpReluBF16) {
    constexpr uint32_t inf = OP == kOpReluF16 ? 0x7C00u : 0x7F80u;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t w = v[k];
      v[k] = relu16(w & 0xFFFFu, inf) | (relu16(w >> 16, inf) << 16);
    }
  }
  return v;
}

// min(x, 1): 0 for 0, else 1.  Written as the instruction itself because the
// compiler turns the plain expression into a compare and a select (two
// instructions and a hazard wait).
__device__ __forceinline__ uint32_t nz01(uint32_t x) {
  uint32_t r;
  asm("v_min_u32 %0, 1, %1" : "=v"(r) : "v"(x));
  return r;
}

// min(x, 1) on each 16-bit half of x at once: 0 for a zero half, else 1, at
// bits 0 and 16.
__device__ __forceinline__ uint32_t pk_nz01(uint32_t x) {
  uint32_t r;
  asm("v_pk_min_u16 %0, %1, %2" : "=v"(r) : "v"(x), "s"(0x00010001u));
  return r;
}

// Per-element nonzero bits of one 16-byte vector (bit k = element k).  For
// 16-bit elements one packed min gives a word's two 0/1 tests at bits 0 and
// 16; the four words' results are interleaved into element order with three
// shift-ors and one fold of the high half down by 15 bits.
template <int ESZ>
__device__ __forceinline__ uint32_t vec_nz_bits(u32x4 v) {
  if constexpr (ESZ == 4) {
    return nz01(v.x) | (nz01(v.y) << 1) | (nz01(v.z) << 2) | (nz01(v.w) << 3);
  } else {
    const uint32_t a = pk_nz01(v.x) | (pk_nz01(v.y) << 2);  // bits 0, 2 and 16, 18
    const uint32_t b = pk_nz01(v.z) | (pk_nz01(v.w) << 2);
    const uint32_t c = a | (b << 4);  // low halves at even bits 0-6, high halves at 16-22
    return (c | (c >> 15)) & 0xFFu;
  }
}

// Per-element nonzero bits of one 16-byte vector placed at bit sh of a
// window mask (bit sh + k = element k), with min(x, 1) as the 0/1 test so
// each element costs one min and one shift-or.
template <int ESZ>
__device__ __forceinline__ uint32_t vec_nz_at(u32x4 v, uint32_t sh) {
  if constexpr (ESZ == 4) {
    return (nz01(v.x) << sh) | (nz01(v.y) << (sh + 1)) | (nz01(v.z) << (sh + 2)) | (nz01(v.w) << (sh + 3));
  } else {
    uint32_t r = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t w = v[k];
      r |= (nz01(w & 0xFFFFu) << (sh + 2 * k)) | (nz01(w >> 16) << (sh + 2 * k + 1));
    }
    return r;
  }
}

// Exclusive prefix over the wavefront's lanes of V per-lane counts at once:
// the counts are packed into fields of one 32-bit word (8 bits each when a
// lane's count is at most 4, 16 bits otherwise) and scanned together.  The
// exclusive prefixes fit their fields (at most 63 * 4 = 252, or 63 * 8), and
// the packed word is a plain sum of fields, so inclusive minus own count
// recovers them exactly even when lane 63's inclusive total carries over.
// Returns each row's exclusive prefix in ex[]; tot[] (lane 63 only) gets the
// row totals.
template <int EPL, int V>
__device__ __forceinline__ void packed_row_scan(const uint32_t (&cnt)[V], uint32_t (&ex)[V], uint32_t (&tot)[V]) {
  constexpr int F = EPL <= 4 ? 8 : 16;   // field width
  constexpr int PER = 32 / F;            // rows per scanned word
  static_assert(V % PER == 0, "rows must fill the packed words");
#pragma unroll
  for (int g = 0; g < V / PER; ++g) {
    uint32_t c = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) c |= cnt[g * PER + i] << (F * i);
    const uint32_t e = wave_incl_scan(c) - c;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int j = g * PER + i;
      ex[j] = __builtin_amdgcn_ubfe(e, F * i, F);
      tot[j] = ex[j] + cnt[j];
    }
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

}  // namespace cdma
