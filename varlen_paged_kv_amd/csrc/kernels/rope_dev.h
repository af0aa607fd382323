// Device code of the rotary embedding, shared by the rotation kernel, the
// attention kernels (query rows turned as they are loaded) and the append
// (new key rows turned as they are stored).
//
// The rotation is the one of "RoFormer: Enhanced Transformer with Rotary
// Position Embedding" (Su et al., section 3.4): coordinates are taken in pairs
// (a, b) and pair i of a row at position m is turned by the angle m * theta_i,
// whose cosine and sine the caller supplies as tables [max_positions,
// rotary_dim / 2] (float32):  a' = a cos - b sin,  b' = a sin + b cos.
// Pairing: half-split (coordinate i with i + rotary_dim / 2) or interleaved
// (2i with 2i + 1); coordinates at or past rotary_dim are unchanged.  The
// TransformerEngine KV-cache page ("Add KV cache for paged/non-paged
// attention", Description) names RoPE for inference as the step that comes
// with the cache path.
//
// Arithmetic (the turned rows are bf16 codes, so it is fixed): each product
// rounded to float32, their difference or sum rounded to float32 (no fused
// multiply-add), then round to nearest even to bf16.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../vpk_internal.h"

namespace vpk {
namespace rope_detail {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// float32 -> bf16, round to nearest with ties to even, a NaN quieted with its
// sign and top payload bits kept ((bits >> 16) | 0x40).  gfx950's conversion
// instruction (v_cvt_pk_bf16_f32, two values per instruction) does exactly
// this: an in-bounds probe on MI355X compared it with that rule on every NaN
// payload class, every tie and 2^20 random patterns, without a difference.
__device__ __forceinline__ uint16_t bf16_rne(float f) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f)); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// a' = a c - b s, b' = a s + b c with every operation rounded on its own
__device__ __forceinline__ void turn(float a, float b, float c, float s, uint16_t& ra, uint16_t& rb) {
#pragma clang fp contract(off)
  const float ac = a * c, bs = b * s, as = a * s, bc = b * c;
  ra = bf16_rne(ac - bs);
  rb = bf16_rne(as + bc);
}

// the first coordinate of a pair: a c - b s; the second: a s + b c
__device__ __forceinline__ uint16_t turn_first(float a, float b, float c, float s) {
#pragma clang fp contract(off)
  const float ac = a * c, bs = b * s;
  return bf16_rne(ac - bs);
}
__device__ __forceinline__ uint16_t turn_second(float a, float b, float c, float s) {
#pragma clang fp contract(off)
  const float as = a * s, bc = b * c;
  return bf16_rne(as + bc);
}

}  // namespace rope_detail

// Chunk c (coordinates 8c .. 8c + 7) of the bf16 head row `row` at position m,
// turned by `r`; `x` is that chunk as loaded.  Half-split pairs read the
// partner chunk from `row` (the same row, so the same cache lines) and 8
// angles; interleaved pairs sit in the chunk itself (4 angles).  Chunks at or
// past r.dim come back unchanged.
__device__ __forceinline__ rope_detail::u32x4 rope_chunk(const RopeArgs& r, const uint16_t* row, int c,
                                                         rope_detail::u32x4 x, int m) {
  using namespace rope_detail;
  const int d0 = c * 8;
  if (d0 >= r.dim) return x;
  const int half = r.dim >> 1;
  const float* cr = r.cos + static_cast<int64_t>(m) * half;
  const float* sr = r.sin + static_cast<int64_t>(m) * half;
  u32x4 y;
  if (r.interleaved) {
    const float4 cv = *reinterpret_cast<const float4*>(cr + (d0 >> 1));
    const float4 sv = *reinterpret_cast<const float4*>(sr + (d0 >> 1));
    const float cs[4] = {cv.x, cv.y, cv.z, cv.w}, sn[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint16_t ra, rb;
      turn(bf16_lo(x[q]), bf16_hi(x[q]), cs[q], sn[q], ra, rb);
      y[q] = ra | (static_cast<uint32_t>(rb) << 16);
    }
    return y;
  }
  const bool first = d0 < half;
  const int i0 = first ? d0 : d0 - half;
  const u32x4 pv = *reinterpret_cast<const u32x4*>(row + (first ? d0 + half : d0 - half));
  const float4 c0 = *reinterpret_cast<const float4*>(cr + i0);
  const float4 c1 = *reinterpret_cast<const float4*>(cr + i0 + 4);
  const float4 s0 = *reinterpret_cast<const float4*>(sr + i0);
  const float4 s1 = *reinterpret_cast<const float4*>(sr + i0 + 4);
  const float cs[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
  const float sn[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint16_t o[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float own = h ? bf16_hi(x[q]) : bf16_lo(x[q]);
      const float par = h ? bf16_hi(pv[q]) : bf16_lo(pv[q]);
      const int e = 2 * q + h;
      // own is the pair's first coordinate a (partner b) in the first half,
      // its second coordinate b (partner a) in the second half
      o[h] = first ? turn_first(own, par, cs[e], sn[e]) : turn_second(par, own, cs[e], sn[e]);
    }
    y[q] = o[0] | (static_cast<uint32_t>(o[1]) << 16);
  }
  return y;
}

}  // namespace vpk
