// Device code of the in-place append, shared by the standalone append kernel
// and the attention kernel (which runs the append as extra workgroups of its
// grid when attention does not depend on the stored bytes).
//
// New token j of sequence b goes to logical position pos = Lc + j: page
// block_table[b][pos / S], slot pos % S.  With the [P, S, Hkv, D] cache layout
// all kv heads of one slot are contiguous, so each token is one contiguous row
// of Hkv * D elements for K and one for V.  ("Add
// flash_attn_varlen_func_with_kvcache", Usage: the cache is updated in place;
// Minor Changes: the cache length is passed per sequence and the new tokens
// carry their own cumulative offsets.)
//
// bf16 caches receive the bf16 bytes unchanged.  fp8 caches receive OCP
// e4m3fn codes of fp32(x) * fp32(1 / scale), rounded to nearest with ties to
// even, saturated to +-448, NaN kept with its sign (8-bit KV cache of the vLLM
// Triton FAv2 PR page's feature list, per-tensor scale).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../vpk_internal.h"
#include "rope_dev.h"

namespace vpk {
namespace append_detail {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Two bf16 values (low half first) -> two e4m3fn codes (low byte first) of
// fp32(x) * inv: nearest, ties to even, satfinite.  A NaN's code takes the
// sign of the unscaled input (1/scale > 0, so it is the product's sign for
// every other input, and it keeps a NaN's sign deterministic).
__device__ __forceinline__ uint32_t enc2(uint32_t two_bf16, float inv) {
  const float lo = __uint_as_float(two_bf16 << 16) * inv;
  const float hi = __uint_as_float(two_bf16 & 0xFFFF0000u) * inv;
  // magnitudes from 448 up (infinities included) saturate; the hardware
  // conversion rounds the rest to nearest, ties to even, subnormal codes
  // included, and keeps the sign of zero
  uint32_t w = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(
                   __builtin_amdgcn_fmed3f(lo, -448.0f, 448.0f), __builtin_amdgcn_fmed3f(hi, -448.0f, 448.0f), 0,
                   false)) & 0xFFFFu;
  // a NaN gives the NaN code with the input's sign
  if (__builtin_isnan(lo)) w = (w & 0xFF00u) | ((two_bf16 >> 8) & 0x80u) | 0x7Fu;
  if (__builtin_isnan(hi)) w = (w & 0x00FFu) | ((((two_bf16 >> 24) & 0x80u) | 0x7Fu) << 8);
  return w;
}

}  // namespace append_detail

// Store the new tokens of workgroup `wg` (tokens [wg * tokens_per_wg, ...) of
// the call) with `nthreads` threads of index `tid`.  First each token's
// destination row (page read from block_table at the index the plan carries,
// slot from the plan) goes to `dst` in LDS (tokens_per_wg entries, followed
// by as many int32 positions when the keys are turned by rotary embedding),
// then the threads copy 16-byte chunks, whose sources and destinations are
// then known up front.  A page id outside [0, num_pages) drops the token and
// raises bit 0 of the device error flag instead of writing out of bounds.
// With p.rope.dim > 0 each key chunk is turned at its token's position before
// it is stored (or quantised), so the cache holds the turned keys.
__device__ __forceinline__ void append_tokens(const AppendParams& p, int wg, int tid, int nthreads,
                                              int64_t* dst) {
  using namespace append_detail;
  const int t0 = wg * p.tokens_per_wg;
  const int nt = min(p.tokens_per_wg, p.total_knew - t0);
  const int chunks = p.row_elems / 8;   // 8 bf16 source elements per chunk
  const int per_tok = 2 * chunks;       // K chunks then V chunks
  const int total = nt * per_tok;
  // four chunks per thread at a time: their loads are issued together, then
  // they are encoded and stored
  constexpr int kBatch = 4;
  auto load_batch = [&](int f0, u32x4 (&x)[kBatch]) {
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int f = f0 + k * nthreads;
      if (f < total) {
        const int i = f / per_tok;
        const int c = f - i * per_tok;
        const bool is_v = c >= chunks;
        const int cc = is_v ? c - chunks : c;
        x[k] = *reinterpret_cast<const u32x4*>((is_v ? p.v_new : p.k_new) +
                                                 static_cast<int64_t>(t0 + i) * p.row_elems + cc * 8);
      }
    }
  };
  // the first batch's sources do not depend on the destinations: their loads
  // are issued before the destination lookups, so both round trips overlap
  u32x4 x[kBatch];
  load_batch(tid, x);
  int32_t* const tpos = reinterpret_cast<int32_t*>(dst + kAppendTokensMax);
  if (p.rope.dim > 0)
    for (int i = tid; i < nt; i += nthreads) tpos[i] = p.kpos[t0 + i];
  for (int i = tid; i < nt; i += nthreads) {
    // block_table index of the token's page id (inside its sequence's row:
    // the host checked the capacity) and the slot in that page
    const int entry = p.tok[2 * (t0 + i)];
    const int slot = p.tok[2 * (t0 + i) + 1];
    const int page = p.block_table[entry];
    if (page < 0 || page >= p.num_pages) {
      atomicOr(p.err_flag, 1);
      dst[i] = -1;
    } else {
      dst[i] = (static_cast<int64_t>(page) * p.page_size + slot) * p.row_elems;
    }
  }
  // fp8: the reciprocals of the scales (fp32 division, rounded once, as the
  // host computes them when the scales are passed by value)
  float k_inv = p.k_inv_scale, v_inv = p.v_inv_scale;
  if (p.fp8 && p.kv_scale_dev) {
    k_inv = 1.0f / p.kv_scale_dev[0];
    v_inv = 1.0f / p.kv_scale_dev[1];
  }
  __syncthreads();
  for (int f0 = tid; f0 < total; f0 += kBatch * nthreads) {
    if (f0 != tid) load_batch(f0, x);
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int f = f0 + k * nthreads;
      if (f >= total) continue;
      const int i = f / per_tok;
      const int c = f - i * per_tok;
      const int64_t dst_row = dst[i];
      if (dst_row < 0) continue;
      const bool is_v = c >= chunks;
      const int cc = is_v ? c - chunks : c;
      if (!is_v && p.rope.dim > 0) {
        // chunk cc of the token row = chunk cc % (D / 8) of head cc / (D / 8)
        const int hc = p.head_dim / 8;
        const int head = cc / hc;
        const uint16_t* hrow = p.k_new + static_cast<int64_t>(t0 + i) * p.row_elems + head * p.head_dim;
        x[k] = rope_chunk(p.rope, hrow, cc - head * hc, x[k], tpos[i]);
      }
      if (p.fp8) {
        const float inv = is_v ? v_inv : k_inv;
        uint8_t* d = static_cast<uint8_t*>(is_v ? p.v_cache : p.k_cache) + dst_row + cc * 8;
        u32x2 y;
        y[0] = enc2(x[k][0], inv) | (enc2(x[k][1], inv) << 16);
        y[1] = enc2(x[k][2], inv) | (enc2(x[k][3], inv) << 16);
        *reinterpret_cast<u32x2*>(d) = y;
      } else {
        uint16_t* d = static_cast<uint16_t*>(is_v ? p.v_cache : p.k_cache) + dst_row + cc * 8;
        *reinterpret_cast<u32x4*>(d) = x[k];
      }
    }
  }
}

}  // namespace vpk
