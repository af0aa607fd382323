// Rotary position embedding of the query rows and the new key rows, gfx950.
//
// The rotation is the one of "RoFormer: Enhanced Transformer with Rotary
// Position Embedding" (Su et al., section 3.4): coordinates are taken in pairs
// (a, b) and pair i of a row at position m is turned by the angle m * theta_i,
// whose cosine and sine the caller supplies as tables [max_positions,
// rotary_dim / 2] (float32).  Pairing: half-split (coordinate i with
// i + rotary_dim / 2) or interleaved (2i with 2i + 1).  Coordinates at or past
// rotary_dim are copied.  The TransformerEngine KV-cache page ("Add KV cache
// for paged/non-paged attention", Description) names RoPE for inference as the
// step that comes with the cache path.
//
// Arithmetic (the turned rows are bf16 codes, so it is fixed): each product
// rounded to float32, their difference or sum rounded to float32 (no fused
// multiply-add), then round to nearest even to bf16.
//
// The pass is HBM-bound and elementwise: one thread per 16-byte chunk of
// output (8 coordinates of one head of one row); in the half-split form a
// thread also reads its partner chunk (same row, same wave, so the same cache
// lines) and 8 angles; in the interleaved form its own chunk holds its 4
// pairs.  Rows with a negative position are skipped (no sequence names them).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../vpk_internal.h"

namespace vpk {
namespace {

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float bf16_f32(uint32_t half_word) { return __uint_as_float(half_word << 16); }

// a' = a c - b s, b' = a s + b c with every operation rounded on its own
__device__ __forceinline__ void turn(float a, float b, float c, float s, uint16_t& ra, uint16_t& rb) {
#pragma clang fp contract(off)
  const float ac = a * c, bs = b * s, as = a * s, bc = b * c;
  ra = bf16_rne(ac - bs);
  rb = bf16_rne(as + bc);
}

__device__ __forceinline__ void unpack8(const uint4 v, float* x) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16_f32(w[i] & 0xffffu);
    x[2 * i + 1] = bf16_f32(w[i] >> 16);
  }
}

__device__ __forceinline__ uint4 pack8(const uint16_t* r) {
  uint4 v;
  v.x = r[0] | (static_cast<uint32_t>(r[1]) << 16);
  v.y = r[2] | (static_cast<uint32_t>(r[3]) << 16);
  v.z = r[4] | (static_cast<uint32_t>(r[5]) << 16);
  v.w = r[6] | (static_cast<uint32_t>(r[7]) << 16);
  return v;
}

template <int D>
__global__ __launch_bounds__(256) void rope_kernel(const RopeParams p) {
  constexpr int CH = D / 8;                      // 16-byte chunks per head row
  const uint64_t chunk = static_cast<uint64_t>(blockIdx.x) * 256 + threadIdx.x;
  // (row, head) of q, then of k_new; each count is below 2^31 (checked by the host)
  const uint32_t job = static_cast<uint32_t>(chunk / CH);
  const int c = static_cast<int>(chunk % CH);
  const uint32_t q_jobs = static_cast<uint32_t>(p.q_rows) * static_cast<uint32_t>(p.hq);
  const uint16_t* src;
  uint16_t* dst;
  int32_t pos;
  if (job < q_jobs) {
    src = p.q + static_cast<size_t>(job) * D;
    dst = p.q_out + static_cast<size_t>(job) * D;
    pos = p.qpos[job / static_cast<uint32_t>(p.hq)];
  } else {
    const uint32_t kj = job - q_jobs;
    if (kj >= static_cast<uint32_t>(p.k_rows) * static_cast<uint32_t>(p.hkv)) return;
    src = p.k + static_cast<size_t>(kj) * D;
    dst = p.k_out + static_cast<size_t>(kj) * D;
    pos = p.kpos[kj / static_cast<uint32_t>(p.hkv)];
  }
  if (pos < 0) return;
  const uint4* s4 = reinterpret_cast<const uint4*>(src);
  uint4* d4 = reinterpret_cast<uint4*>(dst);
  const int R = p.rot_dim;
  const int half = R >> 1;
  const int e = c * 8;                           // first coordinate of this chunk
  if (e >= R) {
    d4[c] = s4[c];
    return;
  }
  const float* cr = p.cos + static_cast<int64_t>(pos) * half;
  const float* sr = p.sin + static_cast<int64_t>(pos) * half;
  float x[8];
  uint16_t r[8];
  if (p.interleaved) {
    unpack8(s4[c], x);
    const float4 cv = *reinterpret_cast<const float4*>(cr + e / 2);
    const float4 sv = *reinterpret_cast<const float4*>(sr + e / 2);
    const float cs[4] = {cv.x, cv.y, cv.z, cv.w}, sn[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) turn(x[2 * i], x[2 * i + 1], cs[i], sn[i], r[2 * i], r[2 * i + 1]);
  } else {
    // chunk in the first half: a = own, b = partner; in the second: a = partner, b = own
    const bool first = e < half;
    const int pair0 = first ? e : e - half;
    const int pc = first ? c + half / 8 : c - half / 8;
    float y[8];
    unpack8(s4[c], x);
    unpack8(s4[pc], y);
    const float4 c0 = *reinterpret_cast<const float4*>(cr + pair0);
    const float4 c1 = *reinterpret_cast<const float4*>(cr + pair0 + 4);
    const float4 s0 = *reinterpret_cast<const float4*>(sr + pair0);
    const float4 s1 = *reinterpret_cast<const float4*>(sr + pair0 + 4);
    const float cs[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
    const float sn[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint16_t ra, rb;
      if (first) {
        turn(x[i], y[i], cs[i], sn[i], ra, rb);
        r[i] = ra;
      } else {
        turn(y[i], x[i], cs[i], sn[i], ra, rb);
        r[i] = rb;
      }
    }
  }
  d4[c] = pack8(r);
}

}  // namespace

int launch_rope(const RopeParams& p, int head_dim, void* stream) {
  if (head_dim != 64 && head_dim != 128) return static_cast<int>(hipErrorInvalidValue);
  if (p.rot_dim < 16 || p.rot_dim > head_dim || p.rot_dim % 16 != 0) return static_cast<int>(hipErrorInvalidValue);
  const int64_t jobs = static_cast<int64_t>(p.q_rows) * p.hq + static_cast<int64_t>(p.k_rows) * p.hkv;
  const int64_t chunks = jobs * (head_dim / 8);
  if (chunks <= 0) return 0;
  const int64_t grid = (chunks + 255) / 256;
  if (grid > 0x7fffffff) return static_cast<int>(hipErrorInvalidValue);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (head_dim == 128)
    hipLaunchKernelGGL(rope_kernel<128>, dim3(static_cast<uint32_t>(grid)), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(rope_kernel<64>, dim3(static_cast<uint32_t>(grid)), dim3(256), 0, s, p);
  return static_cast<int>(hipGetLastError());
}

}  // namespace vpk
