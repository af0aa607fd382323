// Rotary position embedding of rows into turned copies, gfx950 (the rotation
// and its arithmetic are described in rope_dev.h).  Used for the new key rows
// of a call without a cache, which attention reads straight from k_new; query
// rows are turned inside the attention kernels and the new keys of a cached
// call inside the append.
//
// The pass is HBM-bound and elementwise: a thread turns 16-byte chunks of
// output (8 coordinates of one head of one row); in the half-split form it
// also reads the partner chunk (same row, read by the same wave, so the same
// cache lines) and 8 angles; in the interleaved form its own chunk holds its
// 4 pairs.  Rows with a negative position are skipped (no sequence names
// them).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "../vpk_internal.h"
#include "rope_dev.h"

namespace vpk {
namespace {

using rope_detail::bf16_rne;
using rope_detail::turn;

__device__ __forceinline__ float bf16_f32(uint32_t half_word) { return __uint_as_float(half_word << 16); }

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

// Rows per workgroup: at most kRopeRowsMax, chosen so that each tensor gets
// about kRopeTargetWgs workgroups.
constexpr int kRopeRowsMax = 256;
constexpr int kRopeTargetWgs = 1024;

// Workgroup: `rows` consecutive rows of q (the first q_blocks workgroups) or of
// k_new.  Their positions are staged in LDS with one read (the position arrays
// may sit in host memory).  A head row splits into units: in the half-split
// form a unit is a chunk of the first half with its partner chunk (8 pairs,
// two chunks out), in the interleaved form one chunk (4 pairs); the chunks
// past rotary_dim are copy units.  The 256 threads walk the units of the
// block; a thread keeps the angles it read while its position and unit stay
// the same (the heads of a row share them).
template <int D>
__global__ __launch_bounds__(256) void rope_kernel(const RopeParams p, int q_rpw, int k_rpw, int q_blocks) {
  constexpr int CH = D / 8;                      // 16-byte chunks per head row
  __shared__ int32_t spos[kRopeRowsMax];
  const bool is_q = static_cast<int>(blockIdx.x) < q_blocks;
  const int blk = is_q ? blockIdx.x : blockIdx.x - q_blocks;
  const int rpw = is_q ? q_rpw : k_rpw;
  const int H = is_q ? p.hq : p.hkv;
  const int r0 = blk * rpw;
  const int nr = min(rpw, (is_q ? p.q_rows : p.k_rows) - r0);
  const int32_t* pos = is_q ? p.qpos : p.kpos;
  for (int i = threadIdx.x; i < nr; i += 256) spos[i] = pos[r0 + i];
  __syncthreads();
  const size_t base = static_cast<size_t>(r0) * H * D;
  const uint16_t* src = (is_q ? p.q : p.k) + base;
  uint16_t* dst = (is_q ? p.q_out : p.k_out) + base;
  const int rc = p.rot_dim / 8;                  // turned chunks per head row
  const int half = p.rot_dim / 2;
  const bool inter = p.interleaved != 0;
  const uint32_t U = inter ? CH : CH - rc / 2;   // units per head row
  const uint32_t row_units = static_cast<uint32_t>(H) * U;
  const uint32_t units = static_cast<uint32_t>(nr) * row_units;
  int64_t have = -1;                             // (position, unit) of the angles in cs / sn
  float cs[8], sn[8];
  for (uint32_t k = threadIdx.x; k < units; k += 256) {
    const uint32_t row = k / row_units;
    const uint32_t rem = k - row * row_units;
    const uint32_t hrow = row * H + rem / U;     // head row within the block
    const int u = static_cast<int>(rem % U);
    const int m = spos[row];
    if (m < 0) continue;
    const uint4* s4 = reinterpret_cast<const uint4*>(src + static_cast<size_t>(hrow) * D);
    uint4* d4 = reinterpret_cast<uint4*>(dst + static_cast<size_t>(hrow) * D);
    const int rot_units = inter ? rc : rc / 2;
    if (u >= rot_units) {
      const int c = inter ? u : u + rc / 2;
      d4[c] = s4[c];
      continue;
    }
    const int64_t want = static_cast<int64_t>(m) * CH + u;
    const float* cr = p.cos + static_cast<int64_t>(m) * half;
    const float* sr = p.sin + static_cast<int64_t>(m) * half;
    float x[8];
    uint16_t r[8];
    if (inter) {
      const uint4 v = s4[u];
      if (want != have) {
        const float4 cv = *reinterpret_cast<const float4*>(cr + 4 * u);
        const float4 sv = *reinterpret_cast<const float4*>(sr + 4 * u);
        cs[0] = cv.x, cs[1] = cv.y, cs[2] = cv.z, cs[3] = cv.w;
        sn[0] = sv.x, sn[1] = sv.y, sn[2] = sv.z, sn[3] = sv.w;
        have = want;
      }
      unpack8(v, x);
#pragma unroll
      for (int i = 0; i < 4; ++i) turn(x[2 * i], x[2 * i + 1], cs[i], sn[i], r[2 * i], r[2 * i + 1]);
      d4[u] = pack8(r);
    } else {
      // a = chunk u of the first half, b = its partner u + rotary_dim / 16
      const uint4 va = s4[u], vb = s4[u + rc / 2];
      if (want != have) {
        const float4 c0 = *reinterpret_cast<const float4*>(cr + 8 * u);
        const float4 c1 = *reinterpret_cast<const float4*>(cr + 8 * u + 4);
        const float4 s0 = *reinterpret_cast<const float4*>(sr + 8 * u);
        const float4 s1 = *reinterpret_cast<const float4*>(sr + 8 * u + 4);
        cs[0] = c0.x, cs[1] = c0.y, cs[2] = c0.z, cs[3] = c0.w, cs[4] = c1.x, cs[5] = c1.y, cs[6] = c1.z, cs[7] = c1.w;
        sn[0] = s0.x, sn[1] = s0.y, sn[2] = s0.z, sn[3] = s0.w, sn[4] = s1.x, sn[5] = s1.y, sn[6] = s1.z, sn[7] = s1.w;
        have = want;
      }
      float y[8];
      uint16_t rb[8];
      unpack8(va, x);
      unpack8(vb, y);
#pragma unroll
      for (int i = 0; i < 8; ++i) turn(x[i], y[i], cs[i], sn[i], r[i], rb[i]);
      d4[u] = pack8(r);
      d4[u + rc / 2] = pack8(rb);
    }
  }
}

}  // namespace

int launch_rope(const RopeParams& p, int head_dim, void* stream) {
  if (head_dim != 64 && head_dim != 128) return static_cast<int>(hipErrorInvalidValue);
  if (p.rot_dim < 16 || p.rot_dim > head_dim || p.rot_dim % 16 != 0) return static_cast<int>(hipErrorInvalidValue);
  if (p.q_rows < 0 || p.k_rows < 0) return static_cast<int>(hipErrorInvalidValue);
  auto rows_per_wg = [](int rows) { return std::min(kRopeRowsMax, std::max(1, (rows + kRopeTargetWgs - 1) / kRopeTargetWgs)); };
  const int q_rpw = rows_per_wg(p.q_rows), k_rpw = rows_per_wg(p.k_rows);
  const int q_blocks = (p.q_rows + q_rpw - 1) / q_rpw;
  const int k_blocks = (p.k_rows + k_rpw - 1) / k_rpw;
  if (q_blocks + k_blocks == 0) return 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(static_cast<uint32_t>(q_blocks + k_blocks));
  if (head_dim == 128)
    hipLaunchKernelGGL(rope_kernel<128>, grid, dim3(256), 0, s, p, q_rpw, k_rpw, q_blocks);
  else
    hipLaunchKernelGGL(rope_kernel<64>, grid, dim3(256), 0, s, p, q_rpw, k_rpw, q_blocks);
  return static_cast<int>(hipGetLastError());
}

}  // namespace vpk
