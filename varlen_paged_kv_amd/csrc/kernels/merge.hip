// LSE merge of split key ranges, gfx950.
//
// A tile whose key range was cut into n parts left, per part s and row r, the
// part's normalised output O_s[r] (fp32) and its lse_s[r].  The full result is
//   lse = ln sum_s exp(lse_s),   out = sum_s exp(lse_s - lse) O_s,
// taken over the parts in index order (so repeated calls give identical bits).
// A row whose parts all saw no key gets out = 0 and lse = -inf.  This is the
// combine step of split-KV decoding that the flash-attention PR page's
// discussion asks for ("Add flash_attn_varlen_func_with_kvcache", Limitation
// and thread).
//
// One workgroup per split tile; each thread produces 4 consecutive outputs of
// one row, so the partial reads are 16-byte and coalesced along the head dim.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../vpk_internal.h"

namespace vpk {
namespace {

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

constexpr int kRegParts = 4;

__global__ __launch_bounds__(256) void merge_kernel(const MergeParams p) {
  const MergeGroup gr = p.groups[blockIdx.x];
  const SeqInfo sq = gr.s;
  const int D = p.head_dim;
  const int per_row = D / 4;
  const int total = gr.nrows * per_row;
  for (int idx = threadIdx.x; idx < total; idx += blockDim.x) {
    const int r = idx / per_row;
    const int c = idx - r * per_row;
    // the first kRegParts parts' lse and outputs are loaded together (one
    // memory round trip); further parts are read in a second pass
    float ls[kRegParts];
    float4 os[kRegParts];
#pragma unroll
    for (int s = 0; s < kRegParts; ++s) {
      if (s < gr.nsplit) {
        const int pr = gr.part + s * gr.nrows + r;
        ls[s] = p.part_lse[pr];
        os[s] = *reinterpret_cast<const float4*>(p.part_o + static_cast<int64_t>(pr) * D + c * 4);
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int s = 0; s < kRegParts; ++s)
      if (s < gr.nsplit) mx = fmaxf(mx, ls[s]);
    for (int s = kRegParts; s < gr.nsplit; ++s) mx = fmaxf(mx, p.part_lse[gr.part + s * gr.nrows + r]);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float lse_v = -INFINITY;
    if (mx != -INFINITY) {
      float wsum = 0.f;
#pragma unroll
      for (int s = 0; s < kRegParts; ++s) {
        if (s < gr.nsplit) {
          const float w = __expf(ls[s] - mx);
          wsum += w;
          acc.x += w * os[s].x;
          acc.y += w * os[s].y;
          acc.z += w * os[s].z;
          acc.w += w * os[s].w;
        }
      }
      for (int s = kRegParts; s < gr.nsplit; ++s) {
        const int pr = gr.part + s * gr.nrows + r;
        const float w = __expf(p.part_lse[pr] - mx);
        const float4 o = *reinterpret_cast<const float4*>(p.part_o + static_cast<int64_t>(pr) * D + c * 4);
        wsum += w;
        acc.x += w * o.x;
        acc.y += w * o.y;
        acc.z += w * o.z;
        acc.w += w * o.w;
      }
      const float inv = 1.f / wsum;
      acc.x *= inv;
      acc.y *= inv;
      acc.z *= inv;
      acc.w *= inv;
      lse_v = mx + __logf(wsum);
    }
    const int prow = gr.row0 + r;
    const int token = prow / p.g;
    const int qh = gr.kv_head * p.g + (prow - token * p.g);
    uint16_t* orow = p.out + (static_cast<int64_t>(sq.q_start + token) * p.hq + qh) * D + c * 4;
    uint2 w2;
    w2.x = f32_to_bf16_rne(acc.x) | (static_cast<uint32_t>(f32_to_bf16_rne(acc.y)) << 16);
    w2.y = f32_to_bf16_rne(acc.z) | (static_cast<uint32_t>(f32_to_bf16_rne(acc.w)) << 16);
    *reinterpret_cast<uint2*>(orow) = w2;
    if (c == 0 && p.lse) p.lse[static_cast<int64_t>(qh) * p.total_q + sq.q_start + token] = lse_v;
  }
}

}  // namespace

int launch_merge(const MergeParams& p, void* stream) {
  if (p.num_groups <= 0) return 0;
  hipLaunchKernelGGL(merge_kernel, dim3(p.num_groups), dim3(256), 0,
                     static_cast<hipStream_t>(stream), p);
  return static_cast<int>(hipGetLastError());
}

}  // namespace vpk
