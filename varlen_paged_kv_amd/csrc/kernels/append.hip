// In-place append of new K/V tokens into the paged cache, gfx950: one
// workgroup per group of new tokens (the store rule and its sources are
// described in append_dev.h).  Used on its own by kv_cache_append, and before attention
// when attention must read the stored (fp8) bytes of the new tokens.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../vpk_internal.h"
#include "append_dev.h"

namespace vpk {
namespace {

__global__ __launch_bounds__(256) void append_kernel(const AppendParams p) {
  // destination rows, then (rotary embedding) the tokens' positions
  __shared__ int64_t dst[kAppendTokensMax + kAppendTokensMax / 2];
  append_tokens(p, blockIdx.x, threadIdx.x, blockDim.x, dst);
}

}  // namespace

int launch_append(const AppendParams& p, void* stream) {
  if (p.total_knew <= 0) return 0;
  if (p.tokens_per_wg < 1 || p.tokens_per_wg > kAppendTokensMax) return static_cast<int>(hipErrorInvalidValue);
  const int grid = (p.total_knew + p.tokens_per_wg - 1) / p.tokens_per_wg;
  hipLaunchKernelGGL(append_kernel, dim3(grid), dim3(256), 0,
                     static_cast<hipStream_t>(stream), p);
  return static_cast<int>(hipGetLastError());
}

}  // namespace vpk
