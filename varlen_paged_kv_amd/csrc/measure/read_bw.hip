// Measurement helper, not part of the attention path: a streaming read of a
// contiguous device buffer, used by the benchmark to report the decode kernel
// against a read bandwidth measured on the same GPU in the same run.  Each
// thread reads U 16-byte vectors per trip of a grid-stride loop and folds them
// into one word, which it writes (so that no load is removed).  Every index
// stays below the buffer's vector count.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int U>
__global__ __launch_bounds__(256) void stream_read(const u32x4* __restrict__ p, size_t n, uint32_t* out) {
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (U - 1) * stride < n; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = p[i + u * stride];
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x + v[u].y + v[u].z + v[u].w;
  }
  for (; i < n; i += stride) {
    const u32x4 v = p[i];
    acc ^= v.x + v.y + v.z + v.w;
  }
  out[static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x] = acc;
}

}  // namespace

// Read `bytes` (a multiple of 16, 16-byte aligned) at `buf` once with `grid`
// workgroups of 256 threads and `unroll` (1, 4 or 8) loads in flight per
// thread; `out` must hold grid * 256 words.  Enqueued on `stream`; returns the
// hipError_t of the launch.
extern "C" int vpk_measure_stream_read(const void* buf, size_t bytes, int grid, int unroll, void* out,
                                       void* stream) {
  if (!buf || !out || grid <= 0 || bytes % 16 != 0) return static_cast<int>(hipErrorInvalidValue);
  const auto* p = static_cast<const u32x4*>(buf);
  const size_t n = bytes / 16;
  auto* o = static_cast<uint32_t*>(out);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (unroll == 1)
    hipLaunchKernelGGL(stream_read<1>, dim3(grid), dim3(256), 0, s, p, n, o);
  else if (unroll == 4)
    hipLaunchKernelGGL(stream_read<4>, dim3(grid), dim3(256), 0, s, p, n, o);
  else if (unroll == 8)
    hipLaunchKernelGGL(stream_read<8>, dim3(grid), dim3(256), 0, s, p, n, o);
  else
    return static_cast<int>(hipErrorInvalidValue);
  return static_cast<int>(hipGetLastError());
}
