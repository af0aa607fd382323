// Device scratch of the allocation-free entry point (attn_varlen_paged_fwd_noalloc).
//
// One fixed array per device, in the library's code object: the loader places
// it when the library's kernels are loaded on a device, and it lives until the
// process ends.  Host code never passes the array's name to a kernel (in host
// code that name is a stand-in, not a device address): the device address of
// each device's copy is looked up once with hipGetSymbolAddress, with that
// device current, and every later use (kernel arguments, copies) takes that
// address.
#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

#include "../vpk_internal.h"

static __device__ __align__(256) char scratch[vpk::kScratchBytes];

namespace vpk {

int scratch_address(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return static_cast<int>(e);
  static std::mutex mu;
  static std::vector<void*> addr;
  std::lock_guard<std::mutex> lk(mu);
  if (static_cast<size_t>(dev) >= addr.size()) addr.resize(dev + 1, nullptr);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return static_cast<int>(e);
    if (!p) return static_cast<int>(hipErrorInvalidSymbol);
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return 0;
}

}  // namespace vpk
