// noalloc.hip -- the library-owned scratch buffer behind
// lin_attn_chunk_fwd_noalloc, for callers that cannot allocate device memory.
//
// The buffer is a file-scope device array, so each GPU the library runs on
// holds its own copy from module load until the process ends.  In host code
// the array's name is only a host-side stand-in: its device address is looked
// up once per device with hipGetSymbolAddress (with that device current) and
// that address is what the kernels receive.  Every call on one GPU shares the
// one buffer, so calls that overlap in time on the same GPU race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "la_launch.h"

namespace la {

static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];   // device address of `scratch` per device, once resolved
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace la
