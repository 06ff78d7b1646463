// Scratch memory of lowram_decode_attn_noalloc: a file-scope device array
// in place of the caller's workspace, for callers that cannot allocate.
//
// The array's name is only a host-side stand-in for it.  Its device address
// comes from hipGetSymbolAddress, taken once per device with that device
// current and kept per device (each GPU holds its own copy of the array from
// the first use until the process ends).  Host code passes only that
// address to kernels.  Every call on one GPU shares the array, so calls
// that overlap on one GPU (different streams, or another thread) race.
#include <mutex>

#include "lowram_internal.h"

namespace lowram {

constexpr size_t kNoAllocScratchBytes = size_t{64} << 20;

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];
}  // namespace

size_t noalloc_scratch_bytes() { return kNoAllocScratchBytes; }

hipError_t noalloc_scratch(void **ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace lowram
