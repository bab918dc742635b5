// Device scratch for the entry point that allocates nothing
// (treewy_prefill_chain_noalloc): the pseudo-value and gate buffers that pass
// from one chunk's launch to the next live in a file-scope device array
// instead of a caller workspace.
//
// Each GPU the library runs on holds its own copy of the array (kScratchBytes)
// from the first load of the library's code on that GPU until the process
// ends.  In host code the array's name is a host-side stand-in, not a device
// address, so the device address is taken once per device with
// hipGetSymbolAddress (that device current) and kept; only that address is
// handed to kernels.  Every call on one GPU shares the array: calls that
// overlap in time on one GPU race.
#include <mutex>

#include "treewy_internal.h"

namespace treewy {

static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t scratch_buffer(float** ptr, size_t* bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = static_cast<float*>(p);
  }
  *ptr = g_scratch_ptr[dev];
  *bytes = kScratchBytes;
  return hipSuccess;
}

}  // namespace treewy
