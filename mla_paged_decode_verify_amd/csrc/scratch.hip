// The static scratch array behind mla_verify_attn_merge_static: device memory
// that belongs to the library (a file-scope __device__ array, one copy per
// GPU, allocated when the code object is loaded and kept until the process
// ends), so that the entry point itself allocates nothing.
//
// In host code the array's name is only a host-side stand-in, not a device
// address. Its address on each device is looked up once, with that device
// current, through hipGetSymbolAddress, and only that address is ever passed
// to kernels.
#include <mutex>

#include "internal.h"

namespace mla {
namespace {

__device__ __align__(256) unsigned char scratch[MLA_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_addr[kMaxDevices] = {};

}  // namespace

hipError_t static_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_addr[dev] = p;
  }
  *ptr = g_addr[dev];
  return hipSuccess;
}

}  // namespace mla
