// The library's one piece of device memory of its own: a fixed scratch array
// for the allocation-free entry point (muon_momentum_grouped_noalloc), which
// takes no workspace argument.  Each GPU the library runs on holds its own
// copy from the load of the code object until the process ends.
//
// In host code the array's name is a host-side stand-in, not a device
// address, so the address is looked up once per device with
// hipGetSymbolAddress (with that device current) and only that address is
// handed to kernels.

#include <mutex>

#include "../../include/muon355.h"
#include "muon_internal.h"

namespace muon {
namespace {

static __device__ __align__(256) unsigned char scratch[MUON_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

}  // namespace

hipError_t noalloc_scratch(void** ptr, size_t* bytes) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  *bytes = MUON_NOALLOC_SCRATCH_BYTES;
  return hipSuccess;
}

}  // namespace muon
