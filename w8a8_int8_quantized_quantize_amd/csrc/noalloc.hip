// Device scratch of the allocation-free fused linear (w8a8_linear_noalloc).
//
// The activation codes [M, K] and scales [M] that w8a8_linear keeps in a
// caller-provided workspace live here in a file-scope device array instead,
// for callers that cannot allocate device memory.  Each GPU the library runs
// on holds its own copy of the array (kNoAllocScratchBytes) until the process
// ends.  Host code never passes the array's name to a kernel or a copy: in
// host code that name is a host-side stand-in, not the device address.  The
// address is asked of the runtime (hipGetSymbolAddress) once per device, with
// that device current, on the first call there, and kept.
#include "internal.h"

#include <atomic>

namespace w8a8 {
namespace {

static __device__ __align__(256) int8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxScratchDevices];

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev].store(p, std::memory_order_release);  // racing first calls store the same address
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace w8a8
