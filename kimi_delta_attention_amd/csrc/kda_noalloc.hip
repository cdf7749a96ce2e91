// kda_noalloc.hip -- the device scratch of kda_prefill_chunked_noalloc: the
// two-pass prefill's workspace kept in a file-scope device array, for callers
// that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc).
//
// Each device the library runs this entry point on holds its own copy of the
// array until the process ends.  Its address is looked up once per device
// (hipGetSymbolAddress, with that device current) and kept; host code never
// passes the array's name itself to a kernel (on the host it is only a
// stand-in for the symbol).  Every call on a device shares that device's copy,
// so calls that overlap on one device race; nothing in it has to start at zero
// (each call writes every part it reads: the chunk table, the carried state,
// the operand blocks of each window).
#include <hip/hip_runtime.h>

#include <mutex>

#include "kda_internal.h"

namespace kda {
namespace {

__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_ptr[dev] = g_err[dev] == hipSuccess ? p : nullptr;
  });
  *ptr = g_ptr[dev];
  return g_err[dev];
}

}  // namespace kda
