// Fixed device scratch for g4attn_decode_noalloc: the split partials of a
// decode live in a file-scope device array instead of a caller workspace, so
// that the call allocates nothing (for callers that cannot allocate: code
// under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).
//
// Each GPU the library runs on holds its own copy of the array from the
// module load until the process ends.  Host code never passes the array's
// name to a kernel (in host code it is only a stand-in symbol): the device
// address is looked up once per device with hipGetSymbolAddress, with that
// device current, and that address is what the kernels receive.  Every call on
// one GPU shares its array, so calls that overlap on one GPU (different
// streams, different host threads) race on it; calls ordered on one stream
// do not.  The decode kernels write every partial they later read, so the
// array needs no clearing between calls.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.hpp"

namespace g4a {

static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

}  // namespace

hipError_t decode_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_ptr[dev] = g_err[dev] == hipSuccess ? p : nullptr;
  });
  if (g_err[dev] != hipSuccess) return g_err[dev];
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace g4a
