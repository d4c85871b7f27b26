// Library-held device scratch for the decode entry point that allocates
// nothing (kvs_attn_decode_noalloc): the split-K partials of one call live in
// a file-scope device array instead of a caller workspace.  Every GPU the
// library runs on holds its own copy of the array, at its own address, until
// the process ends; calls on one GPU share it.
//
// In host code the array's name stands for a host-side shadow, not a device
// address, so it is never passed to a kernel or a copy: the device address
// comes from hipGetSymbolAddress, taken once per device with that device
// current, and kept per device.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"

namespace kvs {
namespace {

constexpr size_t kScratchBytes = size_t(16) << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

}  // namespace

size_t scratch_bytes() { return kScratchBytes; }

int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = p;
  });
  if (g_scratch_err[dev] != hipSuccess) return (int)g_scratch_err[dev];
  if (!g_scratch_ptr[dev]) return (int)hipErrorInvalidSymbol;
  *out = g_scratch_ptr[dev];
  return 0;
}

}  // namespace kvs
