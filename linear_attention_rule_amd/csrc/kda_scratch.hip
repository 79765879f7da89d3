// Per-device host state: the fixed device scratch of kda_chunk_prefill_noalloc and the
// device properties the launchers query once per device.
//
// The scratch: the chunk records and segment
// states that kda_chunk_prefill keeps in a caller workspace live here instead, for
// callers that cannot allocate (code under stream capture, tight serving loops).
//
// The array is a file-scope device variable, so every GPU the library runs on holds
// its own copy (NOALLOC_SCRATCH_BYTES) from the first use on that device until the
// process ends.  In host code the array's name is only a host-side stand-in: its
// device address comes from hipGetSymbolAddress, taken once per device with that
// device current and kept in a per-device table.  Every call on one GPU shares that
// GPU's array; calls that overlap on one GPU race.
#include <mutex>

#include "kda_internal.h"

namespace kda {

namespace {

__device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES];   // device address of `scratch` per device (null: not yet)

}  // namespace

hipError_t noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t current_device_cus(int* cus) {
  static PerDeviceOnce once;
  return once.run(
      [](int dev, int* v) {
        return hipDeviceGetAttribute(v, hipDeviceAttributeMultiprocessorCount, dev);
      },
      cus);
}

}  // namespace kda
