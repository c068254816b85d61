// The library's fixed device array for callers that cannot allocate (HIP
// graph capture, tight serving loops, harnesses that forbid allocation):
// logmel_stream_push_static keeps its streams' workspace rows and per-push
// offsets here instead of in memory a stream object allocates.
//
// Each GPU the library runs on holds its own copy of the array, at its own
// address, until the process ends. In host code the array's name is only a
// host-side stand-in: the device address comes from hipGetSymbolAddress,
// called once per device with that device current, and only that address
// is ever handed to kernels or copies.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "logmel_launch.h"

namespace {

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

// Device address of each device's copy (nullptr until first looked up).
void* g_scratch_ptr[kStaticMaxDevices] = {};

}  // namespace

// The calling thread's current device must be `device`.
hipError_t logmel_static_scratch(int device, void** ptr) {
  *ptr = nullptr;
  if (device < 0 || device >= kStaticMaxDevices) return hipErrorInvalidDevice;
  if (!g_scratch_ptr[device]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[device] = p;
  }
  *ptr = g_scratch_ptr[device];
  return hipSuccess;
}
