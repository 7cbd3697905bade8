// basa_select_static: basa_select whose two-pass scratch is a device array of
// this library instead of a caller-owned workspace, for callers that cannot
// allocate device memory (code under stream capture, tight serving loops).
//
// The array lives in every device's copy of the code object.  Its device
// address is looked up once per device (hipGetSymbolAddress with that device
// current) and kept; host code never passes the array's own name to a kernel.
#include <mutex>

#include "common.h"

namespace {

constexpr int64_t kScratchBytes = BASA_STATIC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, once found

// Device address of this device's `scratch` (looked up on the first call on
// the device, then cached).
hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

int basa_select_static(const basa_select_desc* d, const void* q, const void* k, int dtype,
                       int32_t* idx, void* stream) {
  try {
    if (!d) return BASA_E_NULLPTR;
    if (d->workspace || d->workspace_bytes) return BASA_E_UNSUPPORTED;
    const int64_t need = basa::select_workspace_bytes(d);
    if (need > kScratchBytes) return BASA_E_SHAPE;
    basa_select_desc with = *d;
    if (need > 0) {
      void* p = nullptr;
      if (scratch_address(&p) != hipSuccess) return BASA_E_LAUNCH;
      with.workspace = p;
      with.workspace_bytes = kScratchBytes;
    }
    return basa_select(&with, q, k, dtype, idx, stream);
  } catch (...) {
    return BASA_E_LAUNCH;
  }
}

}  // extern "C"
