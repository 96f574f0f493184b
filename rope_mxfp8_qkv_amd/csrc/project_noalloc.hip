// Static device scratch for the projection entry point that allocates nothing
// (qkv_rowmx_project_staged_noalloc).
//
// The projection's kernels need device memory beyond their inputs and outputs: the per-XCD
// tile counters of the persistent scheduler, the per-(token, 128-channel) sum-of-squares
// partials and, for calls with few output tiles, the split-contraction planes.  The ordinary
// entry points take that memory as a caller-provided workspace; this file instead holds it in
// one file-scope device array, so a caller that cannot allocate (code under graph capture, a
// serving loop that forbids hipMalloc) can still call the projection.
//
// Every GPU the library runs on holds its own copy of the array (allocated when the library's
// code object is loaded on that device) until the process ends.  Its device address is looked
// up once per device with hipGetSymbolAddress, with that device current, and kept; host code
// only ever passes that address to kernels (the array's own name is a host-side stand-in, not
// a device address).  All calls on one device share the array: calls that overlap on one GPU
// (concurrent streams) race on it.
#include <mutex>

#include "device_common.h"
#include "internal.h"

namespace qkvmx {

namespace {

constexpr int kMaxScratchDevices = 64;

__device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

}  // namespace

// Device address of the current device's scratch array (looked up on the first call per
// device).  Allocates nothing.
hipError_t noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
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

}  // namespace qkvmx
