// Device scratch of muon_step_batched_noalloc: one file-scope array per GPU,
// allocated by the loader with the code object and held until the process
// ends.  The entry point lays its Newton-Schulz workspace and launch tables
// out inside it, so a call allocates no device memory.
//
// In host code `scratch` names a host-side stand-in, not the array's device
// address; noalloc_scratch takes the address of each GPU's copy once, with
// that GPU current, and every host use goes through that address.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "muon_internal.h"

static __device__ __align__(256) unsigned char scratch[muon::NOALLOC_SCRATCH_BYTES];

namespace muon {

namespace {
constexpr int MAX_SCRATCH_DEVICES = 64;
void* g_scratch_ptr[MAX_SCRATCH_DEVICES] = {};
}  // namespace

hipError_t noalloc_scratch(int dev, void** out) {
  if (dev < 0 || dev >= MAX_SCRATCH_DEVICES) return hipErrorInvalidDevice;
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev) return hipErrorInvalidDevice;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace muon
