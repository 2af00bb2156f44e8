// slay_noalloc.hip -- slay_attn_chunked_fwd for callers that cannot allocate
// device memory (code under stream capture, tight serving loops, hosts that
// forbid allocation).  The workspace is a fixed, library-owned device array;
// this entry point calls no allocating routine of any kind.
//
// `scratch` below is a file-scope __device__ array: every GPU the library runs
// on holds its own copy (SLAY_NOALLOC_SCRATCH_BYTES bytes) from the time the
// code object is loaded until the process ends.  In host code its name is only
// a host-side stand-in, never a device address: the device address is looked
// up once per device with hipGetSymbolAddress, with that device current, and
// only that address is handed to the kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "slay.h"
#include "slay_internal.hpp"

namespace {

static __device__ __align__(256) unsigned char scratch[SLAY_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` per device (nullptr: not looked up yet)

// Device address of `scratch` on the device of `stream` (the current device
// for the null stream), looked up once per device with that device current.
hipError_t scratch_address(hipStream_t stream, void** out) {
  int dev = 0;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev]) {
    *out = g_scratch[dev];
    return hipSuccess;
  }
  int cur = 0;
  if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
  if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
  void* p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (cur != dev) {
    const hipError_t e2 = hipSetDevice(cur);
    if (e == hipSuccess) e = e2;
  }
  if (e != hipSuccess) return e;
  if (!p) return hipErrorInvalidSymbol;
  g_scratch[dev] = p;
  *out = p;
  return hipSuccess;
}

}  // namespace

extern "C" slay_status_t slay_attn_chunked_fwd_noalloc(const slay_params_t* params, const void* q, const void* k,
                                                       const void* v, slay_dtype_t io_dtype, int32_t B, int32_t H,
                                                       int64_t L, int32_t dv, int32_t chunk, const float* S0,
                                                       const float* z0, void* o, float* S_out, float* z_out,
                                                       void* stream) {
  return slay::chunked_fwd_entry(params, q, k, v, io_dtype, B, H, L, dv, chunk, S0, z0, o, S_out, z_out, nullptr,
                                 (size_t)SLAY_NOALLOC_SCRATCH_BYTES, stream, scratch_address);
}
