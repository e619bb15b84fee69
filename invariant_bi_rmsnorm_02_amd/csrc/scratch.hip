// Device-resident scratch memory for bi_attn_decode_noalloc: the decode
// workspace (chunk records and work queue) in a fixed array that every GPU the
// library runs on holds from the moment the library's code is loaded on it
// until the process ends, so that call allocates nothing.
//
// `scratch` below is a host-side stand-in in host code, not a device address:
// its per-device address comes from hipGetSymbolAddress, called once per
// device with that device current, and only that address reaches kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "bi.h"
#include "launch.hpp"

static __device__ __align__(256) unsigned char scratch[BI_DECODE_SCRATCH_BYTES];

namespace bi {
namespace {

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // per device id, set once

}  // namespace

hipError_t decode_scratch(hipStream_t stream, void** ptr, size_t* bytes) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  hipDevice_t sdev = 0;
  e = hipStreamGetDevice(stream, &sdev);
  if (e != hipSuccess) return e;
  if (sdev != cur || cur < 0 || cur >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[cur]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[cur] = p;
  }
  *ptr = g_scratch_ptr[cur];
  *bytes = sizeof(scratch);
  return hipSuccess;
}

}  // namespace bi
