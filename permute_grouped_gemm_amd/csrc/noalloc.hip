// Fixed device scratch for the allocation-free entry point (pgg_moe_dx_noalloc).
//
// The workspace of pgg_moe_dx -- header, index and tile tables, fp32 ring --
// lives here in a file-scope device array instead of caller memory.  Each GPU
// the library runs on holds its own copy until the process ends.  In host
// code `scratch` names a host-side stand-in, not device memory, so host code
// never passes it to a kernel: the device address of each GPU's copy is looked
// up once per device (hipGetSymbolAddress with that device current) and kept.
#include <mutex>

#include "pgg_internal.h"

namespace pgg {

namespace {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// The error word of the scratch header, decoded into [code, detail].
__global__ void export_error_kernel(const WsHeader* hdr, int64_t* out) {
  const unsigned long long e = hdr->err;
  if (e == kNoError) {
    out[0] = PGG_DEV_OK;
    out[1] = 0;
  } else {
    out[0] = static_cast<int64_t>(e >> kErrShift);
    out[1] = static_cast<int64_t>(e & kDetailMask);
  }
}

}  // namespace

hipError_t noalloc_scratch(hipStream_t stream, void** ptr) {
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    int cur = -1;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t r = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return e;
    if (r != hipSuccess) return r;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

hipError_t launch_export_error(const WsHeader* hdr, int64_t* out, hipStream_t s) {
  hipLaunchKernelGGL(export_error_kernel, dim3(1), dim3(1), 0, s, hdr, out);
  return hipGetLastError();
}

}  // namespace pgg
