// Allocation-free attention backward: the workspace of csa_sparse_attn_bwd lives in a
// static device array of this translation unit instead of a caller buffer.
//
// For callers that cannot allocate device memory (code under stream capture, tight serving
// loops, harnesses that forbid hipMalloc).  Each GPU the library runs on holds its own copy
// of the array (kScratchBytes) from the first use of the library on that GPU until the
// process ends.  Every call on a GPU uses that GPU's one array, so calls that overlap in time
// on one GPU (two streams, two host threads) race on it and must be serialized by the
// caller.  The backward writes every workspace region it reads within the same call (its
// counters are cleared by a fill kernel at the start of each query chunk), so nothing depends
// on what an earlier call left there.
#include <hip/hip_runtime.h>

#include <mutex>

#include "csa_launch.h"

namespace csa {

namespace {

constexpr size_t kScratchBytes = 256ull << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// Device address of this GPU's scratch array: looked up once per device with that device
// current (the array's host-side name is not a device address).
hipError_t scratch_ptr(hipStream_t s, void** out) {
  hipDevice_t dev = -1;
  hipError_t e = hipStreamGetDevice(s, &dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[dev]) {
    int cur = -1;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace

size_t attn_bwd_scratch_bytes() { return kScratchBytes; }

hipError_t launch_attn_bwd_noalloc(const Shape& sh, AttnIO io, hipStream_t s) {
  void* p = nullptr;
  hipError_t e = scratch_ptr(s, &p);
  if (e != hipSuccess) return e;
  io.ws = p;
  io.ws_bytes = kScratchBytes;
  return launch_attn_bwd(sh, io, s);
}

}  // namespace csa
