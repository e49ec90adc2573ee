// dn_noalloc.hip -- the fixed scratch area behind deltanet_chunk_fwd_noalloc,
// for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The area is a file-scope device array: every GPU the library runs on holds
// its own copy, at its own address, from module load until the process ends.
// Host code never passes the array's name to a kernel or a copy (on the host
// that name is only a stand-in, not a device address); it asks the runtime
// for this device's address once, with the device current, and keeps it.
// Every call on one GPU shares that GPU's copy, which keeps the previous
// call's contents: the chunked forward's kernels write every scratch byte
// they later read, so nothing has to be cleared between calls, and calls
// that overlap in time on one GPU race.

#include <hip/hip_runtime.h>

#include <mutex>

#include "dn_launch.h"

namespace dn {

namespace {

constexpr size_t kScratchBytes = kNoallocScratchBytes;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_addr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(hipStream_t stream, void** out) {
  *out = nullptr;
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  hipDevice_t dev = cur;
  if (stream != nullptr) {
    e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return e;
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_addr[dev] == nullptr) {
    // Look the address up with the stream's device current.
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_addr[dev] = p;
  }
  *out = g_addr[dev];
  return hipSuccess;
}

}  // namespace dn
