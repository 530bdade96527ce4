// noalloc.hip -- the library's one fixed device buffer: chunk-record scratch
// for ckda_chunk_fwd_noalloc, the forward for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc).
//
// `scratch` is a file-scope device array: every GPU the library runs on holds
// its own copy, at its own address, until the process ends.  Host code never
// passes the array's name to a kernel (on the host it names a host-side
// stand-in, not device memory); the device address is looked up once per
// device with hipGetSymbolAddress, with that device current, and kept.  All
// calls on one GPU share that GPU's copy, so calls that overlap in time on one
// GPU race with each other; calls on one stream are ordered and safe.  The
// kernels write every record byte they later read, so nothing needs clearing.
#include <mutex>

#include "ckda_internal.hpp"

namespace ckda {

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace ckda
