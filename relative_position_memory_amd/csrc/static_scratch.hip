// The library's one piece of static device memory: the scratch of
// txl_rel_attn_fwd_noalloc, for callers that cannot allocate (code under graph
// capture, serving loops, harnesses that forbid hipMalloc).
//
// `scratch` is a file-scope __device__ array.  Each device the library runs on
// holds its own copy from the loading of the code object until the process
// ends.  In host code the array's name is only a host-side stand-in: its device
// address is looked up once per device with hipGetSymbolAddress (with that
// device current) and kept; every kernel argument uses that address.
#include <mutex>

#include "txl_internal.h"

namespace txl {

__device__ __align__(256) unsigned char scratch[STATIC_SCRATCH_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
void* g_ptr[MAX_DEVICES] = {};
}  // namespace

hipError_t static_scratch_ptr(void** out) {
  *out = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace txl
