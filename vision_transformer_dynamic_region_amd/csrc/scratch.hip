// Device scratch of the entry points that allocate nothing: a file-scope
// array in the library's code object, so callers that may not allocate
// (code under HIP graph capture, tight serving loops) get working memory
// without hipMalloc.  Each GPU the library runs on holds its own copy,
// kScratchBytes, until the process ends.  In host code the array's name
// stands in for the symbol only; its device address comes from
// hipGetSymbolAddress, once per device with that device current, and is
// what every kernel and copy takes.  Every call on a GPU shares that GPU's
// array: calls that overlap on one GPU race.

#include <atomic>

#include "bra_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[bra::kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];

}  // namespace

namespace bra {

hipError_t scratch_buffer(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_addr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

}  // namespace bra
