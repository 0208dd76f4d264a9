// The fixed scratch area of pion_prefix_query_noalloc: for callers that cannot allocate
// device memory, the split partials and ticket counters of a query live in this
// file-scope device array instead of the per-stream workspace. Each GPU the library runs
// on holds its own copy for the life of the process.
//
// In host code `scratch` is only a stand-in for the device array, not its address; the
// address is taken once per device with hipGetSymbolAddress (that device current) and
// only that pointer is handed to kernels.
#include "kernels.h"

#include <mutex>

namespace pion {
namespace {

constexpr int kMaxScratchDevices = 64;

static __device__ __align__(256) char scratch[kNoallocScratchBytes];

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxScratchDevices] = {};

}  // namespace

hipError_t noalloc_scratch(hipStream_t s, void **ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress((void **)&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    // the ticket counters at the start must begin at zero (the merging workgroup leaves
    // each one at zero); cleared by a fill kernel on the caller's stream, not a memset
    e = launch_zero_counters((int *)p, kMaxCounters, s);
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace pion
