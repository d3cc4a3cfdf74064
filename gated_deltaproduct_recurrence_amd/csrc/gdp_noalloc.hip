// gdp_noalloc.hip -- the static scratch array of gdp_chunk_prefill_noalloc.
//
// Callers that cannot allocate device memory (code under graph capture, tight
// serving loops, harnesses that forbid hipMalloc) get the prefill's workspace
// from this file-scope device array instead of a caller buffer.  Every GPU the
// library runs on holds its own copy of the array until the process ends; all
// calls on one GPU share it, so calls that overlap on one GPU (for instance on
// two streams) race.  The prefill writes every part of its workspace before
// reading it (descriptors, work order, progress counters, WY matrices, segment
// buffers), so no call depends on what the previous one left there.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "gdp.h"
#include "gdp_launch.h"

namespace gdp {
namespace {

__device__ __align__(256) char scratch[GDP_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void *g_scratch_ptr[64] = {};

}  // namespace

hipError_t noalloc_scratch(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    // the array's name is a host-side stand-in: its device address comes from
    // the runtime, once per device, with that device current
    void *p = nullptr;
    if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace gdp
