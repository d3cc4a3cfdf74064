// gdp_validate.hip -- opt-in device checks of the data-dependent arguments.
//
// The pages make cu_seqlens the cumulative, non-decreasing sequence boundaries
// (Megatron Core page, chunk_gated_delta_product_varlen, argument list) and
// state_indices the cache slot of each sequence, with -1 for no write (same page,
// the state-cache arguments).  Checking either takes a read of device data, so
// the calls do not check them by default: every kernel clamps sequence ranges to
// [0, T] and skips slots outside the cache, which keeps a bad value in bounds
// but gives undefined results.  With GDP_DEBUG_VALIDATE=1 in the environment the
// prefill and decode calls first launch gdp_validate_kernel, which ORs a bit per
// kind of fault into a device-global word:
//   GDP_DBG_CU    cu_seqlens decreases somewhere, or an entry lies outside [0, T]
//   GDP_DBG_SLOT  a state index is below -1 or not below the number of cache slots
//   GDP_DBG_DUP   two sequences (entries) share a non-negative state index
// gdp_debug_status reads the word back (synchronising the stream) and may clear it.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "gdp.h"
#include "gdp_launch.h"

namespace gdp {
namespace {

// One word per device (each device holds its own copy of this variable).
__device__ uint32_t debug_word;

__device__ __forceinline__ int64_t idx_at(const void *p, int is64, int64_t i) {
  return is64 ? ((const int64_t *)p)[i] : (int64_t)((const int32_t *)p)[i];
}

// Grid-stride over pairs (i, j): i indexes the boundaries / slots, and for the
// duplicate check j runs over the later slots (the quadratic scan is the price
// of a check that needs no sort and no scratch; it is a debugging aid).
__global__ void __launch_bounds__(256) gdp_validate_kernel(ValidateArgs a) {
  uint32_t bits = 0;
  const int64_t stride = (int64_t)gridDim.x * 256;
  const int64_t first = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (a.cu) {
    for (int64_t i = first; i <= a.N; i += stride) {
      const int64_t x = idx_at(a.cu, a.cu_is64, i);
      if (x < 0 || x > a.T) bits |= GDP_DBG_CU;
      if (i < a.N && idx_at(a.cu, a.cu_is64, i + 1) < x) bits |= GDP_DBG_CU;
    }
  }
  if (a.slots) {
    for (int64_t i = first; i < a.nslots_given; i += stride) {
      const int64_t s = idx_at(a.slots, a.slots_is64, i);
      if (s < -1 || s >= a.num_slots) bits |= GDP_DBG_SLOT;
      if (s < 0) continue;
      for (int64_t j = i + 1; j < a.nslots_given; ++j)
        if (idx_at(a.slots, a.slots_is64, j) == s) {
          bits |= GDP_DBG_DUP;
          break;
        }
    }
  }
  if (bits) atomicOr(a.word, bits);
}

std::mutex g_word_mu;
uint32_t *g_word_ptr[64] = {};

}  // namespace

hipError_t debug_word_ptr(uint32_t **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_word_mu);
  if (!g_word_ptr[dev]) {
    void *p = nullptr;
    // the variable's name is a host-side stand-in: its device address comes
    // from the runtime, per device, with that device current
    if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(debug_word))) != hipSuccess) return e;
    g_word_ptr[dev] = (uint32_t *)p;
  }
  *out = g_word_ptr[dev];
  return hipSuccess;
}

hipError_t launch_validate(ValidateArgs a, hipStream_t stream) {
  if (!a.cu && !a.slots) return hipSuccess;
  hipError_t e = debug_word_ptr(&a.word);
  if (e != hipSuccess) return e;
  const int64_t work = (a.N + 1 > a.nslots_given ? a.N + 1 : a.nslots_given);
  const int64_t blocks = work <= 0 ? 1 : ((work + 255) / 256 < 1024 ? (work + 255) / 256 : 1024);
  hipLaunchKernelGGL(gdp_validate_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace gdp
