// gdp_frontend.hip -- gfx950 conversion kernels of the FlashInfer-convention
// front end (FlashInfer docs, "flashinfer.gdp_prefill.chunk_gated_delta_product",
// parameter list).
//
// That convention differs from the one the prefill kernels take (Megatron Core
// page, core.ssm.ops.gdp.chunk, chunk_gated_delta_product_varlen) only in how
// the operands are stated:
//   - g is the decay itself, alpha in (0, 1], in float32, bfloat16 or float16, or
//     absent (no decay); the prefill kernels take log decays in float32;
//   - beta may be float32 or the input dtype, or absent (all ones);
//   - the states are V-major [N, H, V, K], float32 or bfloat16; the prefill
//     kernels keep K-major [N, H, K, V] float32 states.
// These kernels restate the operands in the prefill kernels' form (in the
// caller's workspace) and write the final state back in the caller's layout.
// float16 q/k/v are restated as bfloat16: the prefill kernels' products with the
// state (kept with a lazy scale far outside float16's range) need bfloat16
// operands, and one matrix-core product takes one operand type; the output is
// formed in bfloat16 and converted to float16.
// The recurrence itself runs in the prefill kernels.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdp_launch.h"

namespace gdp {
namespace {

__device__ __forceinline__ float load_as_f32(const void *p, int64_t i, int dtype) {
  if (dtype == EL_F32) return ((const float *)p)[i];
  if (dtype == EL_BF16) return (float)((const __bf16 *)p)[i];
  return (float)((const _Float16 *)p)[i];
}

// g_log[t, h] = ln(alpha[t, h]) (0 when alpha is absent); beta32[r, h] = beta[r, h]
// (1 when absent), unless beta32 is null (a float32 beta is read in place).  Both
// outputs are contiguous float32.
__global__ void __launch_bounds__(256) gdp_gate_kernel(GateArgs a) {
  const int64_t ng = a.T * a.Hv, nb = a.beta32 ? a.T * a.n * a.Hv : 0;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < ng + nb; i += (int64_t)gridDim.x * 256) {
    if (i < ng) {
      const int64_t t = i / a.Hv, h = i - t * a.Hv;
      a.g_log[i] = a.alpha ? logf(load_as_f32(a.alpha, t * a.a_st + h * a.a_sh, a.alpha_dtype)) : 0.f;
    } else {
      const int64_t j = i - ng, r = j / a.Hv, h = j - r * a.Hv;
      a.beta32[j] = a.beta ? load_as_f32(a.beta, r * a.b_st + h * a.b_sh, a.beta_dtype) : 1.f;
    }
  }
}

// One 64 x 64 tile of one (sequence, head) state per workgroup, transposed
// through LDS: dst[c][r] = src[r][c] for a src of R x C elements (rows of C).
// to_k: src V-major (any state dtype) -> dst K-major float32; else src K-major
// float32 -> dst V-major (the state dtype).
template <bool TO_K>
__global__ void __launch_bounds__(256) gdp_state_transpose_kernel(StateArgs a) {
  __shared__ float tile[64][65];
  const int R = TO_K ? a.V : a.K, C = TO_K ? a.K : a.V;  // src rows x columns
  const int tiles_c = C / 64, tiles_r = R / 64;
  const int64_t mat = blockIdx.x / (tiles_r * tiles_c);
  const int tr = (int)(blockIdx.x / tiles_c % tiles_r), tc = (int)(blockIdx.x % tiles_c);
  const size_t base = (size_t)mat * R * C;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int r = ty; r < 64; r += 4) {
    const size_t i = base + (size_t)(64 * tr + r) * C + 64 * tc + tx;
    tile[r][tx] = TO_K ? load_as_f32(a.src, (int64_t)i, a.state_dtype) : ((const float *)a.src)[i];
  }
  __syncthreads();
  for (int c = ty; c < 64; c += 4) {
    const size_t o = base + (size_t)(64 * tc + c) * R + 64 * tr + tx;
    const float x = tile[tx][c];
    if (TO_K || a.state_dtype == EL_F32) ((float *)a.dst)[o] = x;
    else ((__bf16 *)a.dst)[o] = (__bf16)x;
  }
}

// Row-strided [R, H, D] copy between float16 and bfloat16 (TO_BF16: float16
// source, contiguous bfloat16 destination; else contiguous bfloat16 source,
// strided float16 destination).  D a multiple of 8: each thread moves 8 elements.
template <bool TO_BF16>
__global__ void __launch_bounds__(256) gdp_half_copy_kernel(HalfCopyArgs a) {
  const int64_t per_row = (int64_t)a.H * a.D / 8;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < a.R * per_row; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / per_row, rem = i - r * per_row, hh = rem / (a.D / 8), d8 = rem - hh * (a.D / 8);
    const int64_t strided = r * a.st + hh * a.sh + 8 * d8, dense = (r * a.H + hh) * a.D + 8 * d8;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (TO_BF16) ((__bf16 *)a.dst)[dense + e] = (__bf16)(float)((const _Float16 *)a.src)[strided + e];
      else ((_Float16 *)a.dst)[strided + e] = (_Float16)(float)((const __bf16 *)a.src)[dense + e];
    }
  }
}

}  // namespace

hipError_t launch_half_copy(const HalfCopyArgs &a, bool to_bf16, hipStream_t stream) {
  if (a.D % 8) return hipErrorInvalidValue;
  const int64_t total = a.R * a.H * a.D / 8;
  if (total <= 0) return hipSuccess;
  const int64_t blocks = (total + 255) / 256 < 8192 ? (total + 255) / 256 : 8192;
  if (to_bf16) hipLaunchKernelGGL(gdp_half_copy_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  else hipLaunchKernelGGL(gdp_half_copy_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_gates(const GateArgs &a, hipStream_t stream) {
  const int64_t total = a.T * a.Hv * (1 + (a.beta32 ? a.n : 0));
  if (total <= 0) return hipSuccess;
  const int64_t blocks = (total + 255) / 256 < 4096 ? (total + 255) / 256 : 4096;
  hipLaunchKernelGGL(gdp_gate_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_state_transpose(const StateArgs &a, bool to_k_major, hipStream_t stream) {
  if (a.K % 64 || a.V % 64) return hipErrorInvalidValue;
  const int64_t blocks = a.mats * (a.K / 64) * (a.V / 64);
  if (blocks <= 0) return hipSuccess;
  if (to_k_major)
    hipLaunchKernelGGL(gdp_state_transpose_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(gdp_state_transpose_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace gdp
