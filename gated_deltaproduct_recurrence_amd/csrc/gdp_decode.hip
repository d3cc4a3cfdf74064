// gdp_decode.hip -- gfx950 kernel of the single-token recurrent decode step.
//
// One step per sequence on the state cache, in place (blog page "Attention
// Cache and Sequence Parallelism", section "GDN: fixed state instead of a
// per-token cache": Sbar = lambda S, vhat = Sbar^T k, e = beta (v - vhat),
// S = Sbar + k e^T, r = q^T S; with the n Householder rows per token of the
// FlashInfer docs' recurrence display; the cache slot convention of the
// Megatron Core page, state / state_indices).
//
// The step is a stream over the K x V fp32 state: read once, updated in
// registers, written once.  One workgroup of 4 waves handles one (sequence,
// state head, 64-column tile); lane l owns column l of the tile and wave w
// owns K/4 state rows, so every state access is a 256-byte row segment per
// wave instruction.  The reductions over the K rows (S^T k, S^T q) are a sum
// of the lane's rows in registers followed by a 4-way exchange through LDS.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdp_launch.h"

namespace gdp {
namespace {

typedef __bf16 bf16;
constexpr float LOG2E_D = 1.4426950408889634f;

__device__ __forceinline__ int64_t index_at(const void *p, int is64, int64_t i) {
  return is64 ? ((const int64_t *)p)[i] : (int64_t)((const int32_t *)p)[i];
}
template <typename T> __device__ __forceinline__ float f32(T x) { return (float)x; }

// sum over the 64 lanes of a wave (the value ends up in every lane)
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

// 1 / sqrt(sum x^2 + 1e-6) of a K-element row (every lane reads K / 64 elements)
template <typename T, int K> __device__ __forceinline__ float row_rstd(const T *row, int lane) {
  float ss = 0.f;
#pragma unroll
  for (int u = 0; u < K / 64; ++u) {
    const float x = f32(row[lane + 64 * u]);
    ss = fmaf(x, x, ss);
  }
  return __builtin_amdgcn_rsqf(wave_sum(ss) + 1e-6f);
}

template <typename T, int K, int V>
__global__ void __launch_bounds__(256) gdp_decode_kernel(DecodeArgs a) {
  constexpr int NVT = V / 64, RW = K / 4;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t bid = blockIdx.x;
  const int vt = (int)(bid % NVT);
  const int h = (int)((bid / NVT) % a.Hv);
  const int64_t i = bid / ((int64_t)NVT * a.Hv);
  const int hq = h / (a.Hv / a.Hqk), hk = h / (a.Hv / a.Hk);
  const int col = vt * 64 + lane;
  T *orow = (T *)a.o + i * a.o_st + (int64_t)h * a.o_sh;
  const int64_t slot = index_at(a.slots, a.slots_is64, i);
  if (slot < 0 || slot >= a.num_slots) {  // padding entry: zero output, no state access
    if (w == 0) orow[col] = (T)0.f;
    return;
  }
  float *S = a.cache + ((size_t)slot * a.Hv + h) * ((size_t)K * V) + (size_t)(w * RW) * V + col;
  float s[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r) s[r] = S[(size_t)r * V];
  const float alpha = __builtin_amdgcn_exp2f(a.g[i * a.g_st + (int64_t)h * a.g_sh] * LOG2E_D);
#pragma unroll
  for (int r = 0; r < RW; ++r) s[r] *= alpha;

  __shared__ float red[2][4][64];
  for (int j = 0; j < a.n; ++j) {
    const int64_t row = i * a.n + j;
    const T *kr = (const T *)a.k + row * a.k_st + (int64_t)hk * a.k_sh;
    const float rk = a.l2norm ? row_rstd<T, K>(kr, lane) : 1.f;
    float kap[RW];
#pragma unroll
    for (int r = 0; r < RW; ++r) kap[r] = f32(kr[w * RW + r]) * rk;
    float part = 0.f;
#pragma unroll
    for (int r = 0; r < RW; ++r) part = fmaf(s[r], kap[r], part);
    red[j & 1][w][lane] = part;
    __syncthreads();
    const float vhat = (red[j & 1][0][lane] + red[j & 1][1][lane]) + (red[j & 1][2][lane] + red[j & 1][3][lane]);
    const float vv = f32(((const T *)a.v)[row * a.v_st + (int64_t)h * a.v_sh + col]);
    const float e = a.beta[row * a.b_st + (int64_t)h * a.b_sh] * (vv - vhat);
#pragma unroll
    for (int r = 0; r < RW; ++r) s[r] = fmaf(kap[r], e, s[r]);
  }
  // readout after the last update
  const T *qr = (const T *)a.q + i * a.q_st + (int64_t)hq * a.q_sh;
  const float rq = a.l2norm ? row_rstd<T, K>(qr, lane) : 1.f;
  float part = 0.f;
#pragma unroll
  for (int r = 0; r < RW; ++r) part = fmaf(s[r], f32(qr[w * RW + r]) * rq, part);
  const int rb = a.n & 1;
  red[rb][w][lane] = part;
  __syncthreads();
  if (w == 0) {
    const float ov = (red[rb][0][lane] + red[rb][1][lane]) + (red[rb][2][lane] + red[rb][3][lane]);
    orow[col] = (T)(a.scale * ov);
  }
#pragma unroll
  for (int r = 0; r < RW; ++r) S[(size_t)r * V] = s[r];
}

template <typename T, int K, int V> hipError_t launch(const DecodeArgs &a, hipStream_t stream) {
  const int64_t blocks = (int64_t)a.N * a.Hv * (V / 64);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((gdp_decode_kernel<T, K, V>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

bool decode_supported(int K, int V) { return (K == 64 || K == 128) && (V == 64 || V == 128); }

hipError_t launch_decode(const DecodeArgs &a, int dtype, int K, int V, hipStream_t stream) {
  if (dtype == IN_BF16) {
    if (K == 128 && V == 128) return launch<bf16, 128, 128>(a, stream);
    if (K == 128 && V == 64) return launch<bf16, 128, 64>(a, stream);
    if (K == 64 && V == 128) return launch<bf16, 64, 128>(a, stream);
    if (K == 64 && V == 64) return launch<bf16, 64, 64>(a, stream);
  } else if (dtype == IN_F32) {
    if (K == 128 && V == 128) return launch<float, 128, 128>(a, stream);
    if (K == 128 && V == 64) return launch<float, 128, 64>(a, stream);
    if (K == 64 && V == 128) return launch<float, 64, 128>(a, stream);
    if (K == 64 && V == 64) return launch<float, 64, 64>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdp
