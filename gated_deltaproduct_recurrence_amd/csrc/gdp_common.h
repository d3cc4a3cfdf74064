// gdp_common.h -- device types, constants and the WY inverse shared by the
// forward kernels (gdp_kernels.hip) and the chunked gradients (gdp_bwd_chunk.hip).
#pragma once
#include <hip/hip_runtime.h>

namespace gdp {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int CH = 64;  // chunk length on both streams
constexpr int NTHR = 256;
constexpr float LOG2E = 1.4426950408889634f;

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// ---------------------------------------------------------------- WY inverse
//
// T = (I + A)^-1 for the strictly lower-triangular 64 x 64 A (fp32, LDS), into
// Tf (fp32, LDS, zeros above the diagonal blocks).  Wave w inverts diagonal
// 16 x 16 block w by forward substitution, one lane per column, carrying the
// partial sums of all later rows so that each row needs one dependent step.
// The off-diagonal blocks follow from T_ab = -T_aa sum_{c=b}^{a-1} A_ac T_cb,
// one sweep per block distance a - b, on fp32 MFMA.
template <int LDA>
__device__ __forceinline__ void wy_inverse(const float *A, float *Tf, int tid) {
  const int w = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  for (int idx = tid; idx < 6 * 256; idx += NTHR) {  // blocks strictly above the diagonal
    const int blk = idx >> 8, e = idx & 255;
    const int a = (blk < 3) ? 0 : (blk < 5 ? 1 : 2);
    const int b = (blk < 3) ? blk + 1 : (blk < 5 ? blk - 1 : 3);
    Tf[(16 * a + (e >> 4)) * LDA + 16 * b + (e & 15)] = 0.f;
  }
  {
    const int j = lr;
    const float *Ab = A + (16 * w) * LDA + 16 * w;
    float acc[16], x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      x[i] = (i == j ? 1.f : 0.f) - acc[i];
#pragma unroll
      for (int r = i + 1; r < 16; ++r) acc[r] = fmaf(Ab[r * LDA + i], x[i], acc[r]);
    }
    if (lg == 0) {
      float *Td = Tf + (16 * w) * LDA + 16 * w + j;
#pragma unroll
      for (int r = 0; r < 16; ++r) Td[r * LDA] = x[r];
    }
  }
  __syncthreads();
#pragma unroll
  for (int d = 1; d < 4; ++d) {
    if (w < 4 - d) {
      const int ba = w + d, bb = w;
      f32x4 y = zero4();
      for (int c = bb; c < ba; ++c) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const float av = A[(16 * ba + lr) * LDA + 16 * c + 4 * kk + lg];
          const float bv = Tf[(16 * c + 4 * kk + lg) * LDA + 16 * bb + lr];
          y = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, y, 0, 0, 0);
        }
      }
      f32x4 z = zero4();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float av = Tf[(16 * ba + lr) * LDA + 16 * ba + 4 * lg + i];
        z = __builtin_amdgcn_mfma_f32_16x16x4f32(av, y[i], z, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) Tf[(16 * ba + 4 * lg + i) * LDA + 16 * bb + lr] = -z[i];
    }
    __syncthreads();
  }
}

}  // namespace gdp
