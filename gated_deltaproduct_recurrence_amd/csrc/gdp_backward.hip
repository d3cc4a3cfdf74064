// gdp_backward.hip -- gfx950 kernels of the gradients of the GDP prefill.
//
// The pages give no backward formulas (the blog page "Attention Cache and
// Sequence Parallelism" only notes, in the section "GDN: pass the state, not
// the KV", that the backward dependencies run in the opposite direction).  What
// is computed here is reverse-mode differentiation of the recurrence itself
// (FlashInfer docs, "flashinfer.gdp_prefill.chunk_gated_delta_product", the
// recurrence display, K-major orientation): per token t, with S_{t-1} entering,
//     S^0 = alpha_t S_{t-1};  for j: u_j = v_j - S^j^T k_j, e_j = beta_j u_j,
//     S^{j+1} = S^j + k_j e_j^T;   S_t = S^n;  o_t = scale S_t^T q_t.
// Going backwards with dS = dL/dS_t:
//     dS += scale q_t do_t^T;          dq_t = scale S_t do_t
//     for j = n-1 .. 0:  de = dS^T k_j;  du = beta_j de;  dv_j = du;
//                        dbeta_j = de . u_j;  dk_j = dS e_j - S^j du;  dS -= k_j du^T
//     dalpha_t = <dS, S_{t-1}>,  dg_log_t = alpha_t dalpha_t;  dS <- alpha_t dS.
// (k and q here are the L2-normalised rows when the in-kernel norm is on; the
// finalize kernel maps their gradients back to the raw rows.)
//
// The states S_{t-1} are recomputed: the forward pass leaves the state entering
// every 64-token chunk (return_chunk_states); per chunk this kernel re-runs the
// recurrence once to keep the state entering every 8th token in LDS, and once
// per 8-token block to hold the 8 token states in registers, then walks the
// block backwards.  One wave owns one (sequence, state head, 8-column V tile):
// lane (rg, c) = (lane / 8, lane % 8) holds rows 16 rg .. 16 rg + 15 (K = 128;
// 8 rows for K = 64) of column c, so a column dot over K is a sum over the 8
// lanes of equal c and a row sum over the tile's columns one over the 8 lanes of
// equal rg, both by lane exchanges.  Gradients shared by several waves (dq, dk:
// all V tiles and the state heads of a q/k head; dbeta, dg_log: all V tiles)
// are accumulated with float atomics into zeroed buffers.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdp_launch.h"

namespace gdp {
namespace {

constexpr int CH = 64;     // token chunk of the forward pass's chunk states
constexpr int VT = 8;      // columns per wave
constexpr int BLK = 8;     // tokens per register block (checkpoint spacing)
constexpr int NMAX = 4;    // Householder rows per token served
constexpr float LOG2E_B = 1.4426950408889634f;

__device__ __forceinline__ int64_t idx_at(const void *p, int is64, int64_t i) {
  return is64 ? ((const int64_t *)p)[i] : (int64_t)((const int32_t *)p)[i];
}
// sum over the lanes whose indices differ in the bits LO .. HI (powers of two)
template <int LO, int HI> __device__ __forceinline__ float xsum(float x) {
#pragma unroll
  for (int m = LO; m <= HI; m <<= 1) x += __shfl_xor(x, m, 64);
  return x;
}
__device__ __forceinline__ float col_sum(float x) { return xsum<8, 32>(x); }  // over rg (rows)
__device__ __forceinline__ float row_sum(float x) { return xsum<1, 4>(x); }   // over c (columns)

template <typename T, int K, int V> struct Bwd {
  static constexpr int RK = K / 8;  // rows per lane
  const BwdArgs &a;
  int seq, h, hq, hk, vt, lane, rg, c;
  int64_t t0, L;
  __device__ Bwd(const BwdArgs &args) : a(args) {}

  // the lane's RK entries of row `row` of a [., H, K] tensor (normalised when asked)
  __device__ __forceinline__ void load_row(float (&x)[RK], const T *base, int64_t row, int64_t st, int64_t sh, int head,
                                           float &rstd) const {
    const T *p = base + row * st + (int64_t)head * sh + RK * rg;
#pragma unroll
    for (int i = 0; i < RK; ++i) x[i] = (float)p[i];
    rstd = 1.f;
    if (a.l2norm) {
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < RK; ++i) ss = fmaf(x[i], x[i], ss);
      rstd = __builtin_amdgcn_rsqf(col_sum(ss) + 1e-6f);
#pragma unroll
      for (int i = 0; i < RK; ++i) x[i] *= rstd;
    }
  }
  __device__ __forceinline__ float alpha_of(int64_t t) const {
    return __builtin_amdgcn_exp2f(a.g[t * a.g_st + (int64_t)h * a.g_sh] * LOG2E_B);
  }
  __device__ __forceinline__ float beta_of(int64_t r) const { return a.beta[r * a.b_st + (int64_t)h * a.b_sh]; }
  __device__ __forceinline__ float v_of(int64_t r) const {
    return (float)((const T *)a.v)[r * a.v_st + (int64_t)h * a.v_sh + VT * vt + c];
  }
  // one token forward on S (the lane's part)
  __device__ __forceinline__ void step(float (&S)[RK], int64_t t) const {
    const float al = alpha_of(t);
#pragma unroll
    for (int i = 0; i < RK; ++i) S[i] *= al;
    for (int j = 0; j < a.n; ++j) {
      const int64_t r = t * a.n + j;
      float kv[RK], rk;
      load_row(kv, (const T *)a.k, r, a.k_st, a.k_sh, hk, rk);
      float part = 0.f;
#pragma unroll
      for (int i = 0; i < RK; ++i) part = fmaf(S[i], kv[i], part);
      const float e = beta_of(r) * (v_of(r) - col_sum(part));
#pragma unroll
      for (int i = 0; i < RK; ++i) S[i] = fmaf(kv[i], e, S[i]);
    }
  }
};

template <typename T, int K, int V>
__global__ void __launch_bounds__(256) gdp_backward_kernel(BwdArgs a) {
  using B = Bwd<T, K, V>;
  constexpr int RK = B::RK, NVT = V / VT;
  // per wave: the state entering each 8-token block of the chunk (64 tokens)
  __shared__ float ck[4][CH / BLK][RK * 64];
  B s(a);
  const int w = threadIdx.x >> 6;
  s.lane = threadIdx.x & 63;
  s.rg = s.lane >> 3;
  s.c = s.lane & 7;
  const int64_t wid = (int64_t)blockIdx.x * 4 + w;
  const int64_t nw = (int64_t)a.N * a.Hv * NVT;
  if (wid >= nw) return;
  s.vt = (int)(wid % NVT);
  s.h = (int)((wid / NVT) % a.Hv);
  s.seq = (int)(wid / ((int64_t)NVT * a.Hv));
  s.hq = s.h / (a.Hv / a.Hqk);
  s.hk = s.h / (a.Hv / a.Hk);
  int64_t t0 = idx_at(a.cu, a.cu_is64, s.seq), t1 = idx_at(a.cu, a.cu_is64, s.seq + 1);
  t0 = t0 < 0 ? 0 : (t0 > a.T ? a.T : t0);
  t1 = t1 < t0 ? t0 : (t1 > a.T ? a.T : t1);
  s.t0 = t0;
  s.L = t1 - t0;
  const int ntc = (int)((s.L + CH - 1) / CH);
  const int col = VT * s.vt + s.c;
  const size_t KV = (size_t)K * V;
  const size_t soff = ((size_t)s.seq * a.Hv + s.h) * KV + (size_t)(RK * s.rg) * V + col;  // + i * V
  float *my_ck = &ck[w][0][0];

  float dS[RK];
#pragma unroll
  for (int i = 0; i < RK; ++i) dS[i] = a.dfinal ? a.dfinal[soff + (size_t)i * V] : 0.f;

  for (int cc = ntc - 1; cc >= 0; --cc) {
    const int64_t tb = t0 + (int64_t)CH * cc;
    const int ntok = (int)((t1 - tb) < CH ? (t1 - tb) : CH);
    // the state entering the chunk, then the states entering every 8th token
    float S[RK];
    const int64_t csrow = (int64_t)a.chunk_offsets[s.seq] + cc;
    const float *src = a.chunk_states + (size_t)csrow * a.Hv * KV + (soff - (size_t)s.seq * a.Hv * KV);
#pragma unroll
    for (int i = 0; i < RK; ++i) S[i] = src[(size_t)i * V];
    const int nblk = (ntok + BLK - 1) / BLK;
    for (int b = 0; b < nblk; ++b) {
#pragma unroll
      for (int i = 0; i < RK; ++i) my_ck[(b * RK + i) * 64 + s.lane] = S[i];
      if (b + 1 < nblk)
        for (int m = 0; m < BLK; ++m) s.step(S, tb + BLK * b + m);
    }
    // blocks backwards
    for (int b = nblk - 1; b >= 0; --b) {
      const int nb = (ntok - BLK * b) < BLK ? (ntok - BLK * b) : BLK;
      float ST[BLK][RK];  // state entering token m of the block
#pragma unroll
      for (int i = 0; i < RK; ++i) ST[0][i] = my_ck[(b * RK + i) * 64 + s.lane];
#pragma unroll
      for (int m = 1; m < BLK; ++m) {
        if (m < nb) {
#pragma unroll
          for (int i = 0; i < RK; ++i) ST[m][i] = ST[m - 1][i];
          s.step(ST[m], tb + BLK * b + m - 1);
        }
      }
#pragma unroll
      for (int m = BLK - 1; m >= 0; --m) {
        if (m >= nb) continue;
        const int64_t t = tb + BLK * b + m;
        const float al = s.alpha_of(t);
        // recompute the token's sub-states S^j and u_j, e_j
        float Sj[NMAX][RK], u[NMAX], e[NMAX], bt[NMAX];
        float cur[RK];
#pragma unroll
        for (int i = 0; i < RK; ++i) cur[i] = al * ST[m][i];
#pragma unroll
        for (int j = 0; j < NMAX; ++j) {
          if (j < a.n) {
            const int64_t r = t * a.n + j;
            float kv[RK], rk;
            s.load_row(kv, (const T *)a.k, r, a.k_st, a.k_sh, s.hk, rk);
            float part = 0.f;
#pragma unroll
            for (int i = 0; i < RK; ++i) {
              Sj[j][i] = cur[i];
              part = fmaf(cur[i], kv[i], part);
            }
            bt[j] = s.beta_of(r);
            u[j] = s.v_of(r) - col_sum(part);
            e[j] = bt[j] * u[j];
#pragma unroll
            for (int i = 0; i < RK; ++i) cur[i] = fmaf(kv[i], e[j], cur[i]);
          }
        }
        // readout: o_t = scale S_t^T q_t
        {
          float qv[RK], rq;
          s.load_row(qv, (const T *)a.q, t, a.q_st, a.q_sh, s.hq, rq);
          const float dov = (float)((const T *)a.dout)[t * a.do_st + (int64_t)s.h * a.do_sh + col] * a.scale;
#pragma unroll
          for (int i = 0; i < RK; ++i) {
            const float dq = row_sum(cur[i] * dov);
            if (s.c == 0) atomicAdd(a.dq + t * a.dq_st + (int64_t)s.hq * a.dq_sh + RK * s.rg + i, dq);
            dS[i] = fmaf(qv[i], dov, dS[i]);
          }
        }
#pragma unroll
        for (int j = NMAX - 1; j >= 0; --j) {
          if (j < a.n) {
            const int64_t r = t * a.n + j;
            float kv[RK], rk;
            s.load_row(kv, (const T *)a.k, r, a.k_st, a.k_sh, s.hk, rk);
            float part = 0.f;
#pragma unroll
            for (int i = 0; i < RK; ++i) part = fmaf(dS[i], kv[i], part);
            const float de = col_sum(part);
            const float du = bt[j] * de;
            if (s.rg == 0) a.dv[r * a.dv_st + (int64_t)s.h * a.dv_sh + col] = du;
            const float db = row_sum(de * u[j]);
            if (s.lane == 0) atomicAdd(a.dbeta + r * a.db_st + (int64_t)s.h * a.db_sh, db);
#pragma unroll
            for (int i = 0; i < RK; ++i) {
              const float dk = row_sum(dS[i] * e[j] - Sj[j][i] * du);
              if (s.c == 0) atomicAdd(a.dk + r * a.dk_st + (int64_t)s.hk * a.dk_sh + RK * s.rg + i, dk);
              dS[i] = fmaf(-kv[i], du, dS[i]);
            }
          }
        }
        // decay
        float part = 0.f;
#pragma unroll
        for (int i = 0; i < RK; ++i) part = fmaf(dS[i], ST[m][i], part);
        const float dal = xsum<1, 32>(part);
        if (s.lane == 0) atomicAdd(a.dg + t * a.dg_st + (int64_t)s.h * a.dg_sh, dal * al);
#pragma unroll
        for (int i = 0; i < RK; ++i) dS[i] *= al;
      }
    }
  }
  if (a.ds0) {
#pragma unroll
    for (int i = 0; i < RK; ++i) a.ds0[soff + (size_t)i * V] = dS[i];
  }
}

// Gradients with respect to the raw q and k rows when the kernel normalised
// them: with xh = x r, r = (|x|^2 + 1e-6)^(-1/2) and G the gradient with respect
// to xh, the gradient with respect to x is r (G - xh (xh . G)).  One wave per row.
template <typename T, int K>
__global__ void __launch_bounds__(256) gdp_l2norm_grad_kernel(NormGradArgs a) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= a.rows) return;
  const int64_t r = row / a.heads, hh = row % a.heads;
  const T *x = (const T *)a.x + r * a.x_st + hh * a.x_sh;
  float *g = a.g + r * a.g_st + hh * a.g_sh;
  constexpr int PL = K / 64;
  float xv[PL], gv[PL], ss = 0.f;
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    xv[i] = (float)x[lane + 64 * i];
    gv[i] = g[lane + 64 * i];
    ss = fmaf(xv[i], xv[i], ss);
  }
  const float rs = __builtin_amdgcn_rsqf(xsum<1, 32>(ss) + 1e-6f);
  float dot = 0.f;
#pragma unroll
  for (int i = 0; i < PL; ++i) dot = fmaf(xv[i] * rs, gv[i], dot);
  dot = xsum<1, 32>(dot);
#pragma unroll
  for (int i = 0; i < PL; ++i) g[lane + 64 * i] = rs * (gv[i] - xv[i] * rs * dot);
}

template <typename T, int K, int V> hipError_t launch_bwd(const BwdArgs &a, hipStream_t stream) {
  const int64_t waves = (int64_t)a.N * a.Hv * (V / VT);
  if (waves == 0) return hipSuccess;
  hipLaunchKernelGGL((gdp_backward_kernel<T, K, V>), dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

bool backward_supported(int K, int V, int n) {
  return (K == 64 || K == 128) && (V == 64 || V == 128) && n >= 1 && n <= NMAX;
}

hipError_t launch_backward(const BwdArgs &a, int dtype, int K, int V, hipStream_t stream) {
  if (dtype == IN_BF16) {
    if (K == 128 && V == 128) return launch_bwd<__bf16, 128, 128>(a, stream);
    if (K == 128 && V == 64) return launch_bwd<__bf16, 128, 64>(a, stream);
    if (K == 64 && V == 128) return launch_bwd<__bf16, 64, 128>(a, stream);
    if (K == 64 && V == 64) return launch_bwd<__bf16, 64, 64>(a, stream);
  } else if (dtype == IN_F32) {
    if (K == 128 && V == 128) return launch_bwd<float, 128, 128>(a, stream);
    if (K == 128 && V == 64) return launch_bwd<float, 128, 64>(a, stream);
    if (K == 64 && V == 128) return launch_bwd<float, 64, 128>(a, stream);
    if (K == 64 && V == 64) return launch_bwd<float, 64, 64>(a, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_l2norm_grad(const NormGradArgs &a, int dtype, int K, hipStream_t stream) {
  if (a.rows == 0) return hipSuccess;
  const dim3 grid((unsigned)((a.rows + 3) / 4));
  if (dtype == IN_BF16) {
    if (K == 128) hipLaunchKernelGGL((gdp_l2norm_grad_kernel<__bf16, 128>), grid, dim3(256), 0, stream, a);
    else if (K == 64) hipLaunchKernelGGL((gdp_l2norm_grad_kernel<__bf16, 64>), grid, dim3(256), 0, stream, a);
    else return hipErrorInvalidValue;
  } else if (dtype == IN_F32) {
    if (K == 128) hipLaunchKernelGGL((gdp_l2norm_grad_kernel<float, 128>), grid, dim3(256), 0, stream, a);
    else if (K == 64) hipLaunchKernelGGL((gdp_l2norm_grad_kernel<float, 64>), grid, dim3(256), 0, stream, a);
    else return hipErrorInvalidValue;
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace gdp
