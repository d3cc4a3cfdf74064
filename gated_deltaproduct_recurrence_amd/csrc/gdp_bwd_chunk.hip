// gdp_bwd_chunk.hip -- gfx950 kernels of the chunked (matrix-core) gradients
// of the GDP prefill.
//
// The pages give no backward formulas (the blog page "Attention Cache and
// Sequence Parallelism", section "GDN: pass the state, not the KV", notes only
// that the backward dependencies run in reverse).  What is computed is the
// reverse-mode derivative of the chunked forward (FlashInfer docs,
// "flashinfer.gdp_prefill.chunk_gated_delta_product", recurrence display;
// Megatron Core API docs, core.ssm.ops.gdp.chunk, stage list), written per
// 64-row expanded chunk.  With rows r of the chunk, entering state S0, raw key
// rows k_r with norm factors rk_r (1 without the in-kernel norm), decays
// Gamma_r = 2^G_r (G the base-2 cumulative log decay inside the chunk, on each
// token's first row), Gend = Gamma of the last row, and the output tokens t
// whose last row r_t lies in the chunk:
//     Abar[r,i] = 2^(G_r - G_i) khat_r.khat_i (i < r),  T = (I + diag(beta) Abar)^-1
//     W = Khat S0,  U = V - diag(Gamma) W,  E = T diag(beta) U
//     S_end = Gend S0 + Khat^T diag(Gend / Gamma) E
//     o_t = scale (Gamma_{r_t} S0^T qhat_t + sum_{i <= r_t} 2^(G_{r_t} - G_i) (qhat_t.khat_i) e_i)
// Given D = dL/dS_end and dO, with P~[t,i] = scale 2^(G_{r_t} - G_i) qhat_t.khat_i
// (i <= r_t):
//     dE = diag(Gend / Gamma) Khat D + P~^T dO,  dU = T^T dE,  dv = diag(beta) dU
//     dA = -dU E^T (strictly lower),  Z = dO E^T,  W~ = Z masked and decayed like P~
//     dL/dS0 = Gend D - Khat^T diag(Gamma beta) dU + Qhat^T diag(scale Gamma_{r_t}) dO
//     dkhat = -diag(Gamma beta) dU S0^T + diag(Gend / Gamma) E D^T + (A~ + A~^T) Khat + W~^T Qhat
//     dqhat = diag(scale Gamma_{r_t}) dO S0^T + W~ Khat,   A~ = dA * beta_r 2^(G_r - G_i)
//     dbeta_r = dU_r.U_r + sum_i dA[r,i] Abar[r,i]
// and the derivatives by ln Gamma_r, summed from a token's first row on, give
// its dg_log:
//     -Gamma_r beta_r dU_r.W_r  + sum_i dA[r,i] A[r,i] - sum_i dA[i,r] A[i,r]
//     - (Gend / Gamma_r) X_r.E_r  (X = Khat D), and on the last row Gend <D, S0> + sum_i (Gend / Gamma_i) X_i.E_i
//     + on r_t: scale Gamma_{r_t} qhat_t.(S0 dO_t) + sum_i Z[t,i] P~[t,i];  - sum_t Z[t,r] P~[t,r]
// The gradients by q and k are the ones by their normalised rows; a later
// kernel maps them through the norm.
//
// Kernels, in launch order:
//   gdp_bwd_prep_kernel     one workgroup per (expanded chunk, k head): Gram and
//                           q.k tiles once, then per state head of the group T in
//                           fp32 (the WY inverse), stored as T^T in bf16 with
//                           P~^T and the per-row factors (the chunk's "bundle")
//   gdp_bwd_state_kernel    one workgroup per (sequence, state head), one wave per
//                           16 state columns: walks the expanded chunks forwards
//                           and stores the state entering each one (fp32)
//   gdp_bwd_adjoint_kernel  the same shape, walking backwards with D in fp32
//                           accumulators and storing D at each chunk's end; both
//                           walks load the next chunk's rows and bundle into
//                           registers while the current one is multiplied
//   gdp_bwd_grad_kernel     one workgroup per (expanded chunk, q/k head): every
//                           gradient of the chunk for each state head of the
//                           group in turn, from S0, D, the bundle and the inputs,
//                           with no sequential dependency
// Products whose operands carry D, E or dU use split bf16 operands (x = hi + lo:
// hi.hi + hi.lo + lo.hi, or hi.hi + hi.lo when the other operand is exact in
// bf16 or is T, which is kept in bf16), the others plain bf16; all on
// v_mfma_f32_16x16x32_bf16 with fp32 accumulation.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdp_common.h"
#include "gdp_launch.h"

namespace gdp {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int LDT = 72;  // row of a 64-wide bf16 plane (elements)
constexpr int LDF = 68;  // row of a 64-wide fp32 LDS tile (elements)

// per-row factor rows of the bundle (64 floats each)
enum Fac {
  F_G2 = 0,  // G_r, base-2 cumulative log decay (rows past the chunk keep the last value)
  F_C,       // rk_r 2^(Gend - G_r)
  F_D,       // 2^G_r beta_r rk_r
  F_E,       // scale 2^G_{r_t} rq_t, per output token slot t
  F_RK,      // rk_r
  F_EP,      // scale 2^G_{r_t}, per slot
  F_BETA,    // beta_r
  F_META,    // [0] Gend = 2^G_last
  F_RQ,      // rq_t, per slot
  NFAC
};

// Per (expanded chunk, state head) output of the prep kernel, copied as one
// block into the LDS of its readers.  TCM bounds the chunk's output tokens.
template <int TCM> struct Bundle {
  static constexpr int LDP = TCM + 8;
  static constexpr int PTB = 0;                       // bf16 [64][LDP]: P~^T (row i, token slot t)
  static constexpr int FAC = PTB + CH * LDP * 2;      // fp32 [NFAC][64]
  static constexpr int TTH = FAC + NFAC * CH * 4;     // bf16 [64][LDT]: T^T (row i, column r)
  static constexpr int BYTES = TTH + CH * LDT * 2;
  static_assert(BYTES % 16 == 0 && FAC % 16 == 0, "whole 16-byte segments");
};

// What the forward walk keeps of each expanded chunk and state head (the
// "state record"): W = K S0 of the raw k rows in float32, in the accumulator
// order of the gradient kernel's waves (wave w, row tile rt, lane, 4 rows), then
// S0 rounded to bfloat16, row-major [K][V].  The gradient kernel reads W into
// its registers with 16-byte loads and S0 in k-row slabs; it uses S0 only in
// bfloat16 (its products with S0 and the decay term <D, S0>).
template <int K, int V> struct StateRec {
  static constexpr int WB = CH * V * 4;          // W, float32
  static constexpr int BYTES = WB + K * V * 2;   // then S0, bfloat16
  __device__ static int w_off(int w, int rt, int lane) { return ((w * 4 + rt) * 64 + lane) * 4; }  // floats
};

struct Geo {
  int64_t t0;  // first token of the sequence
  int row0;    // first sub-token row of the chunk, relative to the sequence
  int R;       // rows in the chunk
  int tlo;     // first output token of the chunk (relative to the sequence)
  int Tc;      // output tokens (those whose last row lies in the chunk)
};

__device__ __forceinline__ int64_t cu_at(const BwdChunkArgs &a, int i) {
  const int64_t x = a.cu_is64 ? ((const int64_t *)a.cu)[i] : (int64_t)((const int32_t *)a.cu)[i];
  return x < 0 ? 0 : (x > a.T ? a.T : x);
}
__device__ __forceinline__ void seq_span(const BwdChunkArgs &a, int seq, int64_t &t0, int64_t &t1) {
  t0 = cu_at(a, seq);
  t1 = cu_at(a, seq + 1);
  if (t1 < t0) t1 = t0;
}
__device__ __forceinline__ Geo chunk_geo(int64_t t0, int64_t nsub, int n, int e) {
  Geo g;
  g.t0 = t0;
  g.row0 = CH * e;
  g.R = (int)((nsub - g.row0) < CH ? (nsub - g.row0) : CH);
  g.tlo = g.row0 / n;
  g.Tc = (g.row0 + g.R) / n - g.tlo;
  return g;
}
// the chunk of descriptor row p, or false for a padding row
__device__ __forceinline__ bool row_geo(const BwdChunkArgs &a, int64_t p, Geo &g, int &seq) {
  if (p >= a.ntdp_rows) return false;
  seq = a.chunk_indices_dp[2 * p];
  const int cc = a.chunk_indices_dp[2 * p + 1];
  if (seq < 0 || seq >= a.N || cc < 0) return false;
  int64_t t0, t1;
  seq_span(a, seq, t0, t1);
  const int64_t nsub = (t1 - t0) * a.n;
  if ((int64_t)CH * cc >= nsub) return false;
  g = chunk_geo(t0, nsub, a.n, cc);
  return true;
}

// The walks' (sequence, state head) of this workgroup.  Workgroups are dealt to
// the 8 XCDs round-robin; the remap gives each XCD a contiguous range, so that
// the state heads sharing a k head read its rows through one L2.
__device__ __forceinline__ int64_t walk_chain() {
  const int64_t G = gridDim.x, b = blockIdx.x;
  return (G % 8 == 0) ? (b % 8) * (G / 8) + b / 8 : b;
}

// ---------------------------------------------------------------- fragments
//
// v_mfma_f32_16x16x32_bf16: lane (lg = lane / 16, lr = lane % 16) supplies row
// (A) or column (B) lr and 8 reduction slots; the accumulator lane holds rows
// 4 lg .. 4 lg + 3 of column lr.  "contig" slots are k0 + 8 lg .. + 7; "perm"
// slots are k0 + 4 lg .. + 3 and k0 + 16 + 4 lg .. + 3, the row order of two
// stacked accumulator tiles, so that accumulators serve as the B operand of
// the next product without leaving registers.

__device__ __forceinline__ f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 cat(bf16x4 x, bf16x4 y) {
  return __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7);
}
// ds_read_b64_tr_b16: inside each group of 16 lanes, lane i receives element
// i % 4 of the 8-byte reads of lanes i/4, i/4 + 4, i/4 + 8 and i/4 + 12.  With
// lane j reading row r0 + j/4, columns c0 + 4 (j % 4) .. + 3, lane i receives
// rows r0 .. r0 + 3 of column c0 + i.
__device__ __forceinline__ bf16x4 tr4(const bf16 *t, int ld, int r0, int c0, int lr) {
  const char *p = (const char *)(t + (r0 + (lr >> 2)) * ld + c0 + 4 * (lr & 3));
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(p));
  return __builtin_bit_cast(bf16x4, r);
}
// operand with reduction along the rows of a row-major tile (column c0 + lr)
__device__ __forceinline__ bf16x8 tr_contig(const bf16 *t, int ld, int k0, int c0, int lr, int lg) {
  return cat(tr4(t, ld, k0 + 8 * lg, c0, lr), tr4(t, ld, k0 + 8 * lg + 4, c0, lr));
}
__device__ __forceinline__ bf16x8 tr_perm(const bf16 *t, int ld, int k0, int c0, int lr, int lg) {
  return cat(tr4(t, ld, k0 + 4 * lg, c0, lr), tr4(t, ld, k0 + 16 + 4 * lg, c0, lr));
}
// operand with reduction along a row of a row-major tile (row `row`)
__device__ __forceinline__ bf16x8 ld_contig(const bf16 *t, int ld, int row, int k0, int lg) {
  return *(const bf16x8 *)(t + row * ld + k0 + 8 * lg);
}
__device__ __forceinline__ bf16x8 ld_perm(const bf16 *t, int ld, int row, int k0, int lg) {
  const bf16 *p = t + row * ld + k0 + 4 * lg;
  return cat(*(const bf16x4 *)p, *(const bf16x4 *)(p + 16));
}
// hi/lo bf16 split of two stacked accumulator tiles (perm slots)
__device__ __forceinline__ void split_acc(bf16x8 &hi, bf16x8 &lo, f32x4 a0, f32x4 a1) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16 h0 = (bf16)a0[i], h1 = (bf16)a1[i];
    hi[i] = h0;
    hi[4 + i] = h1;
    lo[i] = (bf16)(a0[i] - (float)h0);
    lo[4 + i] = (bf16)(a1[i] - (float)h1);
  }
}
__device__ __forceinline__ uint2 pack4(f32x4 x) {
  bf16x4 h = bf16x4{(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]};
  return __builtin_bit_cast(uint2, h);
}

// DPP row moves (lanes whose source lies outside the 16-lane row read 0)
template <int CTRL> __device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
// sum over the 16 lanes of each row, left in lane 15 of the row
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp<0x111>(x);  // row_shr:1
  x += dpp<0x112>(x);  // row_shr:2
  x += dpp<0x114>(x);  // row_shr:4
  x += dpp<0x118>(x);  // row_shr:8
  return x;
}
// sum over the four lanes lr, lr + 16, lr + 32, lr + 48, in every lane: the
// gfx950 row swaps (v_permlane16_swap pairs rows 0/1 and 2/3, v_permlane32_swap
// the two halves), with no LDS traffic
__device__ __forceinline__ float col_sum4(float x) {
  const int xi = __builtin_bit_cast(int, x);
  const auto p = __builtin_amdgcn_permlane16_swap(xi, xi, false, false);
  const float y = __builtin_bit_cast(float, (int)p[0]) + __builtin_bit_cast(float, (int)p[1]);
  const int yi = __builtin_bit_cast(int, y);
  const auto q = __builtin_amdgcn_permlane32_swap(yi, yi, false, false);
  return __builtin_bit_cast(float, (int)q[0]) + __builtin_bit_cast(float, (int)q[1]);
}
// inclusive prefix sum over the 64 lanes: shifts inside each 16-lane row, then
// row 0's total into row 1 (and row 2's into row 3), then lane 31 into rows 2, 3
template <int CTRL, int ROWS> __device__ __forceinline__ float dpp_rows(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROWS, 0xF, true));
}
__device__ __forceinline__ float wave_prefix(float x) {
  x += dpp<0x111>(x);            // row_shr:1
  x += dpp<0x112>(x);            // row_shr:2
  x += dpp<0x114>(x);            // row_shr:4
  x += dpp<0x118>(x);            // row_shr:8
  x += dpp_rows<0x142, 0xA>(x);  // row_bcast:15
  x += dpp_rows<0x143, 0xC>(x);  // row_bcast:31
  return x;
}
__device__ __forceinline__ float lane63(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

// Sums over the 16 lanes of each 16-lane row of the 16 values x[4 rt + i]
// (rows 16 rt + 4 lg + i of an accumulator layout): a reduce-scatter over lane
// bits 3, 2, 1, 0 that leaves lane (lg, lr) with the sum for row
// 16 (lr >> 2) + 4 lg + (lr & 3)  (x index lr).  Every exchange is a DPP move
// inside the 16-lane row (xor 8 = row_ror:8; xor 4 from row_shl:4 / row_shr:4;
// xor 2 and xor 1 by quad_perm), so nothing goes through the LDS.
template <int CTRL> __device__ __forceinline__ float dppm(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float rowsum_scatter(float (&x)[16], int lr) {
  float y8[8];
  {
    const bool hi = lr & 8;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float keep = hi ? x[k + 8] : x[k], send = hi ? x[k] : x[k + 8];
      y8[k] = keep + dppm<0x128>(send);  // row_ror:8
    }
  }
  float y4[4];
  {
    const bool hi = lr & 4;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float keep = hi ? y8[k + 4] : y8[k], send = hi ? y8[k] : y8[k + 4];
      const float up = dppm<0x104>(send), dn = dppm<0x114>(send);  // row_shl:4, row_shr:4
      y4[k] = keep + (hi ? dn : up);
    }
  }
  float y2[2];
  {
    const bool hi = lr & 2;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const float keep = hi ? y4[k + 2] : y4[k], send = hi ? y4[k] : y4[k + 2];
      y2[k] = keep + dppm<0x4E>(send);  // quad_perm [2, 3, 0, 1]
    }
  }
  const bool hi = lr & 1;
  const float keep = hi ? y2[1] : y2[0], send = hi ? y2[0] : y2[1];
  return keep + dppm<0xB1>(send);  // quad_perm [1, 0, 3, 2]
}

// A row-major tile of ROWS rows of D bf16 columns (row stride rs elements) in
// 16-byte pieces, thread tid holding pieces tid + j NTH between their global
// loads and their LDS stores.  The loads are unconditional -- a piece of a row
// past the valid ones reads the last valid row, and the store writes zeros
// there -- so that issuing them never waits.
template <int ROWS, int D, int NTH> struct TileRegs {
  static constexpr int SEG = D / 8, N = ROWS * SEG, J = (N + NTH - 1) / NTH;
  u32x4 x[J];
  __device__ __forceinline__ void load(const bf16 *src, int64_t rs, int nvalid, int tid) {
    const int last = nvalid > 0 ? nvalid - 1 : 0;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int u = (N % NTH == 0 || tid + j * NTH < N) ? tid + j * NTH : N - 1;
      const int r = u / SEG, s = u % SEG;
      x[j] = *(const u32x4 *)(src + (int64_t)(r < last ? r : last) * rs + 8 * s);
    }
  }
  template <int LD> __device__ __forceinline__ void store(bf16 *dst, int nvalid, int tid) const {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int u = tid + j * NTH;
      if (N % NTH == 0 || u < N) {
        const int r = u / SEG, s = u % SEG;
        const u32x4 z = {0u, 0u, 0u, 0u};
        *(u32x4 *)(dst + r * LD + 8 * s) = r < nvalid ? x[j] : z;
      }
    }
  }
};
// a contiguous block of BYTES bytes, the same way
template <int BYTES, int NTH> struct BlockRegs {
  static constexpr int N = BYTES / 16, J = (N + NTH - 1) / NTH;
  u32x4 x[J];
  __device__ __forceinline__ void load(const char *src, int tid) {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int u = (N % NTH == 0 || tid + j * NTH < N) ? tid + j * NTH : N - 1;
      x[j] = *(const u32x4 *)(src + 16 * u);
    }
  }
  __device__ __forceinline__ void store(char *dst, int tid) const {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int u = tid + j * NTH;
      if (N % NTH == 0 || u < N) *(u32x4 *)(dst + 16 * u) = x[j];
    }
  }
};
// 1/sqrt(sum x^2 + 1e-6) of `rows` LDS rows of width D; 4 threads per row
template <int D>
__device__ __forceinline__ void rows_rsq(const bf16 *base, int ld, int rows, float *out, int tid, int nth) {
  for (int u = tid; u < 4 * rows; u += nth) {
    const int row = u >> 2, part = u & 3;
    float ss = 0.f;
#pragma unroll 8
    for (int e = part * (D / 4); e < (part + 1) * (D / 4); ++e) {
      const float x = (float)base[row * ld + e];
      ss += x * x;
    }
    ss += __shfl_xor(ss, 1, 64);
    ss += __shfl_xor(ss, 2, 64);
    if (part == 0) out[row] = 1.0f / sqrtf(ss + 1e-6f);
  }
}

// ---------------------------------------------------------------- prep kernel

template <int K, int TCM> struct PrepSmem {
  static constexpr int LDK = K + 8;
  union {
    struct {
      bf16 k[CH * LDK];
      bf16 q[TCM * LDK];
    } rows;  // raw k and q rows, until the Gram and q.k tiles are in registers
    struct {
      float a[CH * LDF];   // A = diag(beta) Abar
      float tf[CH * LDF];  // T
    } wy;                  // per state head
  } u;
  float rk[CH], rq[TCM], g2[CH], beta[CH];
};

template <int K, int TCM>
__global__ void __launch_bounds__(NTHR) gdp_bwd_prep_kernel(BwdChunkArgs a) {
  using S = PrepSmem<K, TCM>;
  using B = Bundle<TCM>;
  constexpr int LDK = S::LDK, KS = K / 32, LDP = B::LDP, NQT = 4 * (TCM / 16), QPW = NQT / 4;
  __shared__ __attribute__((aligned(16))) S sm;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, lr = lane & 15, lg = lane >> 4;
  const int64_t p = blockIdx.x / a.Hk;
  const int hk = (int)(blockIdx.x % a.Hk);
  Geo g;
  int seq;
  if (!row_geo(a, p, g, seq)) return;
  const int n = a.n, grp = a.Hv / a.Hk;
  const int hq = (hk * grp) / (a.Hv / a.Hqk);  // the q head of every state head of the group
  {
    TileRegs<CH, K, NTHR> kr;
    TileRegs<TCM, K, NTHR> qr;
    kr.load((const bf16 *)a.k + hk * a.k_sh + (g.t0 * n + g.row0) * a.k_st, a.k_st, g.R, tid);
    qr.load((const bf16 *)a.q + hq * a.q_sh + (g.t0 + g.tlo) * a.q_st, a.q_st, g.Tc, tid);
    kr.template store<LDK>(sm.u.rows.k, g.R, tid);
    qr.template store<LDK>(sm.u.rows.q, g.Tc, tid);
  }
  __syncthreads();
  if (a.l2norm) {
    rows_rsq<K>(sm.u.rows.k, LDK, CH, sm.rk, tid, NTHR);
    rows_rsq<K>(sm.u.rows.q, LDK, TCM, sm.rq, tid, NTHR);
  } else {
    if (tid < CH) sm.rk[tid] = 1.f;
    if (tid < TCM) sm.rq[tid] = 1.f;
  }
  // Gram tiles (the 10 lower 16 x 16 tiles, wave w holding tiles w, w + 4, w + 8)
  // and q.k tiles of the raw rows, kept in registers for every state head
  f32x4 gram[3], qk[QPW];
#pragma unroll
  for (int it = 0; it < 3; ++it) {
    const int idx = w + 4 * it;
    gram[it] = zero4();
    if (idx < 10) {
      const int ra = idx < 1 ? 0 : (idx < 3 ? 1 : (idx < 6 ? 2 : 3)), rb = idx - ra * (ra + 1) / 2;
#pragma unroll
      for (int s = 0; s < KS; ++s)
        gram[it] = mma(ld_contig(sm.u.rows.k, LDK, 16 * ra + lr, 32 * s, lg),
                       ld_contig(sm.u.rows.k, LDK, 16 * rb + lr, 32 * s, lg), gram[it]);
    }
  }
#pragma unroll
  for (int it = 0; it < QPW; ++it) {
    const int idx = w + 4 * it, ta = idx >> 2, ib = idx & 3;
    qk[it] = zero4();
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qk[it] = mma(ld_contig(sm.u.rows.q, LDK, 16 * ta + lr, 32 * s, lg),
                   ld_contig(sm.u.rows.k, LDK, 16 * ib + lr, 32 * s, lg), qk[it]);
  }
  const float scale = a.scale;
  for (int hh = 0; hh < grp; ++hh) {
    const int h = hk * grp + hh;
    __syncthreads();  // the rows (first head) or the previous head's T, g2, beta are no longer read
    if (w == 0) {
      const int r = lane;
      float gl = 0.f, bt = 0.f;
      if (r < g.R) {
        const int64_t row = g.t0 * n + g.row0 + r;
        bt = a.beta[row * a.b_st + h * a.b_sh];
        if ((g.row0 + r) % n == 0) gl = a.g[(g.t0 + (g.row0 + r) / n) * a.g_st + h * a.g_sh] * LOG2E;
      }
      gl = wave_prefix(gl);
      sm.g2[r] = gl;
      sm.beta[r] = bt;
    }
    __syncthreads();
    // A (the strictly lower part of the lower tiles; wy_inverse reads nothing else)
#pragma unroll
    for (int it = 0; it < 3; ++it) {
      const int idx = w + 4 * it;
      if (idx < 10) {
        const int ra = idx < 1 ? 0 : (idx < 3 ? 1 : (idx < 6 ? 2 : 3)), rb = idx - ra * (ra + 1) / 2;
        const int i = 16 * rb + lr;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 16 * ra + 4 * lg + j;
          sm.u.wy.a[r * LDF + i] = (i < r && r < g.R)
                                       ? sm.beta[r] * exp2f(sm.g2[r] - sm.g2[i]) * sm.rk[r] * sm.rk[i] * gram[it][j]
                                       : 0.f;
        }
      }
    }
    __syncthreads();
    wy_inverse<LDF>(sm.u.wy.a, sm.u.wy.tf, tid);
    char *out = a.bundle + ((size_t)p * a.Hv + h) * B::BYTES;
    // T^T plane: row i, columns r (8 per thread and step)
    for (int u = tid; u < CH * (LDT / 8); u += NTHR) {
      const int i = u / (LDT / 8), r0 = 8 * (u % (LDT / 8));
      bf16x8 hi;
#pragma unroll
      for (int j = 0; j < 8; ++j) hi[j] = (bf16)((r0 + j < CH) ? sm.u.wy.tf[(r0 + j) * LDF + i] : 0.f);
      *(bf16x8 *)(out + B::TTH + 2 * (i * LDT + r0)) = hi;
    }
    // P~^T (row i, token slots t) from the q.k tiles: lane holds 4 consecutive slots of one row i
#pragma unroll
    for (int it = 0; it < QPW; ++it) {
      const int idx = w + 4 * it, ta = idx >> 2, ib = idx & 3;
      const int i = 16 * ib + lr;
      bf16x4 x;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = 16 * ta + 4 * lg + j;
        float y = 0.f;
        if (t < g.Tc && i < g.R) {
          const int rt = (g.tlo + t) * n + n - 1 - g.row0;
          if (i <= rt) y = scale * sm.rq[t] * sm.rk[i] * exp2f(sm.g2[rt] - sm.g2[i]) * qk[it][j];
        }
        x[j] = (bf16)y;
      }
      *(bf16x4 *)(out + B::PTB + 2 * (i * LDP + 16 * ta + 4 * lg)) = x;
    }
    // factor rows
    float *fac = (float *)(out + B::FAC);
    if (tid < CH) {
      const int r = tid;
      const bool in = r < g.R;
      const float gend = sm.g2[g.R - 1], gr = sm.g2[r];
      fac[F_G2 * CH + r] = in ? gr : gend;
      fac[F_C * CH + r] = in ? sm.rk[r] * exp2f(gend - gr) : 0.f;
      fac[F_D * CH + r] = in ? exp2f(gr) * sm.beta[r] * sm.rk[r] : 0.f;
      fac[F_RK * CH + r] = in ? sm.rk[r] : 0.f;
      fac[F_BETA * CH + r] = in ? sm.beta[r] : 0.f;
      fac[F_META * CH + r] = r == 0 ? exp2f(gend) : 0.f;
      const int t = r;
      const bool tin = t < g.Tc;
      const int rt = (g.tlo + t) * n + n - 1 - g.row0;
      const float ep = tin ? scale * exp2f(sm.g2[rt < CH ? rt : CH - 1]) : 0.f;
      fac[F_EP * CH + t] = ep;
      fac[F_E * CH + t] = tin ? ep * sm.rq[t < TCM ? t : 0] : 0.f;
      fac[F_RQ * CH + t] = tin ? sm.rq[t < TCM ? t : 0] : 0.f;
    }
  }
}

// ---------------------------------------------------------------- state kernel

template <int K, int V, int TCM> struct FwdSmem {
  static constexpr int LDK = K + 8, LDV = V + 8;
  bf16 k[CH * LDK];
  bf16 v[CH * LDV];
  char bundle[Bundle<TCM>::BYTES];
};

// the next chunk's k and v rows and bundle, in registers between their loads
// and their LDS stores
template <int K, int V, int TCM, int NTH> struct FwdStage {
  TileRegs<CH, K, NTH> k;
  TileRegs<CH, V, NTH> v;
  // the factor rows and T^T (the forward walk does not read the scores P~^T)
  static constexpr int B0 = Bundle<TCM>::FAC;
  BlockRegs<Bundle<TCM>::BYTES - B0, NTH> b;
  int R;
  __device__ __forceinline__ void load(const BwdChunkArgs &a, const Geo &g, int64_t p, int h, int hk, int tid) {
    R = g.R;
    k.load((const bf16 *)a.k + hk * a.k_sh + (g.t0 * a.n + g.row0) * a.k_st, a.k_st, g.R, tid);
    v.load((const bf16 *)a.v + h * a.v_sh + (g.t0 * a.n + g.row0) * a.v_st, a.v_st, g.R, tid);
    b.load(a.bundle + ((size_t)p * a.Hv + h) * Bundle<TCM>::BYTES + B0, tid);
  }
  __device__ __forceinline__ void commit(FwdSmem<K, V, TCM> &sm, int tid) const {
    k.template store<FwdSmem<K, V, TCM>::LDK>(sm.k, R, tid);
    v.template store<FwdSmem<K, V, TCM>::LDV>(sm.v, R, tid);
    b.store(sm.bundle + B0, tid);
  }
};

// The state entering every expanded chunk, walking each chain forwards:
//     W = K S,  E = T diag(beta) (V - diag(Gamma rk) W),  S <- Gend S + K^T diag(c) E
// with every product on split operands (S, E, T hi/lo; raw k and v rows are
// exact in bf16), so the states carry fp32-level error into the gradients.
template <int K, int V, int TCM>
__global__ void __launch_bounds__(V * 4, 1) gdp_bwd_state_kernel(BwdChunkArgs a) {
  constexpr int NW = V / 16, NTH = 64 * NW, KT = K / 16, KS = K / 32;
  using S = FwdSmem<K, V, TCM>;
  using B = Bundle<TCM>;
  using SR = StateRec<K, V>;
  constexpr int LDK = S::LDK, LDV = S::LDV;
  __shared__ __attribute__((aligned(16))) S sm;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, lr = lane & 15, lg = lane >> 4;
  const int64_t chain = walk_chain();
  const int seq = (int)(chain / a.Hv), h = (int)(chain % a.Hv);
  if (seq >= a.N) return;
  const int hk = h / (a.Hv / a.Hk);
  int64_t t0, t1;
  seq_span(a, seq, t0, t1);
  const int64_t nsub = (t1 - t0) * a.n;
  const int64_t p0 = a.chunk_offsets_dp[seq];
  int nexp = (int)((nsub + CH - 1) / CH);
  if (p0 < 0) nexp = 0;
  else if (p0 + nexp > a.ntdp_rows) nexp = (int)(a.ntdp_rows > p0 ? a.ntdp_rows - p0 : 0);
  const int col = 16 * w + lr;
  const size_t KV = (size_t)K * V;

  f32x4 Sa[KT];
  {
    const float *s0 = a.s0 ? a.s0 + ((size_t)seq * a.Hv + h) * KV : nullptr;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) Sa[kt][i] = s0 ? s0[(size_t)(16 * kt + 4 * lg + i) * V + col] : 0.f;
  }
  FwdStage<K, V, TCM, NTH> st;
  if (nexp > 0) {
    st.load(a, chunk_geo(t0, nsub, a.n, 0), p0, h, hk, tid);
    st.commit(sm, tid);
  }
  __syncthreads();
  const bf16 *tth = (const bf16 *)(sm.bundle + B::TTH);
  const float *fac = (const float *)(sm.bundle + B::FAC);
  for (int e = 0; e < nexp; ++e) {
    if (e + 1 < nexp) st.load(a, chunk_geo(t0, nsub, a.n, e + 1), p0 + e + 1, h, hk, tid);
    char *rec = (char *)a.states + ((size_t)(p0 + e) * a.Hv + h) * SR::BYTES;
    {
      bf16 *dst = (bf16 *)(rec + SR::WB);
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[(size_t)(16 * kt + 4 * lg + i) * V + col] = (bf16)Sa[kt][i];
    }
    // W = K S (S split), stored, then Ut = beta (V - Gamma rk W)
    f32x4 X[4];
    {
      bf16x8 Sh[KS], Sl[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) split_acc(Sh[s], Sl[s], Sa[2 * s], Sa[2 * s + 1]);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        X[rt] = zero4();
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const bf16x8 kf = ld_perm(sm.k, LDK, 16 * rt + lr, 32 * s, lg);
          X[rt] = mma(kf, Sh[s], X[rt]);
          X[rt] = mma(kf, Sl[s], X[rt]);
        }
        *(f32x4 *)((float *)rec + SR::w_off(w, rt, lane)) = X[rt];
        const bf16x4 vv = tr4(sm.v, LDV, 16 * rt + 4 * lg, 16 * w, lr);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * rt + 4 * lg + i;
          X[rt][i] = fac[F_BETA * CH + r] * ((float)vv[i] - exp2f(fac[F_G2 * CH + r]) * fac[F_RK * CH + r] * X[rt][i]);
        }
      }
    }
    // E = T Ut (Ut split), scaled by c
    f32x4 E[4];
    {
      bf16x8 Uh[2], Ul[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) split_acc(Uh[s], Ul[s], X[2 * s], X[2 * s + 1]);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        E[rt] = zero4();
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const bf16x8 ah = tr_perm(tth, LDT, 32 * s, 16 * rt, lr, lg);
          E[rt] = mma(ah, Uh[s], E[rt]);
          E[rt] = mma(ah, Ul[s], E[rt]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) E[rt][i] *= fac[F_C * CH + 16 * rt + 4 * lg + i];
      }
    }
    // S = Gend S + K^T (c E)
    {
      bf16x8 Eh[2], El[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) split_acc(Eh[s], El[s], E[2 * s], E[2 * s + 1]);
      const float gend = fac[F_META * CH];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        Sa[kt] *= gend;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const bf16x8 kf = tr_perm(sm.k, LDK, 32 * s, 16 * kt, lr, lg);
          Sa[kt] = mma(kf, Eh[s], Sa[kt]);
          Sa[kt] = mma(kf, El[s], Sa[kt]);
        }
      }
    }
    if (e + 1 < nexp) {
      __syncthreads();
      st.commit(sm, tid);
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------- adjoint kernel

template <int K, int V, int TCM> struct AdjSmem {
  static constexpr int LDK = K + 8, LDO = V + 8;
  bf16 k[CH * LDK];
  bf16 q[TCM * LDK];
  bf16 o[TCM * LDO];
  char bundle[Bundle<TCM>::BYTES];
};

// the next chunk's k, q, dO rows and bundle, in registers between their loads
// and their LDS stores
template <int K, int V, int TCM, int NTH> struct AdjStage {
  TileRegs<CH, K, NTH> k;
  TileRegs<TCM, K, NTH> q;
  TileRegs<TCM, V, NTH> o;
  BlockRegs<Bundle<TCM>::BYTES, NTH> b;
  int R, Tc;
  __device__ __forceinline__ void load(const BwdChunkArgs &a, const Geo &g, int64_t p, int h, int hk, int hq, int tid) {
    R = g.R;
    Tc = g.Tc;
    k.load((const bf16 *)a.k + hk * a.k_sh + (g.t0 * a.n + g.row0) * a.k_st, a.k_st, g.R, tid);
    q.load((const bf16 *)a.q + hq * a.q_sh + (g.t0 + g.tlo) * a.q_st, a.q_st, g.Tc, tid);
    o.load((const bf16 *)a.dout + h * a.do_sh + (g.t0 + g.tlo) * a.do_st, a.do_st, g.Tc, tid);
    b.load(a.bundle + ((size_t)p * a.Hv + h) * Bundle<TCM>::BYTES, tid);
  }
  __device__ __forceinline__ void commit(AdjSmem<K, V, TCM> &sm, int tid) const {
    k.template store<AdjSmem<K, V, TCM>::LDK>(sm.k, R, tid);
    q.template store<AdjSmem<K, V, TCM>::LDK>(sm.q, Tc, tid);
    o.template store<AdjSmem<K, V, TCM>::LDO>(sm.o, Tc, tid);
    b.store(sm.bundle, tid);
  }
};

template <int K, int V, int TCM>
__global__ void __launch_bounds__(V * 4, 1) gdp_bwd_adjoint_kernel(BwdChunkArgs a) {
  constexpr int NW = V / 16, NTH = 64 * NW, KT = K / 16, KS = K / 32, TS = TCM / 32;
  using S = AdjSmem<K, V, TCM>;
  using B = Bundle<TCM>;
  constexpr int LDK = S::LDK, LDO = S::LDO, LDP = B::LDP;
  __shared__ __attribute__((aligned(16))) S sm;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, lr = lane & 15, lg = lane >> 4;
  const int64_t chain = walk_chain();
  const int seq = (int)(chain / a.Hv), h = (int)(chain % a.Hv);
  if (seq >= a.N) return;
  const int hk = h / (a.Hv / a.Hk), hq = h / (a.Hv / a.Hqk);
  int64_t t0, t1;
  seq_span(a, seq, t0, t1);
  const int64_t nsub = (t1 - t0) * a.n;
  const int64_t p0 = a.chunk_offsets_dp[seq];
  int nexp = (int)((nsub + CH - 1) / CH);
  // (descriptor rows past the capacity, from cu_seqlens contents the descriptor
  // pass did not clamp, are neither read nor written)
  if (p0 < 0) nexp = 0;
  else if (p0 + nexp > a.ntdp_rows) nexp = (int)(a.ntdp_rows > p0 ? a.ntdp_rows - p0 : 0);
  const int col = 16 * w + lr;
  const size_t KV = (size_t)K * V;

  f32x4 D[KT];
  {
    const float *df = a.dfinal ? a.dfinal + ((size_t)seq * a.Hv + h) * KV : nullptr;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) D[kt][i] = df ? df[(size_t)(16 * kt + 4 * lg + i) * V + col] : 0.f;
  }
  AdjStage<K, V, TCM, NTH> st;
  if (nexp > 0) {
    st.load(a, chunk_geo(t0, nsub, a.n, nexp - 1), p0 + nexp - 1, h, hk, hq, tid);
    st.commit(sm, tid);
  }
  __syncthreads();
  const bf16 *tth = (const bf16 *)(sm.bundle + B::TTH);
  const bf16 *ptb = (const bf16 *)(sm.bundle + B::PTB);
  const float *fac = (const float *)(sm.bundle + B::FAC);
  for (int e = nexp - 1; e >= 0; --e) {
    if (e > 0) st.load(a, chunk_geo(t0, nsub, a.n, e - 1), p0 + e - 1, h, hk, hq, tid);
    {  // dL/d(state leaving chunk e), for the gradient kernel
      float *dd = a.dstates + ((size_t)(p0 + e) * a.Hv + h) * KV;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) dd[(size_t)(16 * kt + 4 * lg + i) * V + col] = D[kt][i];
    }
    // X = K D (raw k rows, D split)
    f32x4 X[4];
    {
      bf16x8 Dh[KS], Dl[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) split_acc(Dh[s], Dl[s], D[2 * s], D[2 * s + 1]);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        X[rt] = zero4();
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const bf16x8 kf = ld_perm(sm.k, LDK, 16 * rt + lr, 32 * s, lg);
          X[rt] = mma(kf, Dh[s], X[rt]);
          X[rt] = mma(kf, Dl[s], X[rt]);
        }
      }
    }
    // dE = c X + P~^T dO
    bf16x8 of[TS];
#pragma unroll
    for (int s = 0; s < TS; ++s) of[s] = tr_contig(sm.o, LDO, 32 * s, 16 * w, lr, lg);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) X[rt][i] *= fac[F_C * CH + 16 * rt + 4 * lg + i];
#pragma unroll
      for (int s = 0; s < TS; ++s) X[rt] = mma(ld_contig(ptb, LDP, 16 * rt + lr, 32 * s, lg), of[s], X[rt]);
    }
    // dU = T^T dE (dE split), then dW' = -d dU
    f32x4 U[4];
    {
      bf16x8 Eh[2], El[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) split_acc(Eh[s], El[s], X[2 * s], X[2 * s + 1]);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        U[rt] = zero4();
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const bf16x8 ah = ld_perm(tth, LDT, 16 * rt + lr, 32 * s, lg);
          U[rt] = mma(ah, Eh[s], U[rt]);
          U[rt] = mma(ah, El[s], U[rt]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) U[rt][i] *= -fac[F_D * CH + 16 * rt + 4 * lg + i];
      }
    }
    // D = Gend D + K^T dW' + Q^T diag(e) dO
    {
      bf16x8 Wh[2], Wl[2], eo[TS];
#pragma unroll
      for (int s = 0; s < 2; ++s) split_acc(Wh[s], Wl[s], U[2 * s], U[2 * s + 1]);
#pragma unroll
      for (int s = 0; s < TS; ++s)
#pragma unroll
        for (int j = 0; j < 8; ++j) eo[s][j] = (bf16)((float)of[s][j] * fac[F_E * CH + 32 * s + 8 * lg + j]);
      const float gend = fac[F_META * CH];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        D[kt] *= gend;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const bf16x8 kf = tr_perm(sm.k, LDK, 32 * s, 16 * kt, lr, lg);
          D[kt] = mma(kf, Wh[s], D[kt]);
          D[kt] = mma(kf, Wl[s], D[kt]);
        }
#pragma unroll
        for (int s = 0; s < TS; ++s) D[kt] = mma(tr_contig(sm.q, LDK, 32 * s, 16 * kt, lr, lg), eo[s], D[kt]);
      }
    }
    if (e > 0) {
      __syncthreads();
      st.commit(sm, tid);
      __syncthreads();
    }
  }
  if (a.ds0) {
    float *d0 = a.ds0 + ((size_t)seq * a.Hv + h) * KV;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) d0[(size_t)(16 * kt + 4 * lg + i) * V + col] = D[kt][i];
  }
}

// ---------------------------------------------------------------- gradient kernel

// Store the rows [0, nvalid) of a gradient held as 16-column tiles (tile kt =
// w + m NW of wave w, rows 16 rt + 4 lg + i in accumulator layout) by the
// normalised rows of a raw bf16 tile x (LDS, row stride ldx) with norm factors
// rn: with the in-kernel norm, g_raw = rn (g - xhat (xhat.g)), xhat = rn x; the
// row dots go through `dots` (64 zeroed floats, read after a barrier).  Called
// by every thread of the workgroup.
template <int NKW, int NRT, int K>
__device__ __forceinline__ void store_rows(float *out, int64_t row0, int64_t st, int64_t head_off, int nvalid,
                                           f32x4 (&acc)[NKW][NRT], const bf16 *x, int ldx, const float *rn, float *dots,
                                           int l2norm, int w, int NW, int lr, int lg) {
  constexpr int KT = K / 16;
  if (l2norm) {
#pragma unroll
    for (int m = 0; m < NKW; ++m) {
      const int kt = w + m * NW;
      if (kt >= KT) continue;
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * rt + 4 * lg + i;
          const float d = row_sum16(acc[m][rt][i] * (float)x[r * ldx + 16 * kt + lr]);
          if (lr == 15) atomicAdd(dots + r, d);
        }
    }
    __syncthreads();
  }
  float *ol = out + (row0 + 4 * lg) * st + head_off + lr;
#pragma unroll
  for (int m = 0; m < NKW; ++m) {
    const int kt = w + m * NW;
    if (kt >= KT) continue;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * rt + 4 * lg + i;
        float y = acc[m][rt][i];
        if (l2norm) {
          const float f = rn[r];
          y = f * (y - f * f * (float)x[r * ldx + 16 * kt + lr] * dots[r]);
        }
        if (r < nvalid) ol[(16 * rt + i) * st + 16 * kt] = y;
      }
  }
}

// row partial sums of the gradient kernel (per state head), and the row dots
// of the norm gradients (per workgroup)
enum Red { R_DB = 0, R_DL, R_XE, R_DS, R_QN, R_KN, NRED };

template <int K, int V, int TCM> struct GradLds {
  using B = Bundle<TCM>;
  static constexpr int LDK = K + 8, LDO = V + 8, LDV = V + 8, LDW = TCM + 8;
  static constexpr int K_ = 0;                               // bf16 [64][LDK] raw k rows
  static constexpr int Q_ = K_ + CH * LDK * 2;               // bf16 [TCM][LDK] raw q rows
  static constexpr int O_ = Q_ + TCM * LDK * 2;              // bf16 [TCM][LDO] dO rows
  static constexpr int AB = O_ + TCM * LDO * 2;              // fp32 [64][LDF] Abar, then A~
  static constexpr int RD = AB + CH * LDF * 4;               // fp32 [NRED][64]
  static constexpr int SL = RD + NRED * CH * 4;              // fp32 [3][V / 16][64]: per-wave row partials
  static constexpr int BU = SL + 3 * (V / 16) * CH * 4;      // the bundle
  // the rest lies over the bundle's T^T planes, which are dead once dU is formed:
  static constexpr int PL = BU + B::TTH;
  static constexpr int VR = PL + CH * LDT * 2;               // bf16 [64][LDV] v rows (until U is formed)
  static constexpr int EH = PL, EL = EH + V * LDT * 2, UH = EL + V * LDT * 2, UL = UH + V * LDT * 2;  // E^T, dU^T [v][r]
  static constexpr int P1_END = UL + V * LDT * 2;
  static constexpr int MH = PL, ML = MH + CH * LDT * 2;      // M' = (A~ + A~^T) diag(rk), [r][i]
  static constexpr int W1 = ML + CH * LDT * 2;               // W~ diag(rq), stored [i][t]
  static constexpr int W2 = W1 + CH * LDW * 2;               // diag(rk) W~^T, stored [i][t]
  static constexpr int P2_END = W2 + CH * LDW * 2;
  static constexpr int V_END = VR + CH * LDV * 2;
  static constexpr int M1 = P1_END > P2_END ? P1_END : P2_END, M2 = V_END > BU + B::BYTES ? V_END : BU + B::BYTES;
  static constexpr int GR = M1 > M2 ? M1 : M2;                // fp32 [10][64 lanes][4]: raw Gram tiles,
  static constexpr bool KEEP_GRAM = GR + 10 * 64 * 4 * 4 <= 160 * 1024;  // where they fit
  static constexpr int BYTES = KEEP_GRAM ? GR + 10 * 64 * 4 * 4 : GR;
  static_assert(BYTES <= 160 * 1024, "LDS of one workgroup");
};

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }  // v_exp_f32

// One workgroup per (expanded chunk, q/k head): the state heads of the group in
// turn, each wave owning 16 state columns for the products over rows and one or
// more 16-column k tiles for the products over V.  dq (and dk when the group
// shares its k rows) accumulate in registers over the heads and are stored
// once, through the L2-norm gradient when the in-kernel norm is on; the next
// head's slabs, rows and bundle are loaded while the current head finishes.
template <int K, int V, int TCM>
__global__ void __launch_bounds__(V * 4, 1) gdp_bwd_grad_kernel(BwdChunkArgs a) {
  constexpr int NW = V / 16, NTH = 64 * NW, KT = K / 16, KS = K / 32, VS = V / 32, TS = TCM / 32, TT16 = TCM / 16;
  constexpr int NKW = (KT + NW - 1) / NW;
  using L = GradLds<K, V, TCM>;
  using B = Bundle<TCM>;
  using SR = StateRec<K, V>;
  constexpr int LDK = L::LDK, LDO = L::LDO, LDV = L::LDV, LDP = B::LDP, LDW = L::LDW;
  __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
  bf16 *sk = (bf16 *)(smem + L::K_), *sq = (bf16 *)(smem + L::Q_), *so = (bf16 *)(smem + L::O_);
  bf16 *sv = (bf16 *)(smem + L::VR);
  float *abar = (float *)(smem + L::AB), *red = (float *)(smem + L::RD), *slots = (float *)(smem + L::SL);
  const bf16 *tth = (const bf16 *)(smem + L::BU + B::TTH);
  const bf16 *ptb = (const bf16 *)(smem + L::BU + B::PTB);
  const float *fac = (const float *)(smem + L::BU + B::FAC);
  bf16 *peh = (bf16 *)(smem + L::EH), *pel = (bf16 *)(smem + L::EL), *puh = (bf16 *)(smem + L::UH),
       *pul = (bf16 *)(smem + L::UL);
  bf16 *pmh = (bf16 *)(smem + L::MH), *pml = (bf16 *)(smem + L::ML), *pw1 = (bf16 *)(smem + L::W1),
       *pw2 = (bf16 *)(smem + L::W2);

  int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: w-derived offsets stay scalar
  const int64_t p = blockIdx.x / a.Hqk;
  const int hq = (int)(blockIdx.x % a.Hqk);
  Geo g;
  int seq;
  if (!row_geo(a, p, g, seq)) return;
  const int n = a.n, G = a.Hv / a.Hqk;
  const bool kshared = a.Hk == a.Hqk;  // else one k head per state head
  const int64_t krow0 = g.t0 * n + g.row0;  // first k/v/beta row of the chunk
  const int64_t qrow0 = g.t0 + g.tlo;       // first output token
  const size_t KV = (size_t)K * V;
  int lane = tid & 63, lr = lane & 15, lg = lane >> 4, col = 16 * w + lr;

  // head-dependent operands: W = K S0 and the D slab (this wave's 16 columns,
  // accumulator layout) in registers; dO rows, v rows, bundle (and k rows when
  // not shared) staged through registers into LDS
  f32x4 Wa[4], Da[KT];
  TileRegs<CH, K, NTH> kr;
  TileRegs<TCM, V, NTH> orr;
  TileRegs<CH, V, NTH> vr;
  BlockRegs<B::BYTES, NTH> br;
  auto load_rows = [&](int h, bool with_k) {
    const int hk = h / (a.Hv / a.Hk);
    if (with_k) kr.load((const bf16 *)a.k + hk * a.k_sh + krow0 * a.k_st, a.k_st, g.R, tid);
    orr.load((const bf16 *)a.dout + h * a.do_sh + qrow0 * a.do_st, a.do_st, g.Tc, tid);
    br.load(a.bundle + ((size_t)p * a.Hv + h) * B::BYTES, tid);
    vr.load((const bf16 *)a.v + h * a.v_sh + krow0 * a.v_st, a.v_st, g.R, tid);
  };
  auto load_slabs = [&](int h) {
    const float *Wg = (const float *)((const char *)a.states + ((size_t)p * a.Hv + h) * SR::BYTES);
    const float *Dg = a.dstates + ((size_t)p * a.Hv + h) * KV + (size_t)(4 * lg) * V + col;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) Wa[rt] = *(const f32x4 *)(Wg + SR::w_off(w, rt, lane));
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) Da[kt][i] = Dg[(16 * kt + i) * V];
  };
  auto commit_head = [&](bool with_k) {
    if (with_k) kr.template store<LDK>(sk, g.R, tid);
    orr.template store<LDO>(so, g.Tc, tid);
    br.store(smem + L::BU, tid);
    vr.template store<LDV>(sv, g.R, tid);
    for (int u = tid; u < 4 * CH; u += NTH) red[u] = 0.f;  // R_DB .. R_DS
    if (tid < CH) red[R_KN * CH + tid] = 0.f;              // (the k-row dots when dk is stored per head)
  };
  {
    TileRegs<TCM, K, NTH> qr;
    qr.load((const bf16 *)a.q + hq * a.q_sh + qrow0 * a.q_st, a.q_st, g.Tc, tid);
    load_rows(hq * G, true);
    load_slabs(hq * G);
    qr.template store<LDK>(sq, g.Tc, tid);
    commit_head(true);
    if (tid < CH) red[R_QN * CH + tid] = 0.f;
  }
  f32x4 dK[NKW][4], dQ[NKW][TT16];
#pragma unroll
  for (int m = 0; m < NKW; ++m) {
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) dK[m][rt] = zero4();
#pragma unroll
    for (int ta = 0; ta < TT16; ++ta) dQ[m][ta] = zero4();
  }
  const float scale = a.scale;

#pragma unroll 1
  for (int j = 0; j < G; ++j) {
    const int h = hq * G + j;
    // the lane index is made opaque every head so that the compiler forms each
    // LDS address where it is used instead of keeping dozens of them live
    tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    lane = tid & 63;
    lr = lane & 15;
    lg = lane >> 4;
    col = 16 * w + lr;
    const bf16 *S0g = (const bf16 *)((const char *)a.states + ((size_t)p * a.Hv + h) * SR::BYTES + SR::WB);
    const float *Dg = a.dstates + ((size_t)p * a.Hv + h) * KV;
    __syncthreads();  // this head's rows, bundle and zeroed partial sums are in LDS

    // Abar (strictly lower) from the Gram tiles of the raw rows.  When the group's
    // state heads share the k rows, the tiles of the first head are kept (each by
    // the lane that formed it, so no barrier is needed) and the later heads only
    // rescale them.
    for (int idx = w; idx < 10; idx += NW) {
      const int ra = idx < 1 ? 0 : (idx < 3 ? 1 : (idx < 6 ? 2 : 3));
      const int rb = idx - ra * (ra + 1) / 2;
      f32x4 acc = zero4();
      f32x4 *gsave = (f32x4 *)(smem + L::GR) + idx * 64 + lane;
      if (!L::KEEP_GRAM || j == 0 || !kshared) {
#pragma unroll
        for (int s = 0; s < KS; ++s)
          acc = mma(ld_contig(sk, LDK, 16 * ra + lr, 32 * s, lg), ld_contig(sk, LDK, 16 * rb + lr, 32 * s, lg), acc);
        if (L::KEEP_GRAM && kshared) *gsave = acc;
      } else {
        acc = *gsave;
      }
      const int i = 16 * rb + lr;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r = 16 * ra + 4 * lg + jj;
        abar[r * LDF + i] = (i < r && r < g.R) ? fexp2(fac[F_G2 * CH + r] - fac[F_G2 * CH + i]) * fac[F_RK * CH + r] *
                                                      fac[F_RK * CH + i] * acc[jj]
                                                : 0.f;
      }
    }
    // W = K S0 from the forward walk; X = K D (D split)
    f32x4 *W = Wa, X[4];
    {
      bf16x8 Dh[KS], Dl[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) split_acc(Dh[s], Dl[s], Da[2 * s], Da[2 * s + 1]);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        X[rt] = zero4();
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const bf16x8 kf = ld_perm(sk, LDK, 16 * rt + lr, 32 * s, lg);
          X[rt] = mma(kf, Dh[s], X[rt]);
          X[rt] = mma(kf, Dl[s], X[rt]);
        }
      }
    }
    // U = V - Gamma rk W, Ut = beta U;  E = T Ut (Ut split)
    f32x4 U[4], E[4];
    {
      f32x4 Ut[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const bf16x4 vv = tr4(sv, LDV, 16 * rt + 4 * lg, 16 * w, lr);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * rt + 4 * lg + i;
          U[rt][i] = (float)vv[i] - fexp2(fac[F_G2 * CH + r]) * fac[F_RK * CH + r] * W[rt][i];
          Ut[rt][i] = fac[F_BETA * CH + r] * U[rt][i];
        }
      }
      bf16x8 Uh[2], Ul[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) split_acc(Uh[s], Ul[s], Ut[2 * s], Ut[2 * s + 1]);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        E[rt] = zero4();
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const bf16x8 ah = tr_perm(tth, LDT, 32 * s, 16 * rt, lr, lg);
          E[rt] = mma(ah, Uh[s], E[rt]);
          E[rt] = mma(ah, Ul[s], E[rt]);
        }
      }
    }
    // row partials over this wave's 16 columns go to per-wave slots: lane
    // (lg, lr) holds row 16 (lr >> 2) + 4 lg + (lr & 3)
    const int prow = 16 * (lr >> 2) + 4 * lg + (lr & 3);
    {  // xe_r = c_r X_r.E_r
      float x[16];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) x[4 * rt + i] = X[rt][i] * E[rt][i];
      slots[(R_XE * NW + w) * CH + prow] = fac[F_C * CH + prow] * rowsum_scatter(x, lr);
    }
    // dE = c X + P~^T dO;  dU = T^T dE (dE split)
    f32x4 dU[4];
    {
      bf16x8 of[TS];
#pragma unroll
      for (int s = 0; s < TS; ++s) of[s] = tr_contig(so, LDO, 32 * s, 16 * w, lr, lg);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) X[rt][i] *= fac[F_C * CH + 16 * rt + 4 * lg + i];
#pragma unroll
        for (int s = 0; s < TS; ++s) X[rt] = mma(ld_contig(ptb, LDP, 16 * rt + lr, 32 * s, lg), of[s], X[rt]);
      }
      bf16x8 Eh[2], El[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) split_acc(Eh[s], El[s], X[2 * s], X[2 * s + 1]);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        dU[rt] = zero4();
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const bf16x8 ah = ld_perm(tth, LDT, 16 * rt + lr, 32 * s, lg);
          dU[rt] = mma(ah, Eh[s], dU[rt]);
          dU[rt] = mma(ah, El[s], dU[rt]);
        }
      }
    }
    // dv, and the row partials dU.U (dbeta) and -Gamma beta rk dU.W (decay)
    {
      float *dvl = a.dv + (krow0 + 4 * lg) * a.dv_st + h * a.dv_sh + col;
      float xb[16], xw[16];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * rt + 4 * lg + i;
          if (r < g.R) dvl[(16 * rt + i) * a.dv_st] = fac[F_BETA * CH + r] * dU[rt][i];
          xb[4 * rt + i] = dU[rt][i] * U[rt][i];
          xw[4 * rt + i] = dU[rt][i] * W[rt][i];
        }
      slots[(R_DB * NW + w) * CH + prow] = rowsum_scatter(xb, lr);
      slots[(R_DL * NW + w) * CH + prow] = -fexp2(fac[F_G2 * CH + prow]) * fac[F_BETA * CH + prow] *
                                           fac[F_RK * CH + prow] * rowsum_scatter(xw, lr);
    }
    // the next head's W and D slabs (this head's are dead); its rows follow
    // at the end of the head, when fewer registers are live
    const bool more = j + 1 < G;
    if (more) load_slabs(h + 1);
    __syncthreads();  // every wave is done with the T^T planes and the v rows
    // the per-wave row partials (dbeta, decay, xe) summed over the waves
    if (tid < 3 * CH) {
      const int q = tid / CH, r = tid % CH;
      float x = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) x += slots[(q * NW + ww) * CH + r];
      red[q * CH + r] += x;
    }
    // E^T and dU^T planes [v][r] (hi, lo)
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const int off = col * LDT + 16 * rt + 4 * lg;
      f32x4 eh, uh;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        eh[i] = (float)(bf16)E[rt][i];
        uh[i] = (float)(bf16)dU[rt][i];
      }
      *(uint2 *)(peh + off) = pack4(eh);
      *(uint2 *)(pel + off) = pack4(E[rt] - eh);
      *(uint2 *)(puh + off) = pack4(uh);
      *(uint2 *)(pul + off) = pack4(dU[rt] - uh);
    }
    __syncthreads();

    // ---- products over V
    // the S0 and D rows of this wave's k tiles for the dK products below, issued
    // here so that their HBM latency passes while dA and Z are formed (every load
    // unconditional: a wave past the last k tile reads the last one)
    bf16x8 Ks[NKW][VS];
    f32x4 Kd[NKW][VS][2];
#pragma unroll
    for (int m = 0; m < NKW; ++m) {
      const int kc = 16 * min(w + m * NW, KT - 1) + lr;
#pragma unroll
      for (int s = 0; s < VS; ++s) {
        const float *pd = Dg + (size_t)kc * V + 32 * s + 8 * lg;
        Ks[m][s] = *(const bf16x8 *)(S0g + (size_t)kc * V + 32 * s + 8 * lg);
        Kd[m][s][0] = *(const f32x4 *)pd;
        Kd[m][s][1] = *(const f32x4 *)(pd + 4);
      }
    }
    // dA = -dU E^T (strictly lower tiles): dbeta and decay terms, then A~ into abar
    for (int idx = w; idx < 10; idx += NW) {
      const int ra = idx < 1 ? 0 : (idx < 3 ? 1 : (idx < 6 ? 2 : 3));
      const int ib = idx - ra * (ra + 1) / 2;
      f32x4 acc = zero4();
#pragma unroll
      for (int s = 0; s < VS; ++s) {
        const bf16x8 uh = tr_contig(puh, LDT, 32 * s, 16 * ra, lr, lg), ul = tr_contig(pul, LDT, 32 * s, 16 * ra, lr, lg);
        const bf16x8 eh = tr_contig(peh, LDT, 32 * s, 16 * ib, lr, lg), el = tr_contig(pel, LDT, 32 * s, 16 * ib, lr, lg);
        acc = mma(uh, eh, acc);
        acc = mma(uh, el, acc);
        acc = mma(ul, eh, acc);
      }
      const int i = 16 * ib + lr;
      float csum = 0.f;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r = 16 * ra + 4 * lg + jj;
        const bool in = i < r && r < g.R;
        const float da = in ? -acc[jj] : 0.f;
        const float ab = in ? abar[r * LDF + i] : 0.f;
        const float br_ = fac[F_BETA * CH + r];
        const float xr = row_sum16(da * ab);  // sum_i dA Abar (dbeta); times beta_r: sum_i dA A
        if (lr == 15) {
          atomicAdd(red + R_DB * CH + r, xr);
          atomicAdd(red + R_DL * CH + r, br_ * xr);
        }
        csum += da * ab * br_;
        if (in) abar[r * LDF + i] = da * br_ * fexp2(fac[F_G2 * CH + r] - fac[F_G2 * CH + i]);
      }
      csum = col_sum4(csum);
      if (lg == 0) atomicAdd(red + R_DL * CH + i, -csum);
    }
    // Z = dO E^T (E hi): W~ and its decay terms, kept in registers for the planes
    // With eight waves the first two formed two dA tiles each (ten tiles): with
    // 32 output tokens (eight Z tiles) the Z tiles go to the other six,
    // round-robin
    constexpr int ZW0 = (NW == 8 && TT16 == 2) ? 10 - NW : 0, NZW = NW - ZW0;
    constexpr int NZ = (TT16 * 4 + NZW - 1) / NZW;
    f32x4 Zw[NZ];
#pragma unroll
    for (int m = 0; m < NZ; ++m) {
      const int idx = w < ZW0 ? TT16 * 4 : (w - ZW0) + m * NZW;
      Zw[m] = zero4();
      if (idx < TT16 * 4) {
        const int ta = idx >> 2, ib = idx & 3;
        f32x4 acc = zero4();
#pragma unroll
        for (int s = 0; s < VS; ++s)
          acc = mma(ld_contig(so, LDO, 16 * ta + lr, 32 * s, lg), tr_contig(peh, LDT, 32 * s, 16 * ib, lr, lg), acc);
        const int i = 16 * ib + lr;
        float csum = 0.f;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int t = 16 * ta + 4 * lg + jj;
          const int rt = min((g.tlo + t) * n + n - 1 - g.row0, CH - 1);  // (exact for t < Tc)
          const bool in = t < g.Tc && i <= rt && i < g.R;
          const float z = in ? acc[jj] : 0.f;
          const float zp = z * (float)ptb[i * LDP + t];
          const float xr = row_sum16(zp);
          if (lr == 15 && t < g.Tc) atomicAdd(red + R_DL * CH + rt, xr);
          csum += zp;
          Zw[m][jj] = in ? scale * fexp2(fac[F_G2 * CH + rt] - fac[F_G2 * CH + i]) * z : 0.f;
        }
        csum = col_sum4(csum);
        if (lg == 0) atomicAdd(red + R_DL * CH + i, -csum);
      }
    }
    // dK += -diag(Gamma beta) dU S0^T (hi) + diag(Gend / Gamma) E D^T (split);
    // dQ += diag(e') dO S0^T (hi), with the decay term of the outputs
#pragma unroll
    for (int m = 0; m < NKW; ++m) {
      const int kt = w + m * NW;
      if (kt >= KT) continue;
      const int kc = 16 * kt + lr;
      f32x4 k1[4], k2[4], q1[TT16];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) k1[rt] = k2[rt] = zero4();
#pragma unroll
      for (int ta = 0; ta < TT16; ++ta) q1[ta] = zero4();
      float ds = 0.f;  // this lane's part of <D, S0>
#pragma unroll
      for (int s = 0; s < VS; ++s) {
        const bf16x8 sh = Ks[m][s];
#pragma unroll
        for (int i = 0; i < 4; ++i) ds += Kd[m][s][0][i] * (float)sh[i] + Kd[m][s][1][i] * (float)sh[4 + i];
        bf16x8 dh, dl;
        split_acc(dh, dl, Kd[m][s][0], Kd[m][s][1]);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          k1[rt] = mma(tr_contig(puh, LDT, 32 * s, 16 * rt, lr, lg), sh, k1[rt]);
          const bf16x8 eh = tr_contig(peh, LDT, 32 * s, 16 * rt, lr, lg), el = tr_contig(pel, LDT, 32 * s, 16 * rt, lr, lg);
          k2[rt] = mma(eh, dh, k2[rt]);
          k2[rt] = mma(eh, dl, k2[rt]);
          k2[rt] = mma(el, dh, k2[rt]);
        }
#pragma unroll
        for (int ta = 0; ta < TT16; ++ta) q1[ta] = mma(ld_contig(so, LDO, 16 * ta + lr, 32 * s, lg), sh, q1[ta]);
      }
      ds = lane63(wave_prefix(ds));
      if (lane == 0) atomicAdd(red + R_DS * CH, ds);
      const float g2e = fac[F_G2 * CH + CH - 1];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * rt + 4 * lg + i;
          const float g2r = fac[F_G2 * CH + r];
          dK[m][rt][i] += -fexp2(g2r) * fac[F_BETA * CH + r] * k1[rt][i] + fexp2(g2e - g2r) * k2[rt][i];
        }
      // output decay term scale Gamma_{r_t} qhat_t.(S0 dO_t) = e_t q_t.dQ1_t
#pragma unroll
      for (int ta = 0; ta < TT16; ++ta)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int t = 16 * ta + 4 * lg + jj;
          const float x = row_sum16(q1[ta][jj] * (float)sq[t * LDK + kc]);
          if (lr == 15 && t < g.Tc) {
            const int rt = (g.tlo + t) * n + n - 1 - g.row0;  // < R for t < Tc
            atomicAdd(red + R_DL * CH + rt, fac[F_E * CH + t] * x);
          }
          dQ[m][ta][jj] += fac[F_EP * CH + t] * q1[ta][jj];
        }
    }
    // the next head's rows, bundle (and k rows when not shared), in registers
    // until the end of this head
    if (more) load_rows(h + 1, !kshared);
    __syncthreads();  // E/dU planes dead; abar holds A~
      // W~ planes [i][t]: w1 = W~ rq_t (for W~^T Qhat), w2 = W~ rk_i (for W~ Khat)
#pragma unroll
    for (int m = 0; m < NZ; ++m) {
      const int idx = w < ZW0 ? TT16 * 4 : (w - ZW0) + m * NZW;
      if (idx < TT16 * 4) {
        const int ta = idx >> 2, ib = idx & 3;
        const int i = 16 * ib + lr, t = 16 * ta + 4 * lg;
        f32x4 x1, x2;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          x1[jj] = Zw[m][jj] * fac[F_RQ * CH + t + jj];
          x2[jj] = Zw[m][jj] * fac[F_RK * CH + i];
        }
        *(uint2 *)(pw1 + i * LDW + t) = pack4(x1);
        *(uint2 *)(pw2 + i * LDW + t) = pack4(x2);
      }
    }
    // M' = (A~ + A~^T) diag(rk), split
    for (int u = tid; u < CH * (CH / 8); u += NTH) {
      const int r = u >> 3, i0 = 8 * (u & 7);
      bf16x8 hi, lo;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int i = i0 + jj;
        float m_ = 0.f;
        if (i < r) m_ = abar[r * LDF + i];
        else if (r < i) m_ = abar[i * LDF + r];
        m_ *= fac[F_RK * CH + i];
        hi[jj] = (bf16)m_;
        lo[jj] = (bf16)(m_ - (float)hi[jj]);
      }
      *(bf16x8 *)(pmh + r * LDT + i0) = hi;
      *(bf16x8 *)(pml + r * LDT + i0) = lo;
    }
    __syncthreads();
    // dK += M' K + W1 Q;  dQ += W2^T K
#pragma unroll
    for (int m = 0; m < NKW; ++m) {
      const int kt = w + m * NW;
      if (kt >= KT) continue;
      bf16x8 kb[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) kb[s] = tr_contig(sk, LDK, 32 * s, 16 * kt, lr, lg);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          dK[m][rt] = mma(ld_contig(pmh, LDT, 16 * rt + lr, 32 * s, lg), kb[s], dK[m][rt]);
          dK[m][rt] = mma(ld_contig(pml, LDT, 16 * rt + lr, 32 * s, lg), kb[s], dK[m][rt]);
        }
#pragma unroll
        for (int s = 0; s < TS; ++s)
          dK[m][rt] = mma(ld_contig(pw1, LDW, 16 * rt + lr, 32 * s, lg), tr_contig(sq, LDK, 32 * s, 16 * kt, lr, lg),
                          dK[m][rt]);
      }
#pragma unroll
      for (int ta = 0; ta < TT16; ++ta)
#pragma unroll
        for (int s = 0; s < 2; ++s) dQ[m][ta] = mma(tr_contig(pw2, LDW, 32 * s, 16 * ta, lr, lg), kb[s], dQ[m][ta]);
    }
    // this head's decay gradients (suffix sums from each token's first row) and dbeta
    if (w == 0) {
      const int r = lane;
      const bool in = r < g.R;
      const float xe = in ? red[R_XE * CH + r] : 0.f;
      const float tot = lane63(wave_prefix(xe));
      float x = in ? red[R_DL * CH + r] - xe : 0.f;
      if (r == g.R - 1) x += fac[F_META * CH] * red[R_DS * CH] + tot;
      const float pre = wave_prefix(x);  // suffix sum: total minus the exclusive prefix
      const float suf = lane63(pre) - pre + x;
      if (in && (g.row0 + r) % n == 0) a.dg[(g.t0 + (g.row0 + r) / n) * a.dg_st + h * a.dg_sh] = suf;
      if (in) a.dbeta[(krow0 + r) * a.db_st + h * a.db_sh] = red[R_DB * CH + r];
    }
    // with one k head per state head, this head's dk rows are complete
    if (!kshared) {
      store_rows<NKW, 4, K>(a.dk, krow0, a.dk_st, (h / (a.Hv / a.Hk)) * a.dk_sh, g.R, dK, sk, LDK, fac + F_RK * CH,
                            red + R_KN * CH, a.l2norm, w, NW, lr, lg);
#pragma unroll
      for (int m = 0; m < NKW; ++m)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) dK[m][rt] = zero4();
    }
    if (more) {
      __syncthreads();  // every wave is past this head's LDS reads
      commit_head(!kshared);
    }
  }
  // dq (and the shared dk), through the norm gradient
  store_rows<NKW, TT16, K>(a.dq, qrow0, a.dq_st, hq * a.dq_sh, g.Tc, dQ, sq, LDK, fac + F_RQ * CH, red + R_QN * CH,
                           a.l2norm, w, NW, lr, lg);
  if (kshared)
    store_rows<NKW, 4, K>(a.dk, krow0, a.dk_st, (hq * G / (a.Hv / a.Hk)) * a.dk_sh, g.R, dK, sk, LDK, fac + F_RK * CH,
                          red + R_KN * CH, a.l2norm, w, NW, lr, lg);
}

template <int K, int V, int TCM> hipError_t launch_kv(const BwdChunkArgs &a, hipStream_t stream) {
  if (a.ntdp_rows > 0 && a.Hk > 0) {
    hipLaunchKernelGGL((gdp_bwd_prep_kernel<K, TCM>), dim3((unsigned)(a.ntdp_rows * a.Hk)), dim3(NTHR), 0, stream, a);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  }
  if (a.N > 0) {
    hipLaunchKernelGGL((gdp_bwd_state_kernel<K, V, TCM>), dim3((unsigned)((int64_t)a.N * a.Hv)), dim3(4 * V), 0,
                       stream, a);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    hipLaunchKernelGGL((gdp_bwd_adjoint_kernel<K, V, TCM>), dim3((unsigned)((int64_t)a.N * a.Hv)), dim3(4 * V), 0,
                       stream, a);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  }
  if (a.ntdp_rows > 0) {
    hipLaunchKernelGGL((gdp_bwd_grad_kernel<K, V, TCM>), dim3((unsigned)(a.ntdp_rows * a.Hqk)), dim3(4 * V), 0,
                       stream, a);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int K, int V> hipError_t launch_k(const BwdChunkArgs &a, hipStream_t stream) {
  return a.n == 1 ? launch_kv<K, V, 64>(a, stream) : launch_kv<K, V, 32>(a, stream);
}

}  // namespace

size_t bwd_bundle_bytes(int n) { return n == 1 ? (size_t)Bundle<64>::BYTES : (size_t)Bundle<32>::BYTES; }

size_t bwd_state_record_bytes(int K, int V) { return (size_t)CH * V * 4 + (size_t)K * V * 2; }

bool bwd_chunked_supported(int dtype, int K, int V, int n) {
  return dtype == IN_BF16 && (K == 64 || K == 128) && (V == 64 || V == 128) && n >= 1 && n <= 64;
}

hipError_t launch_bwd_chunked(const BwdChunkArgs &a, int K, int V, hipStream_t stream) {
  if (K == 128 && V == 128) return launch_k<128, 128>(a, stream);
  if (K == 128 && V == 64) return launch_k<128, 64>(a, stream);
  if (K == 64 && V == 128) return launch_k<64, 128>(a, stream);
  if (K == 64 && V == 64) return launch_k<64, 64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace gdp
