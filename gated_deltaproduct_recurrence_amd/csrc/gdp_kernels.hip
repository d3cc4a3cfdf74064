// gdp_kernels.hip -- gfx950 (CDNA4) kernels of chunked Gated DeltaProduct prefill.
//
// Method (FlashInfer docs, "flashinfer.gdp_prefill.chunk_gated_delta_product",
// recurrence display; Megatron Core API docs, core.ssm.ops.gdp.chunk, stage list):
// per token the K x V state S decays by alpha_t, then takes n beta-gated
// Householder updates from the sub-token rows t*n..t*n+n-1, then is read out.
// The chunked form works on 64-row chunks of the Householder-expanded stream.
// For an expanded chunk with start state S0, rows r, base-2 cumulative log
// decay G_r (decays sit on the first sub-row of each token: Megatron stage 1)
// and A[r,i] = beta_r 2^(G_r - G_i) k_r.k_i for i < r:
//     T = (I + A)^-1                                  (WY step, Megatron stage 2)
//     E = T (diag(beta) V - diag(beta 2^G) K S0)      (= U - W S0: the v_new rows)
//     S_end = 2^G_last S0 + K^T diag(2^(G_last - G)) E  (state sweep, stage 3)
// and for token chunk c (n expanded chunks) with start state h_c,
//     o_t = scale (2^Gt_t q_t^T h_c + sum_{r: tok(r) <= t} 2^(Gt_t - Gt_tok(r)) (q_t.k_r) e_r)
// (output combine, stage 4), Gt being the token-stream cumulative decay.
//
// Kernels, in launch order on one stream:
//   gdp_descriptor_kernel  both chunkings' descriptors (one workgroup)
//   gdp_wy_kernel          one workgroup per (expanded chunk, q/k head): the Gram
//                          matrix once, then per state head of the group the
//                          64 x 64 inverse T in fp32 (LDS), stored in bf16/f32 in
//                          MFMA-fragment order
//   gdp_scan_kernel        one workgroup per (sequence, state head, V-tile): walks
//                          the chunks in order with S in fp32 MFMA accumulators
//                          (wave w owns a 16*NB-column slab), computing E = T R,
//                          the state update and the outputs; the next chunk's
//                          k/v/q rows are prefetched into registers and LDS is
//                          double-buffered, so each chunk costs two barriers.
// Every contraction is an MFMA: v_mfma_f32_16x16x32_bf16 for bf16 inputs,
// v_mfma_f32_16x16x4_f32 for f32 inputs and for the fp32 triangular inverse.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdp_launch.h"

namespace gdp {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int CH = 64;  // chunk length on both streams
constexpr int NTHR = 256;
constexpr float LOG2E = 1.4426950408889634f;

// ---------------------------------------------------------------- MFMA fragments
//
// One "fragment" is what a lane contributes to a 16 x 16 x 32 reduction step:
// 8 values of one row (A operand) or one column (B operand).  Lane l supplies
// row/column (l & 15) and reduction slots 8*(l >> 4) .. +8.  Which physical
// reduction index sits in each slot is free as long as A and B agree:
//   * "contig": slots hold k0 + 8g .. k0 + 8g + 7 (both operands from LDS);
//   * "perm":   slots hold k0 + 4g .. +3 and k0 + 16 + 4g .. +3, which is the
//     row order of two stacked 16 x 16 accumulator tiles, so an accumulator can
//     serve as the B operand of the next product without leaving registers.

template <typename T> struct Frag;
template <> struct Frag<bf16> { bf16x8 v; };
template <> struct Frag<float> { float v[8]; };

__device__ __forceinline__ f32x4 mma(const Frag<bf16> &a, const Frag<bf16> &b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(const Frag<float> &a, const Frag<float> &b, f32x4 c) {
#pragma unroll
  for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], c, 0, 0, 0);
  return c;
}

__device__ __forceinline__ Frag<bf16> lds_contig(const bf16 *base, int ld, int row, int k0, int lg) {
  Frag<bf16> f;
  f.v = *(const bf16x8 *)(base + row * ld + k0 + 8 * lg);
  return f;
}
__device__ __forceinline__ Frag<bf16> lds_perm(const bf16 *base, int ld, int row, int k0, int lg) {
  const bf16 *p = base + row * ld + k0 + 4 * lg;
  bf16x4 lo = *(const bf16x4 *)p;
  bf16x4 hi = *(const bf16x4 *)(p + 16);
  Frag<bf16> f;
  f.v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return f;
}
__device__ __forceinline__ Frag<float> lds_contig(const float *base, int ld, int row, int k0, int lg) {
  const float *p = base + row * ld + k0 + 8 * lg;
  f32x4 lo = *(const f32x4 *)p, hi = *(const f32x4 *)(p + 4);
  Frag<float> f;
#pragma unroll
  for (int i = 0; i < 4; ++i) { f.v[i] = lo[i]; f.v[4 + i] = hi[i]; }
  return f;
}
__device__ __forceinline__ Frag<float> lds_perm(const float *base, int ld, int row, int k0, int lg) {
  const float *p = base + row * ld + k0 + 4 * lg;
  f32x4 lo = *(const f32x4 *)p, hi = *(const f32x4 *)(p + 16);
  Frag<float> f;
#pragma unroll
  for (int i = 0; i < 4; ++i) { f.v[i] = lo[i]; f.v[4 + i] = hi[i]; }
  return f;
}
// B operand from two stacked accumulator tiles (rows 32s..32s+15 and 32s+16..32s+31).
__device__ __forceinline__ void from_acc(Frag<bf16> &f, f32x4 lo, f32x4 hi) {
#pragma unroll
  for (int i = 0; i < 4; ++i) { f.v[i] = (bf16)lo[i]; f.v[4 + i] = (bf16)hi[i]; }
}
__device__ __forceinline__ void from_acc(Frag<float> &f, f32x4 lo, f32x4 hi) {
#pragma unroll
  for (int i = 0; i < 4; ++i) { f.v[i] = lo[i]; f.v[4 + i] = hi[i]; }
}
// a fragment stored contiguously (8 elements per lane) in global memory
__device__ __forceinline__ void load_frag(Frag<bf16> &f, const bf16 *p) { f.v = *(const bf16x8 *)p; }
__device__ __forceinline__ void load_frag(Frag<float> &f, const float *p) {
  f32x4 lo = *(const f32x4 *)p, hi = *(const f32x4 *)(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) { f.v[i] = lo[i]; f.v[4 + i] = hi[i]; }
}
__device__ __forceinline__ void store_frag(bf16 *p, const Frag<float> &f) {
  bf16x8 x;
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = (bf16)f.v[i];
  *(bf16x8 *)p = x;
}
__device__ __forceinline__ void store_frag(float *p, const Frag<float> &f) {
  *(f32x4 *)p = f32x4{f.v[0], f.v[1], f.v[2], f.v[3]};
  *(f32x4 *)(p + 4) = f32x4{f.v[4], f.v[5], f.v[6], f.v[7]};
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

template <typename T> __device__ __forceinline__ float to_f(T x) { return (float)x; }

// ---------------------------------------------------------------- small helpers

__device__ __forceinline__ int64_t load_index(const void *p, int is64, int64_t i) {
  return is64 ? ((const int64_t *)p)[i] : (int64_t)((const int32_t *)p)[i];
}

__device__ __forceinline__ float wave_inclusive_sum(float x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x;
}

__device__ __forceinline__ uint32_t word_of(const uint4 &s, int i) {
  return i == 0 ? s.x : (i == 1 ? s.y : (i == 2 ? s.z : s.w));
}

// sum of squares of a 16-byte segment of T values (kept as raw words so that
// the compiler does not split a prefetched segment at its load)
template <typename T> __device__ __forceinline__ float seg_sumsq(const uint4 &s) {
  float a = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = word_of(s, i);
    if constexpr (sizeof(T) == 2) {
      const float lo = __uint_as_float(w << 16), hi = __uint_as_float(w & 0xffff0000u);
      a = fmaf(lo, lo, a);
      a = fmaf(hi, hi, a);
    } else {
      const float x = __uint_as_float(w);
      a = fmaf(x, x, a);
    }
  }
  return a;
}

// Element e of four row segments r[0..3], stored as the 4-element run
// d[0..3] of a transposed tile.
template <typename T> __device__ __forceinline__ void store_col4(T *d, const uint4 (&r)[4], int e) {
  if constexpr (sizeof(T) == 2) {
    const int wi = e >> 1;
    const uint32_t w0 = word_of(r[0], wi), w1 = word_of(r[1], wi), w2 = word_of(r[2], wi), w3 = word_of(r[3], wi);
    uint2 x;
    if (e & 1) {
      x.x = (w0 >> 16) | (w1 & 0xffff0000u);
      x.y = (w2 >> 16) | (w3 & 0xffff0000u);
    } else {
      x.x = (w0 & 0xffffu) | (w1 << 16);
      x.y = (w2 & 0xffffu) | (w3 << 16);
    }
    *(uint2 *)d = x;
  } else {
    *(uint4 *)d = uint4{word_of(r[0], e), word_of(r[1], e), word_of(r[2], e), word_of(r[3], e)};
  }
}

// rows [0, 64) x D columns of a strided global matrix into LDS (row stride ld);
// rows >= nvalid are zero.  One 16-byte segment per thread per step.
template <typename T, int D, int LD>
__device__ __forceinline__ void load_rows(T *dst, const T *src, int64_t rs, int nvalid, int tid) {
  constexpr int EPS = 16 / (int)sizeof(T), SEG = D / EPS;
#pragma unroll 4
  for (int u = tid; u < CH * SEG; u += NTHR) {
    const int r = u / SEG, s = u % SEG;
    uint4 x = {0u, 0u, 0u, 0u};
    if (r < nvalid) x = *(const uint4 *)(src + (int64_t)r * rs + s * EPS);
    *(uint4 *)(dst + r * LD + s * EPS) = x;
  }
}

// 1/sqrt(sum x^2 + 1e-6) of 64 LDS rows of width D; 4 threads per row.
template <typename T, int D>
__device__ __forceinline__ void rows_rstd(const T *base, int ld, float *out, int tid) {
  const int row = tid >> 2, part = tid & 3;
  float ss = 0.f;
#pragma unroll 8
  for (int e = part * (D / 4); e < (part + 1) * (D / 4); ++e) {
    const float x = to_f(base[row * ld + e]);
    ss += x * x;
  }
  ss += __shfl_xor(ss, 1);
  ss += __shfl_xor(ss, 2);
  if (part == 0) out[row] = 1.0f / sqrtf(ss + 1e-6f);
}

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

// ---------------------------------------------------------------- WY kernel

template <typename T, int K> struct WySmem {
  static constexpr int EPS = 16 / (int)sizeof(T);
  static constexpr int LDK = K + EPS;
  static constexpr int LDA = CH + 4;
  union {
    T k[CH * LDK];      // k rows of the chunk (live until the Gram is formed)
    float tf[CH * LDA];  // then the fp32 inverse
  } u;
  float a[CH * LDA];
  float gdp[CH], beta[CH], rk[CH];
};

// the 10 lower-triangular 16 x 16 tiles of a 64 x 64 matrix
__device__ __forceinline__ void lower_tile(int idx, int &ra, int &rb) {
  ra = idx < 1 ? 0 : (idx < 3 ? 1 : (idx < 6 ? 2 : 3));
  rb = idx - ra * (ra + 1) / 2;
}

template <typename T, int K>
__global__ void __launch_bounds__(NTHR) gdp_wy_kernel(PrefillArgs a) {
  using S = WySmem<T, K>;
  constexpr int LDK = S::LDK, LDA = S::LDA, KS = K / 32;
  __shared__ S sm;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, lr = lane & 15, lg = lane >> 4;

  const int64_t p = blockIdx.x / a.Hqk;
  const int hq = (int)(blockIdx.x % a.Hqk);
  if (p >= a.ntdp_rows || p >= a.tws_rows) return;
  const int seq = a.chunk_indices_dp[2 * p], cc = a.chunk_indices_dp[2 * p + 1];
  if (seq < 0 || seq >= a.N || cc < 0) return;  // padding row
  const int n = a.n;
  int64_t t0 = load_index(a.cu, a.cu_is64, seq), t1 = load_index(a.cu, a.cu_is64, seq + 1);
  t0 = t0 < 0 ? 0 : (t0 > a.T ? a.T : t0);
  t1 = t1 < t0 ? t0 : (t1 > a.T ? a.T : t1);
  const int64_t nsub = (t1 - t0) * n, s0 = (int64_t)CH * cc;
  if (s0 >= nsub) return;
  const int nrow = (int)((nsub - s0) < CH ? (nsub - s0) : CH);
  const int64_t row0 = t0 * n + s0;  // first sub-token row of the chunk

  load_rows<T, K, LDK>(sm.u.k, (const T *)a.k + hq * a.k_sh + row0 * a.k_st, a.k_st, nrow, tid);
  __syncthreads();
  if (a.l2norm) rows_rstd<T, K>(sm.u.k, LDK, sm.rk, tid);
  else if (tid < CH) sm.rk[tid] = 1.f;
  __syncthreads();

  // Gram tiles (k_r.k_i rk_r rk_i), kept in registers for every state head of the group
  f32x4 gram[3];
#pragma unroll
  for (int it = 0; it < 3; ++it) {
    const int idx = w + 4 * it;
    gram[it] = zero4();
    if (idx < 10) {
      int ra, rb;
      lower_tile(idx, ra, rb);
#pragma unroll
      for (int s = 0; s < KS; ++s)
        gram[it] = mma(lds_contig(sm.u.k, LDK, 16 * ra + lr, 32 * s, lg),
                       lds_contig(sm.u.k, LDK, 16 * rb + lr, 32 * s, lg), gram[it]);
#pragma unroll
      for (int i = 0; i < 4; ++i) gram[it][i] *= sm.rk[16 * ra + 4 * lg + i] * sm.rk[16 * rb + lr];
    }
  }
  __syncthreads();  // k rows are dead; sm.u.tf reuses them

  const int grp = a.Hv / a.Hqk;
  for (int hh = 0; hh < grp; ++hh) {
    const int h = hq * grp + hh;
    if (w == 0) {
      const int r = lane;
      const int64_t s = s0 + r;
      float gam = 0.f, bt = 0.f;
      if (r < nrow) {
        bt = a.beta[(row0 + r) * a.b_st + h * a.b_sh];
        if (s % n == 0) gam = a.g[(t0 + s / n) * a.g_st + h * a.g_sh] * LOG2E;
      }
      sm.gdp[r] = wave_inclusive_sum(gam, lane);
      sm.beta[r] = bt;
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 3; ++it) {
      const int idx = w + 4 * it;
      if (idx < 10) {
        int ra, rb;
        lower_tile(idx, ra, rb);
        const int c = 16 * rb + lr;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * ra + 4 * lg + i;
          sm.a[r * LDA + c] = (c < r) ? sm.beta[r] * exp2f(sm.gdp[r] - sm.gdp[c]) * gram[it][i] : 0.f;
        }
      }
    }
    __syncthreads();
    wy_inverse<LDA>(sm.a, sm.u.tf, tid);
    // T in fragment order: fragment f = (row tile f/2, reduction half f%2), lane-major
    T *dst = (T *)a.tws + ((size_t)p * a.Hv + h) * (CH * CH);
#pragma unroll
    for (int f = 2 * w; f < 2 * w + 2; ++f) {
      const Frag<float> fr = lds_perm(sm.u.tf, LDA, 16 * (f >> 1) + lr, 32 * (f & 1), lg);
      store_frag(dst + (f * 64 + lane) * 8, fr);
    }
    __syncthreads();  // before the next head reuses sm.a / sm.gdp / sm.u.tf
  }
}

// ---------------------------------------------------------------- scan kernel

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }  // v_exp_f32
__device__ __forceinline__ float frsq(float x) { return __builtin_amdgcn_rsqf(x); }    // v_rsq_f32

template <typename T, int K, int NB> struct ScanSmem {
  static constexpr int EPS = 16 / (int)sizeof(T);  // elements per 16-byte segment
  static constexpr int BV = 64 * NB;                // state columns per workgroup
  static constexpr int LDK = K + EPS;               // k, q rows
  static constexpr int LDKT = CH + EPS;             // k^T rows (one per key dim)
  static constexpr int LDVT = CH + EPS;             // v^T rows (one per state column)
  static constexpr int LDC = CH + EPS;              // P rows
  static constexpr bool kTinLds = sizeof(T) == 2;   // bf16 WY blocks are staged in LDS
  T k[2][CH * LDK];
  T kt[2][K * LDKT];
  T vt[2][BV * LDVT];
  T q[CH * LDK];
  T p[CH * LDC];
  T t[kTinLds ? 2 : 1][kTinLds ? CH * CH : 8];
  float gdp[2][CH], beta[2][CH], rk[2][CH];
  float gtok[CH], rq[CH];
};

// Registers holding the next chunk's rows between their global load and their
// LDS store.  k, q and v use 4-row units (rows 4rb..4rb+3 x one 16-byte
// segment): one thread then holds what a transposed copy needs, and the CB
// threads of a row group hold whole rows for the L2 norm.  Loads are never
// predicated (rows past the end are clamped to the last valid row and zeroed
// at commit), so issuing them never waits.
template <typename T, int K, int BV> struct Prefetch {
  static constexpr int EPS = 16 / (int)sizeof(T);
  static constexpr int KCB = K / EPS, KUNITS = (CH / 4) * KCB;
  static constexpr int VCB = BV / EPS, VUNITS = (CH / 4) * VCB;
  static_assert(KUNITS <= NTHR && VUNITS <= NTHR, "one 4-row unit per thread");
  uint4 k[4], q[4], v[4];
  uint4 tw[2];
  float beta, gam, gtk;
};

__device__ __forceinline__ f32x4 ld4(const float *p) { return *(const f32x4 *)p; }

// 16-byte load at a wave-uniform base plus a 32-bit per-lane byte offset
__device__ __forceinline__ uint4 ldg16(const void *base, uint32_t off) {
  return *(const uint4 *)((const char *)base + off);
}

// The state is kept as S = lam * Sst with a wave-uniform lam, so that the
// per-chunk decay 2^G_last multiplies lam instead of the 64 accumulators of
// each lane; Sst is rescaled only when lam * 2^G_last would drop below this.
constexpr float LAM_MIN = 8.673617e-19f;  // 2^-60

template <typename T, int K, int V, int NB>
__global__ void __launch_bounds__(NTHR, 1) gdp_scan_kernel(PrefillArgs a) {
  using S = ScanSmem<T, K, NB>;
  using P = Prefetch<T, K, S::BV>;
  constexpr int BV = S::BV, NVT = V / BV, KT16 = K / 16, KS = K / 32, EPS = S::EPS;
  constexpr int LDK = S::LDK, LDKT = S::LDKT, LDVT = S::LDVT, LDC = S::LDC;
  constexpr uint32_t ES = sizeof(T);
  __shared__ S sm;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, lr = lane & 15, lg = lane >> 4;

  // Workgroups are dealt to the 8 XCDs round-robin; remap so that each XCD
  // walks a contiguous range of chains (the heads sharing a q/k head, and the
  // V-tiles of one head, then read the same k/q rows through one L2).
  const int64_t G = gridDim.x, bid = blockIdx.x;
  const int64_t chain = (G % 8 == 0) ? (bid % 8) * (G / 8) + bid / 8 : bid;
  const int vt = (int)(chain % NVT);
  const int h = (int)((chain / NVT) % a.Hv);
  const int seq = (int)(chain / ((int64_t)NVT * a.Hv));
  const int hq = h / (a.Hv / a.Hqk);
  const int n = a.n;

  int64_t t0 = load_index(a.cu, a.cu_is64, seq), t1 = load_index(a.cu, a.cu_is64, seq + 1);
  t0 = t0 < 0 ? 0 : (t0 > a.T ? a.T : t0);
  t1 = t1 < t0 ? t0 : (t1 > a.T ? a.T : t1);
  const int64_t L = t1 - t0, nsub = L * n;
  const int nexp = (int)((nsub + CH - 1) / CH);
  const int wcol = w * 16 * NB;     // first column of this wave inside the tile
  const int gcol = vt * BV + wcol;  // ... and inside the head

  const T *qg = (const T *)a.q + hq * a.q_sh;
  const T *kg = (const T *)a.k + hq * a.k_sh;
  const T *vg = (const T *)a.v + h * a.v_sh + vt * BV;
  const float *gg = a.g + h * a.g_sh;
  const float *bg = a.beta + h * a.b_sh;
  const size_t KV = (size_t)K * V;
  const size_t state_off = ((size_t)seq * a.Hv + h) * KV;
  const int64_t tws_row0 = a.chunk_offsets_dp[seq];
  auto wy_block = [&](int e) {  // WY block of expanded chunk e (clamped to the buffer)
    int64_t r = tws_row0 + e;
    r = r < 0 ? 0 : (r >= a.tws_rows ? a.tws_rows - 1 : r);
    return (const T *)a.tws + ((size_t)r * a.Hv + h) * (CH * CH);
  };
  // byte strides of one row (the host guarantees 64 rows stay below 2^31 bytes)
  const uint32_t kst = (uint32_t)a.k_st * ES, vst = (uint32_t)a.v_st * ES, qst = (uint32_t)a.q_st * ES;
  const uint32_t gst = (uint32_t)a.g_st * 4u, bst = (uint32_t)a.b_st * 4u;
  const int krb = tid / P::KCB, kcb = tid % P::KCB;  // k / q unit of this thread
  const int vrb = tid / P::VCB, vcb = tid % P::VCB;  // v unit of this thread

  // ---- prefetch: issue the global loads of expanded chunk e (and, when it
  // starts a token chunk, of that token chunk's q rows and decays)
  P pf;
  auto issue = [&](int e) {
    const int64_t s0 = (int64_t)CH * e;
    const int nrow = (int)((nsub - s0) < CH ? (nsub - s0) : CH);
    const int64_t row0 = t0 * n + s0;
    if (tid < P::KUNITS) {
      const T *kb = kg + row0 * a.k_st;
#pragma unroll
      for (int qd = 0; qd < 4; ++qd)
        pf.k[qd] = ldg16(kb, (uint32_t)min(4 * krb + qd, nrow - 1) * kst + (uint32_t)kcb * 16u);
    }
    if (tid < P::VUNITS) {
      const T *vb = vg + row0 * a.v_st;
#pragma unroll
      for (int qd = 0; qd < 4; ++qd)
        pf.v[qd] = ldg16(vb, (uint32_t)min(4 * vrb + qd, nrow - 1) * vst + (uint32_t)vcb * 16u);
    }
    if constexpr (S::kTinLds) {
      const T *tb = wy_block(e);
      pf.tw[0] = ldg16(tb, (uint32_t)tid * 32u);
      pf.tw[1] = ldg16(tb, (uint32_t)tid * 32u + 16u);
    }
    if (tid < CH) {
      const int r = min(tid, nrow - 1);
      pf.beta = *(const float *)((const char *)(bg + row0 * a.b_st) + (uint32_t)r * bst);
      // token of sub-row s0 + r relative to the first token of this chunk's rows
      const int64_t tokf = s0 / n;
      const int rel = (int)(s0 - tokf * n) + r;
      pf.gam = *(const float *)((const char *)(gg + (t0 + tokf) * a.g_st) + (uint32_t)(rel / n) * gst);
    }
    if (e % n == 0) {
      const int c = e / n;
      const int64_t tokbase = t0 + (int64_t)CH * c;
      const int ntok = (int)((L - (int64_t)CH * c) < CH ? (L - (int64_t)CH * c) : CH);
      if (tid < P::KUNITS) {
        const T *qb = qg + tokbase * a.q_st;
#pragma unroll
        for (int qd = 0; qd < 4; ++qd)
          pf.q[qd] = ldg16(qb, (uint32_t)min(4 * krb + qd, ntok - 1) * qst + (uint32_t)kcb * 16u);
      }
      if (tid < CH)
        pf.gtk = *(const float *)((const char *)(gg + tokbase * a.g_st) + (uint32_t)min(tid, ntok - 1) * gst);
    }
  };
  // ---- commit: wait for the prefetched rows, zero the rows past the end, and
  // store them (with the transposed copies, L2 norms and decay cumsums) to LDS slot sl
  auto commit = [&](int e, int sl) {
    const int64_t s0 = (int64_t)CH * e;
    const int nrow = (int)((nsub - s0) < CH ? (nsub - s0) : CH);
    if (tid < P::KUNITS) {
      if (nrow < CH) {
#pragma unroll
        for (int qd = 0; qd < 4; ++qd)
          if (4 * krb + qd >= nrow) pf.k[qd] = uint4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) *(uint4 *)(sm.k[sl] + (4 * krb + qd) * LDK + kcb * EPS) = pf.k[qd];
#pragma unroll
      for (int e2 = 0; e2 < EPS; ++e2) store_col4<T>(sm.kt[sl] + (kcb * EPS + e2) * LDKT + 4 * krb, pf.k, e2);
      if (a.l2norm) {
        float ss[4];
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) ss[qd] = seg_sumsq<T>(pf.k[qd]);
#pragma unroll
        for (int off = 1; off < P::KCB; off <<= 1)
#pragma unroll
          for (int qd = 0; qd < 4; ++qd) ss[qd] += __shfl_xor(ss[qd], off);
        if (kcb == 0)
          *(f32x4 *)(sm.rk[sl] + 4 * krb) =
              f32x4{frsq(ss[0] + 1e-6f), frsq(ss[1] + 1e-6f), frsq(ss[2] + 1e-6f), frsq(ss[3] + 1e-6f)};
      } else if (kcb == 0) {
        *(f32x4 *)(sm.rk[sl] + 4 * krb) = f32x4{1.f, 1.f, 1.f, 1.f};
      }
    }
    if (tid < P::VUNITS) {
      if (nrow < CH) {
#pragma unroll
        for (int qd = 0; qd < 4; ++qd)
          if (4 * vrb + qd >= nrow) pf.v[qd] = uint4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int e2 = 0; e2 < EPS; ++e2) store_col4<T>(sm.vt[sl] + (vcb * EPS + e2) * LDVT + 4 * vrb, pf.v, e2);
    }
    if constexpr (S::kTinLds) {
      *(uint4 *)(sm.t[sl] + tid * 16) = pf.tw[0];
      *(uint4 *)(sm.t[sl] + tid * 16 + 8) = pf.tw[1];
    }
    if (tid < CH) {
      const int rem = (int)(s0 % n);
      const bool valid = tid < nrow;
      const bool decay = valid && ((rem + tid) % n == 0);  // first sub-row of its token
      sm.gdp[sl][tid] = wave_inclusive_sum(decay ? pf.gam * LOG2E : 0.f, lane);
      sm.beta[sl][tid] = valid ? pf.beta : 0.f;
    }
    if (e % n == 0) {
      const int c = e / n;
      const int ntok = (int)((L - (int64_t)CH * c) < CH ? (L - (int64_t)CH * c) : CH);
      if (tid < P::KUNITS) {
        if (ntok < CH) {
#pragma unroll
          for (int qd = 0; qd < 4; ++qd)
            if (4 * krb + qd >= ntok) pf.q[qd] = uint4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) *(uint4 *)(sm.q + (4 * krb + qd) * LDK + kcb * EPS) = pf.q[qd];
        if (a.l2norm) {
          float ss[4];
#pragma unroll
          for (int qd = 0; qd < 4; ++qd) ss[qd] = seg_sumsq<T>(pf.q[qd]);
#pragma unroll
          for (int off = 1; off < P::KCB; off <<= 1)
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) ss[qd] += __shfl_xor(ss[qd], off);
          if (kcb == 0)
            *(f32x4 *)(sm.rq + 4 * krb) =
                f32x4{frsq(ss[0] + 1e-6f), frsq(ss[1] + 1e-6f), frsq(ss[2] + 1e-6f), frsq(ss[3] + 1e-6f)};
        } else if (kcb == 0) {
          *(f32x4 *)(sm.rq + 4 * krb) = f32x4{1.f, 1.f, 1.f, 1.f};
        }
      }
      if (tid < CH) sm.gtok[tid] = wave_inclusive_sum(tid < ntok ? pf.gtk * LOG2E : 0.f, lane);
    }
  };

  // ---- state S = lam * Sst (K x BV slab of this wave): fp32 accumulators
  f32x4 Sacc[KT16][NB];
#pragma unroll
  for (int at = 0; at < KT16; ++at)
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (a.s0) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          Sacc[at][b][i] = a.s0[state_off + (size_t)(16 * at + 4 * lg + i) * V + gcol + 16 * b + lr];
      } else {
        Sacc[at][b] = zero4();
      }
    }
  float lam = 1.f;

  if (nexp > 0) {
    issue(0);
    commit(0, 0);
  }
  __syncthreads();

  // O^T (this wave's 16*NB state columns x the 64 tokens of the chunk): the
  // outputs are accumulated transposed, O^T = lam Sst^T Q^T diag(.) + E^T P^T,
  // so that the state and E accumulators serve directly as A operands and each
  // lane ends up holding 4 consecutive output columns of one token.
  f32x4 O[NB][4];
  for (int e = 0; e < nexp; ++e) {
    const int sl = e & 1;
    const int c = e / n;
    const int j = e - c * n;
    const int ntok = (int)((L - (int64_t)CH * c) < CH ? (L - (int64_t)CH * c) : CH);

    Frag<T> Sb[KS][NB];
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int b = 0; b < NB; ++b) from_acc(Sb[s][b], Sacc[2 * s][b], Sacc[2 * s + 1][b]);

    if (j == 0) {
      // state entering token chunk c
      if (a.chunk_states) {
        const int64_t row = (int64_t)a.chunk_offsets[seq] + c;
        if (row >= 0 && row < a.cs_rows) {
          float *dst = a.chunk_states + ((size_t)row * a.Hv + h) * KV;
#pragma unroll
          for (int at = 0; at < KT16; ++at)
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                dst[(size_t)(16 * at + 4 * lg + i) * V + gcol + 16 * b + lr] = lam * Sacc[at][b][i];
        }
      }
      // O^T = (Sst^T Q^T) diag(lam 2^Gt rq)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int t = 16 * a4 + lr;
        const float f = lam * fexp2(sm.gtok[t]) * sm.rq[t];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          f32x4 acc = zero4();
#pragma unroll
          for (int s = 0; s < KS; ++s) acc = mma(Sb[s][b], lds_perm(sm.q, LDK, t, 32 * s, lg), acc);
          O[b][a4] = acc * f;
        }
      }
    }

    if (e + 1 < nexp) issue(e + 1);

    // scores P[t][r] = rq_t rk_r 2^(Gt_t - Gt_tok(r)) q_t.k_r for tok(r) <= t, tok(r) = (64j + r)/n
    const int64_t s0 = (int64_t)CH * e;
    const int nrow = (int)((nsub - s0) < CH ? (nsub - s0) : CH);
    const T *kq = sm.k[sl];
    const float *rk = sm.rk[sl];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int tt = w + 4 * it, ta = tt >> 2, tb = tt & 3;
      const bool live = (CH * j + 16 * tb) / n <= 16 * ta + 15;
      f32x4 acc = zero4();
      if (live) {
#pragma unroll
        for (int s = 0; s < KS; ++s)
          acc = mma(lds_contig(sm.q, LDK, 16 * ta + lr, 32 * s, lg), lds_contig(kq, LDK, 16 * tb + lr, 32 * s, lg),
                    acc);
      }
      const int r = 16 * tb + lr;
      const int tk = (CH * j + r) / n;
      const float colf = (r < nrow) ? rk[r] : 0.f;
      const float gk = sm.gtok[tk];
      const f32x4 gt = ld4(sm.gtok + 16 * ta + 4 * lg), rq = ld4(sm.rq + 16 * ta + 4 * lg);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * ta + 4 * lg + i;
        const float val = (live && tk <= t) ? rq[i] * colf * fexp2(gt[i] - gk) * acc[i] : 0.f;
        sm.p[t * LDC + r] = (T)val;
      }
    }

    // R = diag(beta) V - diag(beta 2^G rk lam) K Sst   (this wave's columns)
    const float *gd = sm.gdp[sl];
    const float *bt = sm.beta[sl];
    const T *vtl = sm.vt[sl];
    f32x4 R[4][NB];
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const int r0 = 16 * a4 + 4 * lg;
      const f32x4 btv = ld4(bt + r0), gdv = ld4(gd + r0), rkv = ld4(rk + r0);
      f32x4 coef;
#pragma unroll
      for (int i = 0; i < 4; ++i) coef[i] = btv[i] * fexp2(gdv[i]) * rkv[i] * lam;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        f32x4 x = zero4();
#pragma unroll
        for (int s = 0; s < KS; ++s) x = mma(lds_perm(kq, LDK, 16 * a4 + lr, 32 * s, lg), Sb[s][b], x);
        const T *vp = vtl + (wcol + 16 * b + lr) * LDVT + r0;
        f32x4 vv;
        if constexpr (sizeof(T) == 2) {
          const bf16x4 v4 = *(const bf16x4 *)vp;
#pragma unroll
          for (int i = 0; i < 4; ++i) vv[i] = (float)v4[i];
        } else {
          vv = *(const f32x4 *)vp;
        }
        R[a4][b] = btv * vv - coef * x;
      }
    }
    __syncthreads();  // P complete

    // WY fragments of this chunk: fragment f = 2 * (row tile) + (reduction half),
    // lane-major; the (0,1) and (1,1) halves are zero (T is lower triangular)
    Frag<T> tfr[6];
    {
      const T *tl;
      if constexpr (S::kTinLds) tl = sm.t[sl] + lane * 8;
      else tl = wy_block(e) + lane * 8;
      load_frag(tfr[0], tl + 0 * 512);
      load_frag(tfr[1], tl + 2 * 512);
      load_frag(tfr[2], tl + 4 * 512);
      load_frag(tfr[3], tl + 5 * 512);
      load_frag(tfr[4], tl + 6 * 512);
      load_frag(tfr[5], tl + 7 * 512);
    }

    // E = T R
    Frag<T> Rb[2][NB];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int b = 0; b < NB; ++b) from_acc(Rb[s][b], R[2 * s][b], R[2 * s + 1][b]);
    f32x4 E[4][NB];
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4)
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        f32x4 acc = zero4();
        acc = mma(tfr[a4 < 2 ? a4 : 2 * a4 - 2], Rb[0][b], acc);
        if (a4 >= 2) acc = mma(tfr[2 * a4 - 1], Rb[1][b], acc);
        E[a4][b] = acc;
      }

    // O^T += E^T P^T  (k-steps whose P block is entirely masked are skipped)
    Frag<T> Eb[2][NB];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int b = 0; b < NB; ++b) from_acc(Eb[s][b], E[2 * s][b], E[2 * s + 1][b]);
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        if ((CH * j + 32 * s) / n > 16 * a4 + 15) continue;
        const Frag<T> pb = lds_perm(sm.p, LDC, 16 * a4 + lr, 32 * s, lg);
#pragma unroll
        for (int b = 0; b < NB; ++b) O[b][a4] = mma(Eb[s][b], pb, O[b][a4]);
      }

    // state update.  True form: S = 2^G_last S + K^T diag(2^(G_last - G) rk) E.
    // Kept lazily: Sst += K^T diag(2^-G rk / lam) E and lam *= 2^G_last, unless
    // lam would fall below LAM_MIN, in which case Sst is rescaled to lam = 1.
    const float glast = gd[CH - 1];
    const float dl = lam * fexp2(glast);
    const bool lazy = dl >= LAM_MIN;
    const float base = lazy ? 0.f : glast;  // exponent offset of the E scaling
    const float rl = lazy ? 1.f / lam : 1.f;
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const int r0 = 16 * a4 + 4 * lg;
      const f32x4 gdv = ld4(gd + r0), rkv = ld4(rk + r0);
      f32x4 f;
#pragma unroll
      for (int i = 0; i < 4; ++i) f[i] = fexp2(base - gdv[i]) * rkv[i] * rl;
#pragma unroll
      for (int b = 0; b < NB; ++b) E[a4][b] *= f;
    }
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int b = 0; b < NB; ++b) from_acc(Eb[s][b], E[2 * s][b], E[2 * s + 1][b]);
    if (!lazy) {
#pragma unroll
      for (int at = 0; at < KT16; ++at)
#pragma unroll
        for (int b = 0; b < NB; ++b) Sacc[at][b] *= dl;
    }
#pragma unroll
    for (int at = 0; at < KT16; ++at) {
      const Frag<T> k0 = lds_perm(sm.kt[sl], LDKT, 16 * at + lr, 0, lg);
      const Frag<T> k1 = lds_perm(sm.kt[sl], LDKT, 16 * at + lr, 32, lg);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        Sacc[at][b] = mma(k0, Eb[0][b], Sacc[at][b]);
        Sacc[at][b] = mma(k1, Eb[1][b], Sacc[at][b]);
      }
    }
    lam = lazy ? dl : 1.f;

    if (e + 1 < nexp) commit(e + 1, sl ^ 1);

    // outputs of token chunk c once its last expanded chunk is in: lane holds
    // O[t = 16 a4 + lr][16 b + 4 lg .. +3] of this wave's columns
    if (j == n - 1 || e == nexp - 1) {
      T *ob = (T *)a.o + (t0 + (int64_t)CH * c) * a.o_st + h * a.o_sh + gcol;
      const uint32_t ost = (uint32_t)a.o_st * ES;
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int t = 16 * a4 + lr;
        if (t < ntok) {
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            const f32x4 x = O[b][a4] * a.scale;
            const uint32_t off = (uint32_t)t * ost + (uint32_t)(16 * b + 4 * lg) * ES;
            if constexpr (sizeof(T) == 2) {
              *(bf16x4 *)((char *)ob + off) = bf16x4{(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]};
            } else {
              *(f32x4 *)((char *)ob + off) = x;
            }
          }
        }
      }
    }
    __syncthreads();
  }

  // final state and cache slot
  float *fdst = a.final_state ? a.final_state + state_off : nullptr;
  float *cdst = nullptr;
  if (a.cache) {
    const int64_t slot = load_index(a.slots, a.slots_is64, seq);
    if (slot >= 0 && slot < a.num_slots) cdst = a.cache + ((size_t)slot * a.Hv + h) * KV;
  }
#pragma unroll
  for (int at = 0; at < KT16; ++at)
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const size_t off = (size_t)(16 * at + 4 * lg + i) * V + gcol + 16 * b + lr;
        const float x = lam * Sacc[at][b][i];
        if (fdst) fdst[off] = x;
        if (cdst) cdst[off] = x;
      }
}

// ---------------------------------------------------------------- fused kernel
//
// One workgroup of 8 waves per (sequence, state head, V-tile) does the whole
// chunked pass, WY step included, so the per-chunk WY matrix never leaves the CU:
//   waves 0-3  consumers: the state S (fp32 accumulators, one 16*NB-column slab
//              per wave), scores, R = beta V - ..., E = T R, the outputs and the
//              state update of expanded chunk e;
//   wave  4    WY wave: row scalars, the Gram matrix, A and T = (I + A)^-1 of
//              chunk e+1, entirely wave-local (a private fp32 LDS tile holds A
//              below the diagonal and T^T on and above it);
//   waves 5-7  loaders: direct global->LDS loads of the k rows of chunk e+2
//              (3-slot ring), the v rows of chunk e+1, the betas and decays of
//              chunk e+2 and the q rows of the next token chunk (2-slot rings),
//              plus the q-row norms and the token-stream decay cumsum.
// Two workgroup barriers per chunk separate the phases; between two barriers
// each role only touches LDS slots no other role uses in that span.  Tiles of
// 64 rows are stored unpadded with an XOR swizzle of their 16-byte segments;
// k^T and v fragments come from the transposing LDS read of gfx950.

typedef short s16x4 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16: inside each group of 16 lanes, lane i receives element
// i % 4 of the 8-byte reads of lanes i/4, i/4 + 4, i/4 + 8 and i/4 + 12.
__device__ __forceinline__ bf16x4 lds_tr4(const char *p) {
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(p));
  return __builtin_bit_cast(bf16x4, r);
}

// Byte offset of (row, byte) in a swizzled tile of rows of W bytes: segment g
// of row r sits at slot g ^ (r mod W/16), so that 16 consecutive rows spread
// one logical segment over all bank groups.
template <int W> __device__ __forceinline__ int sw_off(int row, int byte) {
  constexpr int NS = W / 16;
  return row * W + ((((byte >> 4) ^ row) & (NS - 1)) << 4) + (byte & 15);
}
// bf16 fragments from swizzled tiles (k0, c0 in elements)
template <int W> __device__ __forceinline__ Frag<bf16> sw_contig(const char *t, int row, int k0, int lg) {
  Frag<bf16> f;
  f.v = *(const bf16x8 *)(t + sw_off<W>(row, 2 * (k0 + 8 * lg)));
  return f;
}
template <int W> __device__ __forceinline__ Frag<bf16> sw_perm(const char *t, int row, int k0, int lg) {
  const bf16x4 lo = *(const bf16x4 *)(t + sw_off<W>(row, 2 * (k0 + 4 * lg)));
  const bf16x4 hi = *(const bf16x4 *)(t + sw_off<W>(row, 2 * (k0 + 16 + 4 * lg)));
  Frag<bf16> f;
  f.v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return f;
}
// reduction index down the rows: lane (lr, lg) gets t[k0 + 4lg + j][c0 + lr] and t[k0 + 16 + 4lg + j][c0 + lr]
template <int W> __device__ __forceinline__ Frag<bf16> sw_colfrag(const char *t, int c0, int k0, int lr, int lg) {
  const int row = k0 + 4 * lg + (lr >> 2), byte = 2 * (c0 + 4 * (lr & 3));
  const bf16x4 lo = lds_tr4(t + sw_off<W>(row, byte)), hi = lds_tr4(t + sw_off<W>(row + 16, byte));
  Frag<bf16> f;
  f.v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return f;
}
// rows r0..r0+3 of column c0 + lr (r0 uniform in each 16-lane group)
template <int W> __device__ __forceinline__ f32x4 sw_col4(const char *t, int r0, int c0, int lr) {
  const bf16x4 x = lds_tr4(t + sw_off<W>(r0 + (lr >> 2), 2 * (c0 + 4 * (lr & 3))));
  return f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
}

// Direct global->LDS load of a 64-row tile (rows past nrows repeat the last
// row; they are never used unmasked).  Each wave-wide load fills 1 KiB of LDS,
// 16 bytes per lane in lane order, so the swizzle is applied to the source.
template <int W>
__device__ __forceinline__ void tile_load(char *tile, const char *g, uint32_t rstride, int nrows, int lane) {
  constexpr int NS = W / 16, RPI = 64 / NS;
#pragma unroll
  for (int i = 0; i < 64 / RPI; ++i) {
    const int r = i * RPI + lane / NS, slot = lane % NS;
    const char *src = g + (uint32_t)min(r, nrows - 1) * rstride + (uint32_t)((slot ^ (r & (NS - 1))) << 4);
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)src,
                                     (__attribute__((address_space(3))) void *)(tile + i * 1024), 16, 0, 0);
  }
}
__device__ __forceinline__ void scalar_load(float *dst, const float *src) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)src,
                                   (__attribute__((address_space(3))) void *)dst, 4, 0, 0);
}
__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

template <int K, int NB> struct FusedSmem {
  static constexpr int KW = 2 * K;        // bytes per k / q row
  static constexpr int VW = 2 * 64 * NB;  // bytes per v row of the tile
  static constexpr int LDC = CH + 8;      // P rows (bf16, padded)
  static constexpr int LDA = CH + 4;      // WY tile (fp32)
  char k[3][CH * KW];
  char v[2][CH * VW];
  char q[2][CH * KW];
  bf16 t[2][6 * 64 * 8];
  bf16 p[CH * LDC];
  float wa[CH * LDA];
  float rawb[3][CH], rawg[3][CH], beta[3][CH], gdp[3][CH], rk[3][CH];
  float rawt[2][CH], gtok[2][CH], rq[2][CH];
};

// WY fragment fi = 0..5 <-> (row tile, reduction half): (0,0) (1,0) (2,0) (2,1) (3,0) (3,1)
__device__ __forceinline__ int frag_row(int fi) { return fi < 2 ? fi : (fi < 4 ? 2 : 3); }
__device__ __forceinline__ int frag_half(int fi) { return (fi == 3 || fi == 5) ? 1 : 0; }

// WY wave, first half: the chunk's row scalars (masked beta, base-2 decay
// cumsum, k-row rstd from the Gram diagonal), A below the diagonal, and the
// inverses of the four diagonal 16 x 16 blocks (stored transposed in place).
template <int K, int LDA>
__device__ __forceinline__ void wy_wave_a(const char *k, const float *rawb, const float *rawg, float *beta,
                                          float *gdp, float *rk, float *wa, int nrow, int rem, int n, int l2norm,
                                          int lane) {
  constexpr int KS = K / 32, KW = 2 * K;
  const int lr = lane & 15, lg = lane >> 4;
  {
    const bool valid = lane < nrow;
    const bool decay = valid && ((rem + lane) % n == 0);  // first sub-row of its token
    gdp[lane] = wave_inclusive_sum(decay ? rawg[lane] * LOG2E : 0.f, lane);
    beta[lane] = valid ? rawb[lane] : 0.f;
  }
  f32x4 gram[10];
#pragma unroll
  for (int idx = 0; idx < 10; ++idx) {
    int ra, rb;
    lower_tile(idx, ra, rb);
    f32x4 acc = zero4();
#pragma unroll
    for (int s = 0; s < KS; ++s)
      acc = mma(sw_contig<KW>(k, 16 * ra + lr, 32 * s, lg), sw_contig<KW>(k, 16 * rb + lr, 32 * s, lg), acc);
    gram[idx] = acc;
    if (ra == rb) {  // diagonal tile: lane (lg, lr) holds G[16ra + 4lg + i][16ra + lr]
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * lg + i == lr) rk[16 * ra + lr] = l2norm ? frsq(acc[i] + 1e-6f) : 1.f;
    }
  }
#pragma unroll
  for (int idx = 0; idx < 10; ++idx) {
    int ra, rb;
    lower_tile(idx, ra, rb);
    const int c = 16 * rb + lr, r0 = 16 * ra + 4 * lg;
    const f32x4 bt = ld4(beta + r0), gd = ld4(gdp + r0), rr = ld4(rk + r0);
    const float gc = gdp[c], rc = rk[c];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float val = (c < r0 + i) ? bt[i] * rr[i] * rc * fexp2(gd[i] - gc) * gram[idx][i] : 0.f;
      wa[(r0 + i) * LDA + c] = val;
    }
  }
  // diagonal blocks: lane (block lg, column lr) by forward substitution, carrying
  // the partial sums of the later rows; column lr of T_bb goes to row lr of the block
  const float *Ab = wa + (16 * lg) * LDA + 16 * lg;
  float acc[16], x[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    x[i] = (i == lr ? 1.f : 0.f) - acc[i];
#pragma unroll
    for (int r = i + 1; r < 16; ++r) acc[r] = fmaf(Ab[r * LDA + i], x[i], acc[r]);
  }
  float *d = wa + (16 * lg + lr) * LDA + 16 * lg;
#pragma unroll
  for (int r = 0; r < 16; r += 4) *(f32x4 *)(d + r) = f32x4{x[r], x[r + 1], x[r + 2], x[r + 3]};
}

// WY wave, second half: the off-diagonal blocks T_ab = -T_aa sum_{c=b}^{a-1} A_ac T_cb
// (stored transposed at block (b, a)) and the bf16 fragments of T.
template <int LDA> __device__ __forceinline__ void wy_wave_b(float *wa, bf16 *tout, int lane) {
  const int lr = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int dd = 1; dd < 4; ++dd) {
#pragma unroll
    for (int ba = dd; ba < 4; ++ba) {
      const int bb = ba - dd;
      f32x4 y = zero4();
#pragma unroll
      for (int c = bb; c < ba; ++c)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          y = __builtin_amdgcn_mfma_f32_16x16x4f32(wa[(16 * ba + lr) * LDA + 16 * c + 4 * kk + lg],
                                                    wa[(16 * bb + lr) * LDA + 16 * c + 4 * kk + lg], y, 0, 0, 0);
      f32x4 z = zero4();
#pragma unroll
      for (int i = 0; i < 4; ++i)
        z = __builtin_amdgcn_mfma_f32_16x16x4f32(wa[(16 * ba + 4 * lg + i) * LDA + 16 * ba + lr], y[i], z, 0, 0, 0);
      *(f32x4 *)(wa + (16 * bb + lr) * LDA + 16 * ba + 4 * lg) = -z;
    }
  }
  // lane (lr, lg) of fragment (a4, s) holds T[16 a4 + lr][32 s + 4 lg + i] and
  // T[16 a4 + lr][32 s + 16 + 4 lg + i]; blocks right of the diagonal are zero
#pragma unroll
  for (int fi = 0; fi < 6; ++fi) {
    const int a4 = frag_row(fi), s = frag_half(fi);
    Frag<float> f;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int cb = 2 * s + hh;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        f.v[4 * hh + i] = (cb <= a4) ? wa[(16 * cb + 4 * lg + i) * LDA + 16 * a4 + lr] : 0.f;
    }
    store_frag(tout + (fi * 64 + lane) * 8, f);
  }
}

template <int K, int V, int NB>
__global__ void __launch_bounds__(2 * NTHR, 1) gdp_fused_kernel(PrefillArgs a) {
  using S = FusedSmem<K, NB>;
  constexpr int BV = 64 * NB, NVT = V / BV, KT16 = K / 16, KS = K / 32;
  constexpr int KW = S::KW, VW = S::VW, LDC = S::LDC, LDA = S::LDA;
  __shared__ S sm;

  // the wave index is uniform per wave: role branches below contain barriers
  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

  // Workgroups are dealt to the 8 XCDs round-robin; remap so that each XCD
  // walks a contiguous range of chains (the heads sharing a q/k head, and the
  // V-tiles of one head, then read the same k/q rows through one L2).
  const int64_t G = gridDim.x, bid = blockIdx.x;
  const int64_t chain = (G % 8 == 0) ? (bid % 8) * (G / 8) + bid / 8 : bid;
  const int vt = (int)(chain % NVT);
  const int h = (int)((chain / NVT) % a.Hv);
  const int seq = (int)(chain / ((int64_t)NVT * a.Hv));
  const int hq = h / (a.Hv / a.Hqk);
  const int n = a.n;

  int64_t t0 = load_index(a.cu, a.cu_is64, seq), t1 = load_index(a.cu, a.cu_is64, seq + 1);
  t0 = t0 < 0 ? 0 : (t0 > a.T ? a.T : t0);
  t1 = t1 < t0 ? t0 : (t1 > a.T ? a.T : t1);
  const int64_t L = t1 - t0, nsub = L * n;
  const int nexp = (int)((nsub + CH - 1) / CH);
  const int ntc = (int)((L + CH - 1) / CH);  // token chunks
  const size_t KV = (size_t)K * V;
  const size_t state_off = ((size_t)seq * a.Hv + h) * KV;
  auto rows_of = [&](int e) { return (int)((nsub - (int64_t)CH * e) < CH ? (nsub - (int64_t)CH * e) : CH); };
  auto toks_of = [&](int c) { return (int)((L - (int64_t)CH * c) < CH ? (L - (int64_t)CH * c) : CH); };

  // ------------------------------------------------------------ loaders
  const bf16 *qg = (const bf16 *)a.q + hq * a.q_sh;
  const bf16 *kg = (const bf16 *)a.k + hq * a.k_sh;
  const bf16 *vg = (const bf16 *)a.v + h * a.v_sh + vt * BV;
  const float *gg = a.g + h * a.g_sh;
  const float *bg = a.beta + h * a.b_sh;
  const uint32_t kst = (uint32_t)a.k_st * 2u, vst = (uint32_t)a.v_st * 2u, qst = (uint32_t)a.q_st * 2u;
  auto load_k = [&](int e) {
    tile_load<KW>(sm.k[e % 3], (const char *)(kg + (t0 * n + (int64_t)CH * e) * a.k_st), kst, rows_of(e), lane);
  };
  auto load_v = [&](int e) {
    tile_load<VW>(sm.v[e & 1], (const char *)(vg + (t0 * n + (int64_t)CH * e) * a.v_st), vst, rows_of(e), lane);
  };
  auto load_scalars = [&](int e) {  // raw beta and decay of each sub-row of chunk e
    const int64_t s0 = (int64_t)CH * e;
    const int r = min(lane, rows_of(e) - 1);
    const int64_t tok = (s0 + r) / n;
    scalar_load(sm.rawb[e % 3], bg + (t0 * n + s0 + r) * a.b_st);
    scalar_load(sm.rawg[e % 3], gg + (t0 + tok) * a.g_st);
  };
  auto load_q = [&](int c) {  // q rows and token decays of token chunk c
    const int64_t tokbase = t0 + (int64_t)CH * c;
    tile_load<KW>(sm.q[c & 1], (const char *)(qg + tokbase * a.q_st), qst, toks_of(c), lane);
    scalar_load(sm.rawt[c & 1], gg + (tokbase + min(lane, toks_of(c) - 1)) * a.g_st);
  };
  auto finish_q = [&](int c) {  // after load_q(c) has landed: q-row rstd and token decay cumsum
    const int sl = c & 1, ntok = toks_of(c);
    float ss = 0.f;
    if (a.l2norm) {
#pragma unroll
      for (int sg = 0; sg < KW / 16; ++sg) ss += seg_sumsq<bf16>(*(const uint4 *)(sm.q[sl] + sw_off<KW>(lane, 16 * sg)));
    }
    sm.rq[sl][lane] = a.l2norm ? frsq(ss + 1e-6f) : 1.f;
    sm.gtok[sl][lane] = wave_inclusive_sum(lane < ntok ? sm.rawt[sl][lane] * LOG2E : 0.f, lane);
  };

  // ------------------------------------------------------------ roles
  // Each role runs its own loop with the same barrier sequence (two in the
  // prologue when there is work, two per expanded chunk), so that the
  // registers live in one role never count against another.
  if (w < 4) {
    const int wcol = w * 16 * NB;     // first column of this wave inside the tile
    const int gcol = vt * BV + wcol;  // ... and inside the head
    f32x4 Sacc[KT16][NB];
    f32x4 O[NB][4];
    float lam = 1.f;
#pragma unroll
    for (int at = 0; at < KT16; ++at)
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        if (a.s0) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            Sacc[at][b][i] = a.s0[state_off + (size_t)(16 * at + 4 * lg + i) * V + gcol + 16 * b + lr];
        } else {
          Sacc[at][b] = zero4();
        }
      }
    if (nexp > 0) {
      __syncthreads();
      __syncthreads();
    }
    for (int e = 0; e < nexp; ++e) {
      const int ks = e % 3, ts = e & 1;
      const int c = e / n;
      const int j = e - c * n;
      const int qs = c & 1;
      // lane-derived LDS and global offsets are re-formed every chunk (an opaque
      // copy of the lane index) instead of being hoisted into long-lived registers
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int lr = ln & 15, lg = ln >> 4;
        // ---- phase A: X = K Sst (and at a token-chunk start O^T = Sst^T Q^T), scores, R
        const int nrow = rows_of(e);
        const char *kt = sm.k[ks];
        const char *qt = sm.q[qs];
        const float *rk = sm.rk[ks], *gd = sm.gdp[ks], *bt = sm.beta[ks];
        const float *gtok = sm.gtok[qs], *rqv = sm.rq[qs];
        if (j == 0 && a.chunk_states) {  // state entering token chunk c
          const int64_t row = (int64_t)a.chunk_offsets[seq] + c;
          if (row >= 0 && row < a.cs_rows) {
            // the lane offset is made opaque so that the 16*NB*4 store addresses are
            // formed here rather than hoisted out of the loop into live registers
            uint32_t lo = (uint32_t)(4 * lg * V + gcol + lr);
            asm volatile("" : "+v"(lo));
            float *dst = a.chunk_states + ((size_t)row * a.Hv + h) * KV + lo;
#pragma unroll
            for (int at = 0; at < KT16; ++at)
#pragma unroll
              for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int i = 0; i < 4; ++i) dst[(16 * at + i) * V + 16 * b] = lam * Sacc[at][b][i];
          }
        }
        f32x4 X[4][NB];
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4)
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            X[a4][b] = zero4();
            if (j == 0) O[b][a4] = zero4();
          }
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          Frag<bf16> Sb[NB];
#pragma unroll
          for (int b = 0; b < NB; ++b) from_acc(Sb[b], Sacc[2 * s][b], Sacc[2 * s + 1][b]);
#pragma unroll
          for (int a4 = 0; a4 < 4; ++a4) {
            const Frag<bf16> kf = sw_perm<KW>(kt, 16 * a4 + lr, 32 * s, lg);
#pragma unroll
            for (int b = 0; b < NB; ++b) X[a4][b] = mma(kf, Sb[b], X[a4][b]);
          }
          if (j == 0) {
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4) {
              const Frag<bf16> qf = sw_perm<KW>(qt, 16 * a4 + lr, 32 * s, lg);
#pragma unroll
              for (int b = 0; b < NB; ++b) O[b][a4] = mma(Sb[b], qf, O[b][a4]);
            }
          }
        }
        if (j == 0) {
#pragma unroll
          for (int a4 = 0; a4 < 4; ++a4) {
            const int t = 16 * a4 + lr;
            const float f = lam * fexp2(gtok[t]) * rqv[t];
#pragma unroll
            for (int b = 0; b < NB; ++b) O[b][a4] *= f;
          }
        }
        // scores P[t][r] = rq_t rk_r 2^(Gt_t - Gt_tok(r)) q_t.k_r for tok(r) <= t, tok(r) = (64j + r)/n
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const int tt = w + 4 * it, ta = tt >> 2, tb = tt & 3;
          const bool live = (CH * j + 16 * tb) / n <= 16 * ta + 15;
          f32x4 acc = zero4();
          if (live) {
#pragma unroll
            for (int s = 0; s < KS; ++s)
              acc = mma(sw_contig<KW>(qt, 16 * ta + lr, 32 * s, lg), sw_contig<KW>(kt, 16 * tb + lr, 32 * s, lg), acc);
          }
          const int r = 16 * tb + lr;
          const int tk = (CH * j + r) / n;
          const float colf = (r < nrow) ? rk[r] : 0.f;
          const float gk = gtok[tk];
          const f32x4 gt = ld4(gtok + 16 * ta + 4 * lg), rq = ld4(rqv + 16 * ta + 4 * lg);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = 16 * ta + 4 * lg + i;
            const float val = (live && tk <= t) ? rq[i] * colf * fexp2(gt[i] - gk) * acc[i] : 0.f;
            sm.p[t * LDC + r] = (bf16)val;
          }
        }
        // R = diag(beta) V - diag(beta 2^G rk lam) X, kept in X
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const int r0 = 16 * a4 + 4 * lg;
          const f32x4 btv = ld4(bt + r0), gdv = ld4(gd + r0), rkv = ld4(rk + r0);
          f32x4 coef;
#pragma unroll
          for (int i = 0; i < 4; ++i) coef[i] = btv[i] * fexp2(gdv[i]) * rkv[i] * lam;
#pragma unroll
          for (int b = 0; b < NB; ++b) X[a4][b] = btv * sw_col4<VW>(sm.v[ts], r0, wcol + 16 * b, lr) - coef * X[a4][b];
        }
        __syncthreads();  // P complete
        // ---- phase B: E = T R, O^T += E^T P^T, state update, outputs
        Frag<bf16> tfr[6];
#pragma unroll
        for (int fi = 0; fi < 6; ++fi) load_frag(tfr[fi], sm.t[ts] + (fi * 64 + lane) * 8);
        Frag<bf16> Rb[2][NB];
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int b = 0; b < NB; ++b) from_acc(Rb[s][b], X[2 * s][b], X[2 * s + 1][b]);
        f32x4 E[4][NB];
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4)
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            f32x4 acc = mma(tfr[a4 < 2 ? a4 : 2 * a4 - 2], Rb[0][b], zero4());
            if (a4 >= 2) acc = mma(tfr[2 * a4 - 1], Rb[1][b], acc);
            E[a4][b] = acc;
          }
        Frag<bf16> Eb[2][NB];
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int b = 0; b < NB; ++b) from_acc(Eb[s][b], E[2 * s][b], E[2 * s + 1][b]);
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4)
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            if ((CH * j + 32 * s) / n > 16 * a4 + 15) continue;  // P block entirely masked
            const Frag<bf16> pf = lds_perm(sm.p, LDC, 16 * a4 + lr, 32 * s, lg);
#pragma unroll
            for (int b = 0; b < NB; ++b) O[b][a4] = mma(Eb[s][b], pf, O[b][a4]);
          }
        // Sst += K^T diag(2^-G rk / lam) E and lam *= 2^G_last, unless lam would fall
        // below LAM_MIN (then Sst is rescaled to lam = 1)
        const float glast = gd[CH - 1];
        const float dl = lam * fexp2(glast);
        const bool lazy = dl >= LAM_MIN;
        const float base = lazy ? 0.f : glast;
        const float rl = lazy ? 1.f / lam : 1.f;
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const int r0 = 16 * a4 + 4 * lg;
          const f32x4 gdv = ld4(gd + r0), rkv = ld4(rk + r0);
          f32x4 f;
#pragma unroll
          for (int i = 0; i < 4; ++i) f[i] = fexp2(base - gdv[i]) * rkv[i] * rl;
#pragma unroll
          for (int b = 0; b < NB; ++b) E[a4][b] *= f;
        }
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int b = 0; b < NB; ++b) from_acc(Eb[s][b], E[2 * s][b], E[2 * s + 1][b]);
        if (!lazy) {
#pragma unroll
          for (int at = 0; at < KT16; ++at)
#pragma unroll
            for (int b = 0; b < NB; ++b) Sacc[at][b] *= dl;
        }
#pragma unroll
        for (int at = 0; at < KT16; ++at) {
          const Frag<bf16> k0 = sw_colfrag<KW>(kt, 16 * at, 0, lr, lg);
          const Frag<bf16> k1 = sw_colfrag<KW>(kt, 16 * at, 32, lr, lg);
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            Sacc[at][b] = mma(k0, Eb[0][b], Sacc[at][b]);
            Sacc[at][b] = mma(k1, Eb[1][b], Sacc[at][b]);
          }
        }
        lam = lazy ? dl : 1.f;
        // outputs of token chunk c once its last expanded chunk is in: lane holds
        // O[t = 16 a4 + lr][16 b + 4 lg .. +3] of this wave's columns
        if (j == n - 1 || e == nexp - 1) {
          const int ntok = toks_of(c);
          const uint32_t ost = (uint32_t)a.o_st * 2u;
          uint32_t lo = (uint32_t)lr * ost + (uint32_t)(8 * lg);
          asm volatile("" : "+v"(lo));
          char *ob = (char *)((bf16 *)a.o + (t0 + (int64_t)CH * c) * a.o_st + h * a.o_sh + gcol) + lo;
#pragma unroll
          for (int a4 = 0; a4 < 4; ++a4) {
            if (16 * a4 + lr < ntok) {
#pragma unroll
              for (int b = 0; b < NB; ++b) {
                const f32x4 x = O[b][a4] * a.scale;
                *(bf16x4 *)(ob + (uint32_t)(16 * a4) * ost + 32 * b) = bf16x4{(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]};
              }
            }
          }
        }
      __syncthreads();
    }
    float *fdst = a.final_state ? a.final_state + state_off : nullptr;
    float *cdst = nullptr;
    if (a.cache) {
      const int64_t slot = load_index(a.slots, a.slots_is64, seq);
      if (slot >= 0 && slot < a.num_slots) cdst = a.cache + ((size_t)slot * a.Hv + h) * KV;
    }
#pragma unroll
    for (int at = 0; at < KT16; ++at)
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const size_t off = (size_t)(16 * at + 4 * lg + i) * V + gcol + 16 * b + lr;
          const float x = lam * Sacc[at][b][i];
          if (fdst) fdst[off] = x;
          if (cdst) cdst[off] = x;
        }
  } else if (w == 4) {
    // WY wave: T of chunk 0 in the prologue, then T of chunk e+1 during chunk e
    // (its k rows and raw scalars landed before the barrier that opened chunk e)
    if (nexp > 0) {
      __syncthreads();
      wy_wave_a<K, LDA>(sm.k[0], sm.rawb[0], sm.rawg[0], sm.beta[0], sm.gdp[0], sm.rk[0], sm.wa, rows_of(0), 0, n,
                        a.l2norm, lane);
      wy_wave_b<LDA>(sm.wa, sm.t[0], lane);
      __syncthreads();
    }
    for (int e = 0; e < nexp; ++e) {
      const bool has = e + 1 < nexp;
      const int k1 = (e + 1) % 3;
      if (has)
        wy_wave_a<K, LDA>(sm.k[k1], sm.rawb[k1], sm.rawg[k1], sm.beta[k1], sm.gdp[k1], sm.rk[k1], sm.wa,
                          rows_of(e + 1), (int)(((int64_t)CH * (e + 1)) % n), n, a.l2norm, lane);
      __syncthreads();
      if (has) wy_wave_b<LDA>(sm.wa, sm.t[(e + 1) & 1], lane);
      __syncthreads();
    }
  } else if (w == 5) {
    // k rows: chunks 0 and 1 in the prologue, chunk e+2 during chunk e
    if (nexp > 0) {
      load_k(0);
      if (nexp > 1) load_k(1);
      wait_vm();
      __syncthreads();
      __syncthreads();
    }
    for (int e = 0; e < nexp; ++e) {
      if (e + 2 < nexp) load_k(e + 2);
      __syncthreads();
      wait_vm();
      __syncthreads();
    }
  } else if (w == 6) {
    // v rows: chunk 0 in the prologue, chunk e+1 during chunk e
    if (nexp > 0) {
      load_v(0);
      wait_vm();
      __syncthreads();
      __syncthreads();
    }
    for (int e = 0; e < nexp; ++e) {
      if (e + 1 < nexp) load_v(e + 1);
      __syncthreads();
      wait_vm();
      __syncthreads();
    }
  } else {
    // betas and decays of chunk e+2, q rows of token chunk c+1 from the start of
    // token chunk c, and their norms and decay cumsum once they have landed
    if (nexp > 0) {
      load_scalars(0);
      if (nexp > 1) load_scalars(1);
      load_q(0);
      wait_vm();
      finish_q(0);
      __syncthreads();
      __syncthreads();
    }
    for (int e = 0; e < nexp; ++e) {
      const int c = e / n;
      const int j = e - c * n;
      if (e + 2 < nexp) load_scalars(e + 2);
      if (j == 0 && c + 1 < ntc) load_q(c + 1);
      __syncthreads();
      wait_vm();
      if ((e + 1) % n == 0 && c + 1 < ntc) finish_q(c + 1);
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------- descriptors
//
// Megatron Core page, chunk_indices / chunk_indices_dp / chunk_offsets: one
// workgroup scans the per-sequence chunk counts 1024 sequences at a time
// (carrying the running totals), writes the offsets, and fills the rows of
// those sequences by binary search over the tile's offsets in LDS; the
// remaining rows up to the capacities are padded with (-1, -1).

__device__ __forceinline__ void block_scan_2(int64_t &xa, int64_t &xb, int64_t *wsa, int64_t *wsb,
                                             int64_t &tota, int64_t &totb) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t ya = __shfl_up(xa, off), yb = __shfl_up(xb, off);
    if (lane >= off) { xa += ya; xb += yb; }
  }
  if (lane == 63) { wsa[w] = xa; wsb[w] = xb; }
  __syncthreads();
  if (tid == 0) {
    int64_t ra = 0, rb = 0;
    for (int i = 0; i < 16; ++i) {
      const int64_t ta = wsa[i], tb = wsb[i];
      wsa[i] = ra; wsb[i] = rb;
      ra += ta; rb += tb;
    }
    wsa[16] = ra; wsb[16] = rb;
  }
  __syncthreads();
  xa += wsa[w]; xb += wsb[w];  // inclusive
  tota = wsa[16]; totb = wsb[16];
}

__global__ void __launch_bounds__(1024) gdp_descriptor_kernel(DescArgs a) {
  __shared__ int64_t st[1025], sd[1025];
  __shared__ int64_t wsa[17], wsb[17];
  const int tid = threadIdx.x;
  int64_t carry_t = 0, carry_d = 0;
  for (int64_t base = 0; base < a.N; base += 1024) {
    const int64_t i = base + tid;
    int64_t ct = 0, cd = 0;
    if (i < a.N) {
      int64_t L = load_index(a.cu, a.cu_is64, i + 1) - load_index(a.cu, a.cu_is64, i);
      if (L < 0) L = 0;
      ct = (L + CH - 1) / CH;
      cd = (L * a.n + CH - 1) / CH;
    }
    int64_t xt = ct, xd = cd, tot_t, tot_d;
    block_scan_2(xt, xd, wsa, wsb, tot_t, tot_d);
    st[tid + 1] = carry_t + xt;
    sd[tid + 1] = carry_d + xd;
    if (tid == 0) { st[0] = carry_t; sd[0] = carry_d; }
    if (i < a.N) {
      a.chunk_offsets[i] = (int32_t)(carry_t + xt - ct);
      a.chunk_offsets_dp[i] = (int32_t)(carry_d + xd - cd);
    }
    __syncthreads();
    const int cnt = (int)((a.N - base) < 1024 ? (a.N - base) : 1024);
    for (int pass = 0; pass < 2; ++pass) {
      const int64_t *so = pass ? sd : st;
      int32_t *rows = pass ? a.chunk_indices_dp : a.chunk_indices;
      const int64_t cap = pass ? a.ntdp_cap : a.nt_cap;
      const int64_t r1 = so[cnt] < cap ? so[cnt] : cap;
      for (int64_t p = so[0] + tid; p < r1; p += 1024) {
        int lo = 0, hi = cnt - 1;  // largest j with so[j] <= p
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (so[mid] <= p) lo = mid; else hi = mid - 1;
        }
        rows[2 * p] = (int32_t)(base + lo);
        rows[2 * p + 1] = (int32_t)(p - so[lo]);
      }
    }
    carry_t += tot_t;
    carry_d += tot_d;
    __syncthreads();
  }
  if (tid == 0) {
    a.chunk_offsets[a.N] = (int32_t)carry_t;
    a.chunk_offsets_dp[a.N] = (int32_t)carry_d;
  }
  for (int64_t p = carry_t + tid; p < a.nt_cap; p += 1024) a.chunk_indices[2 * p] = a.chunk_indices[2 * p + 1] = -1;
  for (int64_t p = carry_d + tid; p < a.ntdp_cap; p += 1024)
    a.chunk_indices_dp[2 * p] = a.chunk_indices_dp[2 * p + 1] = -1;
}

// ---------------------------------------------------------------- launchers

namespace {
template <typename T, int K, int V, int NB>
hipError_t launch_scan(const PrefillArgs &a, hipStream_t stream) {
  constexpr int NVT = V / (64 * NB);
  const int64_t blocks = (int64_t)a.N * a.Hv * NVT;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((gdp_scan_kernel<T, K, V, NB>), dim3((unsigned)blocks), dim3(NTHR), 0, stream, a);
  return hipGetLastError();
}

template <typename T, int K, int V>
hipError_t launch_split(const PrefillArgs &a, hipStream_t stream) {
  const int64_t wy_blocks = a.ntdp_rows * a.Hqk;
  if (wy_blocks > 0) {
    hipLaunchKernelGGL((gdp_wy_kernel<T, K>), dim3((unsigned)wy_blocks), dim3(NTHR), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // Wider V-tiles when there are enough chains to fill the chip; narrower
  // ones otherwise, so that few long chains still spread over more CUs.
  if constexpr (V == 128 && sizeof(T) == 2) {
    if ((int64_t)a.N * a.Hv * 2 > 256) return launch_scan<T, K, V, 2>(a, stream);
  }
  return launch_scan<T, K, V, 1>(a, stream);
}

template <int K, int V>
hipError_t launch_fused(const PrefillArgs &a, hipStream_t stream) {
  const int64_t blocks = (int64_t)a.N * a.Hv;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((gdp_fused_kernel<K, V, V / 64>), dim3((unsigned)blocks), dim3(2 * NTHR), 0, stream, a);
  return hipGetLastError();
}

// The fused kernel keeps one chain per CU busy for its whole length; it is
// chosen when there are enough chains to give every CU one.  Otherwise the
// split pair (parallel WY kernel, then the scan) spreads the WY work of few
// long chains over the whole chip.
template <typename T, int K, int V>
hipError_t launch_all(const PrefillArgs &a, int path, hipStream_t stream) {
  if constexpr (sizeof(T) == 2) {
    const bool fused = path == PATH_FUSED || (path == PATH_AUTO && (int64_t)a.N * a.Hv >= 256);
    if (fused) return launch_fused<K, V>(a, stream);
  }
  return launch_split<T, K, V>(a, stream);
}
}  // namespace

bool prefill_supported(int dtype, int K, int V) {
  const bool kv = (K == 64 || K == 128) && (V == 64 || V == 128);
  if (dtype == IN_BF16) return kv;
  if (dtype == IN_F32) return kv && K == 64;
  return false;
}

size_t wy_buffer_bytes(int dtype, int64_t rows, int64_t Hv) {
  return (size_t)rows * (size_t)Hv * CH * CH * (dtype == IN_BF16 ? 2 : 4);
}

hipError_t launch_prefill(const PrefillArgs &a, int dtype, int K, int V, int path, hipStream_t stream) {
  if (dtype == IN_BF16) {
    if (K == 128 && V == 128) return launch_all<bf16, 128, 128>(a, path, stream);
    if (K == 128 && V == 64) return launch_all<bf16, 128, 64>(a, path, stream);
    if (K == 64 && V == 128) return launch_all<bf16, 64, 128>(a, path, stream);
    if (K == 64 && V == 64) return launch_all<bf16, 64, 64>(a, path, stream);
  } else if (dtype == IN_F32) {
    if (K == 64 && V == 64) return launch_all<float, 64, 64>(a, path, stream);
    if (K == 64 && V == 128) return launch_all<float, 64, 128>(a, path, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_descriptors(const DescArgs &a, hipStream_t stream) {
  hipLaunchKernelGGL(gdp_descriptor_kernel, dim3(1), dim3(1024), 0, stream, a);
  return hipGetLastError();
}

}  // namespace gdp
