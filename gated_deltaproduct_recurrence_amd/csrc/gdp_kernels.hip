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

#include <cstdlib>
#include <cstring>

#include "gdp_common.h"
#include "gdp_launch.h"

namespace gdp {


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
    if constexpr (sizeof(T) == 2) {  // both bf16 squares of the word in one v_dot2c_f32_bf16
      typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
      const bf16x2 v = __builtin_bit_cast(bf16x2, w);
      a = __builtin_amdgcn_fdot2_f32_bf16(v, v, a, false);
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

  const int64_t p = blockIdx.x / a.Hk;
  const int hk = (int)(blockIdx.x % a.Hk);  // k head; its state heads share the Gram tiles
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

  load_rows<T, K, LDK>(sm.u.k, (const T *)a.k + hk * a.k_sh + row0 * a.k_st, a.k_st, nrow, tid);
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

  const int grp = a.Hv / a.Hk;
  for (int hh = 0; hh < grp; ++hh) {
    const int h = hk * grp + hh;
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
  const int hq = h / (a.Hv / a.Hqk), hk = h / (a.Hv / a.Hk);
  const int n = a.n;

  int64_t t0 = load_index(a.cu, a.cu_is64, seq), t1 = load_index(a.cu, a.cu_is64, seq + 1);
  t0 = t0 < 0 ? 0 : (t0 > a.T ? a.T : t0);
  t1 = t1 < t0 ? t0 : (t1 > a.T ? a.T : t1);
  const int64_t L = t1 - t0, nsub = L * n;
  const int nexp = (int)((nsub + CH - 1) / CH);
  const int wcol = w * 16 * NB;     // first column of this wave inside the tile
  const int gcol = vt * BV + wcol;  // ... and inside the head

  const T *qg = (const T *)a.q + hq * a.q_sh;
  const T *kg = (const T *)a.k + hk * a.k_sh;
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
// One workgroup of 8 waves per (sequence, state head) does the whole chunked
// pass, WY step included, so the per-chunk WY matrix never leaves the CU:
//   waves 0-3  consumers: the state S (fp32 accumulators, one 16*NB-column slab
//              per wave), X = K S, the scores, R, E = T R, the state update of
//              expanded chunk e, and the outputs, which they store to o;
//   waves 4-7  helpers: wave 4 issues every direct global->LDS load (the k rows
//              and the betas and decays of chunk e+2 in 3-slot rings, the v
//              rows of chunk e+1 and the q rows of token chunk c+2 in 2-slot
//              rings) and forms the masked betas, the decay cumsums, the
//              q-row norms and the per-row token tables; waves 5-7 run the WY
//              step of chunk e+1 (Gram matrix, k-row norms, A, T = (I + A)^-1),
//              the per-row coefficients the consumers use and, on wave 5, the
//              chunk's scale scalars.
// Two workgroup barriers per chunk separate the phases; between two barriers
// each role only touches LDS slots no other role uses in that span.  Tiles of
// 64 rows are stored unpadded with an XOR swizzle of their 16-byte segments;
// k^T, v and T fragments come from the transposing LDS read of gfx950.
//
// WY step on one wave: the Gram tiles are formed with the k rows of the later
// block as the B operand, so each lane ends up holding a row of A (the A-operand
// layout of a 16 x 16 x 16 product).  The four diagonal 16 x 16 blocks are
// inverted by row substitution, all four at once, with the rows already solved
// broadcast across each 16-lane row by DPP (row_newbcast); the blocks below the
// diagonal then follow from T_ab = -T_aa sum_{c=b}^{a-1} A_ac T_cb on bf16 MFMA.

typedef short s16x4 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16: inside each group of 16 lanes, lane i receives element
// i % 4 of the 8-byte reads of lanes i/4, i/4 + 4, i/4 + 8 and i/4 + 12.
__device__ __forceinline__ bf16x4 lds_tr4(const char *p) {
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(p));
  return __builtin_bit_cast(bf16x4, r);
}

// Tiles of 64 rows of W bytes are stored with their 16-byte segments permuted
// per row: segment g of row r sits at slot g ^ swz(r).  The permutation depends
// on how the tile is read (measured on gfx950, where 16-byte reads are served
// 16 lanes at a time and 8-byte reads, plain or transposing, 32 at a time):
//   TK = 1, k and q tiles (256-byte rows): swz(r) = 2 (r mod 8).  16 lanes
//     reading one segment of 16 consecutive rows (the k/q fragments) meet two
//     segments' worth of distinct slots; the transposing k^T reads (8 rows x 4
//     segments per 32 lanes) are served at the same rate as with any other
//     row permutation tried.
//   TK = 0, v tiles (256-byte rows): r = 8m + t (t < 8) maps to 2t + (t / 4 xor m),
//     a bijection on 16 rows, which keeps the transposing v reads at the
//     conflict-free rate.
// Tiles of 128-byte rows keep swz(r) = r mod 8.
template <int NS, int TK = 0> __device__ __forceinline__ int swz(int r) {
  static_assert(NS == 16 || NS == 8, "rows of 128 or 256 bytes");
  if constexpr (NS == 16 && TK == 1) return (r & 7) << 1;
  if constexpr (NS == 16) return ((r & 7) << 1) | (((r >> 2) ^ (r >> 3)) & 1);
  return r & 7;
}
template <int W, int TK = 0> __device__ __forceinline__ int sw_off(int row, int byte) {
  constexpr int NS = W / 16;
  return row * W + ((((byte >> 4) ^ swz<NS, TK>(row)) & (NS - 1)) << 4) + (byte & 15);
}
// bf16 fragment from a swizzled tile: row `row`, reduction slots k0 + 8lg .. +7
template <int W, int TK = 0> __device__ __forceinline__ Frag<bf16> sw_contig(const char *t, int row, int k0, int lg) {
  Frag<bf16> f;
  f.v = *(const bf16x8 *)(t + sw_off<W, TK>(row, 2 * (k0 + 8 * lg)));
  return f;
}
// the same from an unswizzled bf16 tile with a row stride of ld elements
__device__ __forceinline__ bf16x4 tr_col4(const bf16 *t, int ld, int r0, int c0, int lr) {
  return lds_tr4((const char *)(t + (r0 + (lr >> 2)) * ld + c0 + 4 * (lr & 3)));
}

__device__ __forceinline__ f32x4 mma16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x4 bf4(f32x4 x) { return bf16x4{(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]}; }

// Per-lane part of a family of accesses to a swizzled tile of rows of W bytes:
// the lane's row r (taken mod W/16) and byte b inside its row.  The access at
// row R + r (R a multiple of W/16) and byte B + b (B a multiple of 16 below W
// whose segment bits do not overlap those of b) sits at
// R * W + l + (B ^ x) with l = r * W + (b mod 16), x = 16 ((b / 16) ^ swz(r)).
struct SwLane {
  uint32_t l, x;
};
template <int N> struct IC {
  static constexpr int value = N;
};
template <int W, int TK = 0> __device__ __forceinline__ SwLane sw_lane(int r, int b) {
  constexpr int NS = W / 16;
  return SwLane{(uint32_t)(r * W + (b & 15)), (uint32_t)((((b >> 4) ^ swz<NS, TK>(r)) & (NS - 1)) << 4)};
}

// DPP move of x (row mask ROWS; lanes of disabled rows and lanes whose source
// lies outside their row read 0)
template <int CTRL, int ROWS = 0xF> __device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROWS, 0xF, true));
}
// inclusive prefix sum over the 64 lanes: shifts inside each 16-lane row, then
// row 0's total into row 1 (and row 2's into row 3), then lane 31 into rows 2, 3
__device__ __forceinline__ float wave_scan(float x) {
  x += dpp<0x111>(x);       // row_shr:1
  x += dpp<0x112>(x);       // row_shr:2
  x += dpp<0x114>(x);       // row_shr:4
  x += dpp<0x118>(x);       // row_shr:8
  x += dpp<0x142, 0xA>(x);  // row_bcast:15
  x += dpp<0x143, 0xC>(x);  // row_bcast:31
  return x;
}

// Row substitution for a unit-lower-triangular 16 x 16 system (I + L) T = I:
// lane (lg, lr) holds row lr of -L (nl) and the entries T[lr][4lg + i]; step m
// adds -L[lr][m] times row m, which lane (lg, m) of the same 16-lane row holds:
// v_fmac_f32 with its first source read through DPP row_newbcast:m.  Each step
// is one block of inline assembly (the compiler does not fold a DPP move into
// an fmac).  A register written by step m-1 is read through DPP 3 instructions
// later, and each block starts with 2 wait states for whatever the compiler
// placed right before it: the VALU-write -> DPP-read hazard needs 2.
template <int M> __device__ __forceinline__ void subst(float (&t)[4], const float (&nl)[16]) {
  asm volatile("s_nop 1\n"
               "v_fmac_f32_dpp %0, %0, %4 row_newbcast:%5 row_mask:0xf bank_mask:0xf\n"
               "v_fmac_f32_dpp %1, %1, %4 row_newbcast:%5 row_mask:0xf bank_mask:0xf\n"
               "v_fmac_f32_dpp %2, %2, %4 row_newbcast:%5 row_mask:0xf bank_mask:0xf\n"
               "v_fmac_f32_dpp %3, %3, %4 row_newbcast:%5 row_mask:0xf bank_mask:0xf\n"
               : "+v"(t[0]), "+v"(t[1]), "+v"(t[2]), "+v"(t[3])
               : "v"(nl[M]), "i"(M));
  if constexpr (M < 14) subst<M + 1>(t, nl);
}

// Direct global->LDS load of a 64-row tile (rows past nrows repeat the last
// row; they are never used unmasked).  Each wave-wide load fills 1 KiB of LDS,
// 16 bytes per lane in lane order, so the swizzle is applied to the source.
template <int W, int TK = 0>
__device__ __forceinline__ void tile_load(char *tile, const char *g, uint32_t rstride, int nrows, int lane) {
  constexpr int NS = W / 16, RPI = 64 / NS;
#pragma unroll
  for (int i = 0; i < 64 / RPI; ++i) {
    const int r = i * RPI + lane / NS, slot = lane % NS;
    const char *src = g + (uint32_t)min(r, nrows - 1) * rstride + (uint32_t)((slot ^ swz<NS, TK>(r)) << 4);
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)src,
                                     (__attribute__((address_space(3))) void *)(tile + i * 1024), 16, 0, 0);
  }
}
// The same for a full tile, with the per-lane source offsets of its 64*W/1024
// loads computed once (they depend only on the row stride): the loads then take
// a uniform base plus a 32-bit lane offset and need no address arithmetic.
// Lane offsets of a full 64-row tile load.  Row r = RPI i + lane / NS of load i
// has the swizzle of r mod 16 (256-byte rows) or r mod 8 (128-byte rows), so
// only PER distinct lane offsets exist; the row offset RPI i rs is uniform.
template <int W, int TK = 0> struct TileOffs {
  static constexpr int NS = W / 16, RPI = 64 / NS, PER = (NS == 16 ? 16 : 8) / RPI;
  uint32_t o[PER];
  uint32_t rs;  // row stride in bytes
};
template <int W, int TK = 0> __device__ __forceinline__ TileOffs<W, TK> tile_offs(uint32_t rstride, int lane) {
  using TO = TileOffs<W, TK>;
  TO t;
  t.rs = rstride;
#pragma unroll
  for (int p = 0; p < TO::PER; ++p) {
    const int r = p * TO::RPI + lane / TO::NS, slot = lane % TO::NS;
    t.o[p] = (uint32_t)(lane / TO::NS) * rstride + (uint32_t)((slot ^ swz<TO::NS, TK>(r)) << 4);
  }
  return t;
}
template <int W, int TK = 0>
__device__ __forceinline__ void tile_load_full(char *tile, const char *g, const TileOffs<W, TK> &t) {
  using TO = TileOffs<W, TK>;
#pragma unroll
  for (int i = 0; i < 64 / TO::RPI; ++i) {
    const char *gr = g + (uint32_t)(i * TO::RPI) * t.rs;  // uniform
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)(gr + t.o[i % TO::PER]),
                                     (__attribute__((address_space(3))) void *)(tile + i * 1024), 16, 0, 0);
  }
}
__device__ __forceinline__ void scalar_load(float *dst, const float *src) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)src,
                                   (__attribute__((address_space(3))) void *)dst, 4, 0, 0);
}
__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)
// Workgroup barrier for LDS traffic only: this wave's LDS accesses are complete
// (lgkmcnt(0)) and no memory access moves across it, but outstanding global
// loads and stores stay in flight (__syncthreads would wait for them, which
// turns every prefetch and output store into a stall).  A wave whose
// direct-to-LDS loads feed the next phase waits for them itself before it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// pacing of the chains that share a q/k head (fused kernel): checked every
// PACE_EVERY chunks, a chain may lead the others of its group by PACE_AHEAD
// chunks, and a check polls at most PACE_SPIN times.  Measured on the
// long-context workload (pairs of state heads per q/k head): without pacing
// the pairs drift apart and HBM fetch grows from 15.3 to 17-20 GB per call;
// with these values it stays at 15.3 GB at no measurable cost in time.
constexpr int PACE_EVERY = 8, PACE_AHEAD = 4, PACE_SPIN = 500;

template <int K, int V> struct FusedSmem {
  static constexpr int KW = 2 * K;        // bytes per k / q row
  static constexpr int VW = 2 * V;       // bytes per v row
  static constexpr int LDC = CH + 8;      // P rows (bf16, padded)
  static constexpr int LDT = CH + 16;     // rows of T^T (bf16, padded)
  char k[3][CH * KW];
  char v[2][CH * VW];
  char q[2][CH * KW];
  bf16 t[CH * LDT];         // T^T of the chunk being consumed: entry (r, c) of T at
                            // [c * LDT + (r ^ (8 ((c / 8) mod 2)))], the xor halving the
                            // bank conflicts of the 16-row stores without costing the
                            // transposing reads any
  bf16 p[CH * LDC];         // P: entry (t, r) with r = 32 s + 16 h + 4 g + i at
                            // [t * LDC + 32 s + 8 g + 4 h + i], so that a lane's 8 values of
                            // an MFMA operand are one 16-byte read
  float gram[10][64 * 4];   // Gram tiles of the next chunk, lane order; the diagonal
                            // ones are then reused for the rows of -L
  bf16 alow[6][256];        // A below the diagonal blocks, row-major 16 x 16
  bf16 tdiag[4][64 * 4];    // diagonal blocks of T (A-operand layout, lane order)
  bf16 tdrow[4][256];       // diagonal blocks of T, row-major
  float rawb[2][CH], rawg[2][CH];          // raw betas / decays
  float beta[3][CH], gdp[3][CH];           // masked betas, base-2 decay cumsum
  float rk[2][CH], c1[2][CH], wgt[2][CH];  // k-row rstd, 2^G rk (the X weights of R) and the state-update weights
  float rawt[2][CH], gtok[2][CH], rq[2][CH], qfac[2][CH];  // rq: q-row rstd; qfac carries the output scale
  float gkr[2][CH], rkg[2][CH];  // rkg = rk 2^(-Gt_tok(r)) (used when qsafe)
  int tokr[2][CH];
  int qsafe[2];                   // the token chunk's decay cumsum stays above -100 (base 2)
  float scal[2][4];               // per expanded chunk: lazy scale entering it, that scale times the
                                  // chunk's decay, the reciprocal the state update uses, unused
  int sflag[2];                   // per expanded chunk: SF_* bits
};
// Bits of FusedSmem::sflag.  A "fast" token chunk keeps the lazy scale above
// LAM_MIN through all of its expanded chunks (a rescale, when needed, is done at
// its start): its outputs are then formed from the raw masked scores and the
// state-update rows E_w = diag(f) E, with every per-row and per-token factor
// collected at staging.
constexpr int SF_FAST = 1, SF_LAZY = 2, SF_RESCALE = 4, SF_TF = 8;

// SUM: segment summaries only (the states of the segmented path): no outputs,
// so the scores, P, O^T, the q rows and the per-row token tables are skipped.
// One workgroup forms both summaries of its segment, which share the k rows,
// the decays and the WY matrix: NCW = 8 consumer waves, waves 0-3 holding B
// (zero start state, the real values) and waves 4-7 holding M (identity start
// state, zero values, so their E = T Y has no V term).
// LT = 2 (n = 2 only): outputs per expanded chunk.  With two Householder rows
// per token an expanded chunk holds whole tokens (32 of them, token blocks 2j
// and 2j+1 of its token chunk), so each token's output is the state entering
// that expanded chunk read out with q_t, plus the masked scores against that
// chunk's rows only: O^T (two token blocks), the scores (eight tiles) and the
// O += E P^T product (half the rows) are spread evenly over the two expanded
// chunks of a token chunk, and all the decay factors are those of the
// expanded-stream cumsum.  LT = 0: outputs per token chunk (any n).
template <int K, int V, int NCW, bool SUM, int LT = 0>
__global__ void __launch_bounds__(64 * (NCW + 4), 1) gdp_fused_kernel(PrefillArgs a) {
  static_assert(LT == 0 || (LT == 2 && !SUM && NCW == 4), "per-expanded-chunk outputs: n = 2, four consumer waves");
  static_assert(!SUM || (NCW == 8 && K == V), "summaries: four consumer waves each for B and M");
  using S = FusedSmem<K, V>;
  // NCG consumer waves of 16 NB state columns each cover all V columns (in
  // summary mode once for B and once for M); the 16 score tiles (4 token
  // blocks x 4 row blocks) are shared out RBW per wave
  constexpr int NCG = SUM ? NCW / 2 : NCW;
  constexpr int NB = V / (16 * NCG), BV = V, NVT = 1, KT16 = K / 16, KS = K / 32;
  constexpr int RBW = LT ? 2 : 16 / NCW;   // score row blocks per wave
  constexpr int OTB = LT ? LT : 4;          // token blocks of O per wave
  static_assert(NB >= 1 && 16 * NB * NCG == V && (LT || SUM || RBW * NCW == 16), "consumer waves must tile V and the scores");
  constexpr int KW = S::KW, VW = S::VW, LDC = S::LDC, LDT = S::LDT;
  // 16-byte alignment lets the 8- and 16-byte LDS accesses below compile to
  // single b64 / b128 instructions (at 4-byte alignment an 8-byte store is split
  // into a write2_b32 that takes twice the cycles)
  __shared__ __attribute__((aligned(16))) S sm;

  // the wave index is uniform per wave: role branches below contain barriers
  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

  // Workgroups are dealt to the 8 XCDs round-robin; remap so that each XCD
  // walks a contiguous range of chains (the heads sharing a q/k head, and the
  // V-tiles of one head, then read the same k/q rows through one L2).
  const int64_t G = gridDim.x, bid = blockIdx.x;
  const int64_t chain = a.order ? (int64_t)a.order[bid] : ((G % 8 == 0) ? (bid % 8) * (G / 8) + bid / 8 : bid);
  const int vt = (int)(chain % NVT);
  const int h = (int)((chain / NVT) % a.Hv);
  const int seq = (int)(chain / ((int64_t)NVT * a.Hv));
  const int hq = h / (a.Hv / a.Hqk), hk = h / (a.Hv / a.Hk);
  const int n = LT ? LT : a.n;  // per-expanded-chunk outputs are launched for n = 2 only

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

  // the consumer body, instantiated per half of the score row blocks so that
  // every register array index is a compile-time constant
  auto consumer = [&](auto halfc) {
    constexpr int rb0 = decltype(halfc)::value * RBW;
    constexpr bool MP = SUM && decltype(halfc)::value == 1;  // a wave of the M summary
    // ---------------------------------------------------------------- consumers
    const int wcol = (w % NCG) * 16 * NB;  // first column of this wave inside the tile
    // the wave's score tiles: token block tb, row blocks rb0 .. rb0 + RBW - 1 (with
    // LT, tb is the token block inside the expanded chunk's 32 tokens)
    const int tb = LT ? (w >> 1) : (w & 3);
    const int gcol = vt * BV + wcol;  // ... and inside the head
    const char *smb = (const char *)&sm;
    auto off_of = [&](const void *p) { return (uint32_t)((const char *)p - smb); };
    auto rd8 = [&](uint32_t at) { return *(const bf16x4 *)(smb + at); };
    auto rd16 = [&](uint32_t at) { return *(const bf16x8 *)(smb + at); };
    auto tr8 = [&](uint32_t at) { return lds_tr4(smb + at); };
    // per-lane parts of the LDS addresses; each access below is one xor-add of a
    // compile-time segment offset plus an immediate row offset
    const int rl0 = 4 * lg + (lr >> 2);  // row of a transposing read inside its 16-row group
    const SwLane Lcont = sw_lane<KW, 1>(lr, 16 * lg);         // k / q rows, reduction slots 8lg..
    const SwLane Lcolk = sw_lane<KW, 1>(rl0, 16 * (lr & 3));  // k^T fragments (state-row order)
    // (the v-column, T^T-column and P-row parts are re-derived every chunk
    // from the lane index, which keeps them out of the registers live across
    // the chunk loop)
    // The state rows are kept in a permuted key order: accumulator row 4g + i of
    // tile at holds key kap(at, g, i) = 32 (at / 2) + 8 g + 4 (at % 2) + i, so that
    // the two tiles of one 32-deep reduction step form the B operand whose slots
    // pair with contiguous 16-byte k (or q) fragments.
    auto kap = [](int at, int g, int i) { return 32 * (at >> 1) + 8 * g + 4 * (at & 1) + i; };
    f32x4 Sacc[KT16][NB];
    f32x4 O[NB][OTB];
    float lam = 1.f;
#pragma unroll
    for (int at = 0; at < KT16; ++at)
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        if constexpr (MP) {
#pragma unroll
          for (int i = 0; i < 4; ++i) Sacc[at][b][i] = kap(at, lg, i) == gcol + 16 * b + lr ? 1.f : 0.f;
        } else if (a.s0) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            Sacc[at][b][i] = a.s0[state_off + (size_t)kap(at, lg, i) * V + gcol + 16 * b + lr];
        } else {
          Sacc[at][b] = zero4();
        }
      }
    const int64_t cs_row0 = a.chunk_states ? (int64_t)a.chunk_offsets[seq] : 0;
    // the state entering token chunk cc, lam Sst, into its chunk_states row
    auto store_chunk_state = [&](int cc) {
      const int64_t row = cs_row0 + cc;
      if (row >= 0 && row < a.cs_rows) {
        uint32_t lo = (uint32_t)(8 * lg * V + gcol + lr);
        asm volatile("" : "+v"(lo));
        float *dst = a.chunk_states + ((size_t)row * a.Hv + h) * KV + lo;
#pragma unroll
        for (int at = 0; at < KT16; ++at)
#pragma unroll
          for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[kap(at, 0, i) * V + 16 * b] = lam * Sacc[at][b][i];
      }
    };
    // With per-token-chunk outputs, token chunk 0 enters with the start state
    // and the state entering token chunk c + 1 is stored at the end of token
    // chunk c, after its last state update, where no load of the loader shares
    // the vector memory path with the stores (lam Sst is unchanged by the
    // rescale that may open the next chunk).  With per-expanded-chunk outputs
    // it is stored at the start of each token chunk.
    if constexpr (!LT) {
      if (a.chunk_states && nexp > 0) store_chunk_state(0);
    }
    // wait for the start state here: a wait placed by the compiler at its first
    // use inside the loop would also wait, every chunk, for the output stores
    wait_vm();
    if (nexp > 0) {  // the helpers' prologue
      lds_barrier();
      lds_barrier();
      lds_barrier();
    }
    float lam_c = 1.f;  // the lazy scale at the start of the current token chunk
    for (int e = 0; e < nexp; ++e) {
      const int ks = e % 3, ts = e & 1;
      const int c = e / n;
      const int j = e - c * n;
      const int qs = c & 1;
      // the chunk's scale scalars and flags (helper 2 wrote them a chunk ahead)
      const int fl = __builtin_amdgcn_readfirstlane(sm.sflag[ts]);
      const bool fast = !SUM && (fl & SF_FAST), lazy = fl & SF_LAZY, tfs = fl & SF_TF;
      const float dl = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, sm.scal[ts][1])));
      if (fl & SF_RESCALE) {  // rescale at the token chunk's start: Sst *= lam, lam = 1
#pragma unroll
        for (int at = 0; at < KT16; ++at)
#pragma unroll
          for (int b = 0; b < NB; ++b) Sacc[at][b] *= lam;
        lam = 1.f;
      }
      if (LT || j == 0) lam_c = lam;
      // the lane constants are made opaque every chunk so that the compiler forms
      // each address where it is used instead of hoisting dozens of them
      SwLane lcont = Lcont, lcolk = Lcolk;
      int ln = lane;
      asm volatile("" : "+v"(lcont.l), "+v"(lcont.x), "+v"(lcolk.l), "+v"(lcolk.x), "+v"(ln));
      const int lr = ln & 15, lg = ln >> 4;
      const int rt = 4 * lg + (lr >> 2);  // row of a transposing read inside its 16-row group
      const SwLane lcolv = sw_lane<VW>(rt, 8 * (lr & 3));                // v columns
      const uint32_t lt = (uint32_t)((rt * LDT + ((4 * (lr & 3)) ^ (8 * ((rt >> 3) & 1)))) * 2);  // T^T columns
      const uint32_t lp = (uint32_t)((lr * LDC + 8 * lg) * 2);        // P rows
      const uint32_t kt = off_of(sm.k[ks]), qt = off_of(sm.q[qs]);
      const float *gtok = sm.gtok[qs], *qfac = sm.qfac[qs];
      const float *rk = sm.rk[ts], *gkr = sm.gkr[ts];
      const int *tokr = sm.tokr[ts];
      // ---- phase A: X = K Sst (and at a token-chunk start O^T = Sst^T Q^T), scores, R
      if constexpr (LT) {
        // state entering token chunk c (written out here rather than through
        // store_chunk_state: the call form changes this instantiation's
        // register allocation, and it ran 3-4% slower)
        if (j == 0 && a.chunk_states) {
          const int64_t row = cs_row0 + c;
          if (row >= 0 && row < a.cs_rows) {
            uint32_t lo = (uint32_t)(8 * lg * V + gcol + lr);
            asm volatile("" : "+v"(lo));
            float *dst = a.chunk_states + ((size_t)row * a.Hv + h) * KV + lo;
#pragma unroll
            for (int at = 0; at < KT16; ++at)
#pragma unroll
              for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int i = 0; i < 4; ++i) dst[kap(at, 0, i) * V + 16 * b] = lam * Sacc[at][b][i];
          }
        }
      }
      f32x4 X[4][NB];
      // Scores, transposed, of the wave's token block tb against its row blocks:
      // lane (lg, lr) of tile pa holds Sc[r = 16 (rb0 + pa) + 4 lg + i][t = 16 tb + lr]
      // = k_r.q_t.  They reuse the k fragments of X = K Sst as the A operand.
      f32x4 Pacc[RBW];
      // at a token-chunk start with the in-kernel norm: the sum of squares of q
      // row 16 tb + lr over the 32 elements this lane reads
      float qss = 0.f;
      const bool qnorm = j == 0 && a.l2norm;
      if constexpr (LT) {
        // X = K Sst, the wave's score tiles and O^T = Sst^T Q^T of the expanded
        // chunk's two token blocks (rows 32 j + 16 a4 + lr of the q tile), all on
        // the same Sst fragments; k and q fragments of step s+1 are read while
        // step s multiplies
        Frag<bf16> kf[4], qf[2][2];
        float qs2[2] = {0.f, 0.f};
        // token block 0 meets row blocks 0-1 only: the wave holding its row
        // blocks 2-3 forms no score tiles (O += E P^T never reads them)
        const bool ptiles = !(tb == 0 && rb0 >= 2);
        auto load_kf = [&](int s, int a4) {
          const uint32_t xs = lcont.x ^ (uint32_t)(64 * s);
          kf[a4].v = rd16(xs + (kt + lcont.l) + 16 * a4 * KW);
        };
        auto load_qf = [&](int s, int buf) {
          const uint32_t xs = lcont.x ^ (uint32_t)(64 * s);
#pragma unroll
          for (int a4 = 0; a4 < 2; ++a4) qf[buf][a4].v = rd16(xs + (qt + lcont.l) + 16 * (2 * j + a4) * KW);
        };
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) load_kf(0, a4);
        load_qf(0, 0);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          if (s + 1 < KS) load_qf(s + 1, (s + 1) & 1);
          __builtin_amdgcn_sched_barrier(0);
          Frag<bf16> Sb[NB];
#pragma unroll
          for (int b = 0; b < NB; ++b) from_acc(Sb[b], Sacc[2 * s][b], Sacc[2 * s + 1][b]);
          const Frag<bf16> &qw = tb ? qf[s & 1][1] : qf[s & 1][0];
#pragma unroll
          for (int a4 = 0; a4 < 4; ++a4) {
#pragma unroll
            for (int b = 0; b < NB; ++b) X[a4][b] = mma(kf[a4], Sb[b], s == 0 ? zero4() : X[a4][b]);
            if (ptiles && a4 >= rb0 && a4 < rb0 + RBW) Pacc[a4 - rb0] = mma(kf[a4], qw, s == 0 ? zero4() : Pacc[a4 - rb0]);
            if (s + 1 < KS) load_kf(s + 1, a4);
          }
#pragma unroll
          for (int a4 = 0; a4 < 2; ++a4)
#pragma unroll
            for (int b = 0; b < NB; ++b) O[b][a4] = mma(Sb[b], qf[s & 1][a4], s == 0 ? zero4() : O[b][a4]);
          if (a.l2norm && w < 2) qs2[0] += seg_sumsq<bf16>(__builtin_bit_cast(uint4, qf[s & 1][decltype(halfc)::value].v));
          __builtin_amdgcn_sched_barrier(0);
        }
        // q-row rstd: waves 0 and 1 form it for token blocks 0 and 1 of the
        // expanded chunk and leave it in LDS for every wave's staging
        if (a.l2norm && w < 2) {
          float x = qs2[0];
          x += __shfl_xor(x, 16, 64);
          x += __shfl_xor(x, 32, 64);
          if (lg == 0) sm.rq[ts][16 * decltype(halfc)::value + lr] = frsq(x + 1e-6f);
        }
      } else
      // k (and q) fragments of reduction step s+1 are read while step s multiplies
      {
        // rolling single buffer: fragment a4 of step s+1 is read right after the
        // last product of step s that uses it
        Frag<bf16> kf[4], qw[2];
        auto load_kf = [&](int s, int a4) {  // reduction slots 32s + 8lg .. +7 of row block a4
          const uint32_t xs = lcont.x ^ (uint32_t)(64 * s);
          kf[a4].v = rd16(xs + (kt + lcont.l) + 16 * a4 * KW);
        };
        auto load_qw = [&](int s, int buf) {
          const uint32_t xs = lcont.x ^ (uint32_t)(64 * s);
          qw[buf].v = rd16(xs + (qt + lcont.l) + 16 * tb * KW);
        };
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) load_kf(0, a4);
        if constexpr (!SUM) load_qw(0, 0);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          if constexpr (!SUM) {
            if (s + 1 < KS) load_qw(s + 1, (s + 1) & 1);
          }
          __builtin_amdgcn_sched_barrier(0);
          Frag<bf16> Sb[NB];
#pragma unroll
          for (int b = 0; b < NB; ++b) from_acc(Sb[b], Sacc[2 * s][b], Sacc[2 * s + 1][b]);
#pragma unroll
          for (int a4 = 0; a4 < 4; ++a4) {
#pragma unroll
            for (int b = 0; b < NB; ++b) X[a4][b] = mma(kf[a4], Sb[b], s == 0 ? zero4() : X[a4][b]);
            if constexpr (!SUM) {
              if (a4 >= rb0 && a4 < rb0 + RBW)
                Pacc[a4 - rb0] = mma(kf[a4], qw[s & 1], s == 0 ? zero4() : Pacc[a4 - rb0]);
            }
            if (s + 1 < KS) load_kf(s + 1, a4);
          }
          if constexpr (!SUM) {
            if (qnorm) qss += seg_sumsq<bf16>(__builtin_bit_cast(uint4, qw[s & 1].v));
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // q-row rstd of the wave's 16 tokens (the four lanes lg of a row hold a
      // quarter each); the outputs of token chunk c take it when staged
      if (!SUM && !LT && qnorm) {
        qss += __shfl_xor(qss, 16, 64);
        qss += __shfl_xor(qss, 32, 64);
        if (lg == 0) sm.rq[qs][16 * tb + lr] = frsq(qss + 1e-6f);
      }
      if (!SUM && !LT && j == 0) {  // a token chunk starts: O^T = Sst^T Q^T
        Frag<bf16> qf[2][4];
        auto load_q = [&](int s, int buf) {
          const uint32_t xs = lcont.x ^ (uint32_t)(64 * s);
#pragma unroll
          for (int a4 = 0; a4 < 4; ++a4) qf[buf][a4].v = rd16(xs + (qt + lcont.l) + 16 * a4 * KW);
        };
        load_q(0, 0);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          if (s + 1 < KS) load_q(s + 1, (s + 1) & 1);
          __builtin_amdgcn_sched_barrier(0);
          Frag<bf16> Sb[NB];
#pragma unroll
          for (int b = 0; b < NB; ++b) from_acc(Sb[b], Sacc[2 * s][b], Sacc[2 * s + 1][b]);
#pragma unroll
          for (int a4 = 0; a4 < 4; ++a4)
#pragma unroll
            for (int b = 0; b < NB; ++b) O[b][a4] = mma(Sb[b], qf[s & 1][a4], s == 0 ? zero4() : O[b][a4]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (!SUM && !LT && j == 0 && !fast) {  // O^T columns t times lam scale 2^Gt_t (the q-row rstd comes at staging)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const float f = lam * qfac[16 * a4 + lr];
#pragma unroll
          for (int b = 0; b < NB; ++b) O[b][a4] *= f;
        }
      }
      if (LT && !fast) {  // O^T columns t times lam scale 2^G(t), G(t) the expanded cumsum at t's rows
#pragma unroll
        for (int a4 = 0; a4 < 2; ++a4) {
          const float f = lam * a.scale * fexp2(sm.gdp[ks][2 * (16 * a4 + lr)]);
#pragma unroll
          for (int b = 0; b < NB; ++b) O[b][a4] *= f;
        }
      }
      // P[t][r] = scale rk_r 2^(Gt_t - Gt_tok(r)) q_t.k_r for tok(r) <= t, i.e. for
      // r below n (t + 1) - 64 j; written to the P tile as rows t of contiguous r.
      // When the token chunk's decay cumsum stays above -100 the decay factor is
      // the product qfac_t rkg_r of per-token and per-row factors (both finite and
      // normal); otherwise it is formed per entry.
      if (!SUM && !(LT && tb == 0 && rb0 >= 2)) {
        const int t = 16 * tb + lr;  // (with LT: the token inside the expanded chunk)
        const int rlim = LT ? 2 * (t + 1) : n * (t + 1) - CH * j;
        const bool fact = !LT && sm.qsafe[qs] != 0;
        const uint32_t pw = off_of(sm.p) + lp + (uint32_t)(32 * tb * LDC);
        if (fast) {  // raw masked scores: the factors sit in E_w and at staging
#pragma unroll
          for (int pa = 0; pa < RBW; ++pa) {
            const int a4 = rb0 + pa, r0 = 16 * a4 + 4 * lg;
            f32x4 val;
#pragma unroll
            for (int i = 0; i < 4; ++i) val[i] = r0 + i < rlim ? Pacc[pa][i] : 0.f;
            *(bf16x4 *)((char *)&sm + pw + 64 * (a4 >> 1) + 8 * (a4 & 1)) = bf4(val);
          }
        } else if (LT) {  // per entry: scale rk_r 2^(G(t) - G_r), both on the expanded cumsum
          const float *gd = sm.gdp[ks];
          const float gt = gd[2 * t], rq = a.scale;
#pragma unroll
          for (int pa = 0; pa < RBW; ++pa) {
            const int a4 = rb0 + pa, r0 = 16 * a4 + 4 * lg;
            const f32x4 rk4 = ld4(rk + r0), gk4 = ld4(gd + r0);
            f32x4 val;
#pragma unroll
            for (int i = 0; i < 4; ++i) val[i] = r0 + i < rlim ? rq * rk4[i] * fexp2(gt - gk4[i]) * Pacc[pa][i] : 0.f;
            *(bf16x4 *)((char *)&sm + pw + 64 * (a4 >> 1) + 8 * (a4 & 1)) = bf4(val);
          }
        } else if (fact) {
          const float qv = qfac[t];
          const float *rkg = sm.rkg[ts];
#pragma unroll
          for (int pa = 0; pa < RBW; ++pa) {
            const int a4 = rb0 + pa, r0 = 16 * a4 + 4 * lg;
            const f32x4 f4 = ld4(rkg + r0) * qv;
            f32x4 val;
#pragma unroll
            for (int i = 0; i < 4; ++i) val[i] = r0 + i < rlim ? f4[i] * Pacc[pa][i] : 0.f;
            *(bf16x4 *)((char *)&sm + pw + 64 * (a4 >> 1) + 8 * (a4 & 1)) = bf4(val);
          }
        } else {
          const float gt = gtok[t], rq = a.scale;
#pragma unroll
          for (int pa = 0; pa < RBW; ++pa) {
            const int a4 = rb0 + pa, r0 = 16 * a4 + 4 * lg;
            const f32x4 rk4 = ld4(rk + r0), gk4 = ld4(gkr + r0);
            f32x4 val;
#pragma unroll
            for (int i = 0; i < 4; ++i) val[i] = r0 + i < rlim ? rq * rk4[i] * fexp2(gt - gk4[i]) * Pacc[pa][i] : 0.f;
            *(bf16x4 *)((char *)&sm + pw + 64 * (a4 >> 1) + 8 * (a4 & 1)) = bf4(val);
          }
        }
      }
      // R = diag(beta) (V + Y) with Y = -lam diag(2^G rk) X; the beta sits in the
      // WY matrix (T diag(beta)), so V + Y is formed here in fp32 and rounded to
      // bf16 once (the residual of the delta rule, often much smaller than V or
      // Y), which halves the E product after the barrier.  The chunk's v rows
      // landed before the last barrier.  V + Y is read in the slot order of
      // two stacked accumulator tiles (the B operand's "perm" order).
      Frag<bf16> Yb[2][NB];
      {
        Frag<bf16> vfr[2][NB];
        if constexpr (!MP) {
          const uint32_t vb = off_of(sm.v[ts]) + lcolv.l;
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            const uint32_t va = (lcolv.x ^ (uint32_t)(2 * wcol + 32 * b)) + vb;
#pragma unroll
            for (int s = 0; s < 2; ++s)
              vfr[s][b].v = __builtin_shufflevector(tr8(va + 32 * s * VW), tr8(va + (32 * s + 16) * VW), 0, 1, 2, 3, 4, 5, 6, 7);
          }
        }
        const float *cf = sm.c1[ts];
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const f32x4 coef = ld4(cf + 16 * a4 + 4 * lg) * (-lam);
#pragma unroll
          for (int b = 0; b < NB; ++b) X[a4][b] *= coef;
        }
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            if constexpr (MP) {  // zero values
              from_acc(Yb[s][b], X[2 * s][b], X[2 * s + 1][b]);
            } else {
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                Yb[s][b].v[i] = (bf16)(X[2 * s][b][i] + (float)vfr[s][b].v[i]);
                Yb[s][b].v[4 + i] = (bf16)(X[2 * s + 1][b][i] + (float)vfr[s][b].v[4 + i]);
              }
            }
          }
      }
      lds_barrier();  // P complete
      // ---- phase B: E = T R, O^T += E^T P^T, state update, outputs
      // fragments of T diag(beta) (A operand, from its transpose through the
      // transposing read)
      Frag<bf16> tfr[6];
      {
        const uint32_t tb = off_of(sm.t) + lt;
#pragma unroll
        for (int fi = 0; fi < 6; ++fi) {
          const int a4 = fi < 2 ? fi : (fi < 4 ? 2 : 3), s = (fi == 3 || fi == 5) ? 1 : 0;
          tfr[fi].v = __builtin_shufflevector(tr8(tb + (32 * s * LDT + 16 * a4) * 2), tr8(tb + ((32 * s + 16) * LDT + 16 * a4) * 2),
                                              0, 1, 2, 3, 4, 5, 6, 7);
        }
      }
      // the P fragments of the first token block and the k^T fragments of the
      // first state row block
      // first token of each 32-row half (with LT the rows 32 s.. hold tokens 16 s..)
      const int tokb0 = (SUM || LT) ? 0 : tokr[0], tokb1 = SUM ? 0 : (LT ? 16 : tokr[32]);
      Frag<bf16> pf[2][2];
      const uint32_t pr = off_of(sm.p) + lp;
      auto load_pf = [&](int a4, int buf) {  // P rows of token block a4
#pragma unroll
        for (int s = 0; s < 2; ++s)
          pf[buf][s].v = rd16(pr + (16 * a4 * LDC + 32 * s) * 2);
      };
      const uint32_t kcb = kt + lcolk.l;
      Frag<bf16> kc[2][2];
      auto load_kc = [&](int at, int buf) {  // lane lr of tile at: key kap(at, lr / 4, lr % 4)
        const uint32_t x = (lcolk.x ^ (uint32_t)(64 * (at >> 1))) + kcb + 8 * (at & 1);
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
          kc[buf][h2].v = __builtin_shufflevector(tr8(x + 32 * h2 * KW), tr8(x + (32 * h2 + 16) * KW), 0, 1, 2, 3, 4, 5, 6, 7);
      };
      __builtin_amdgcn_sched_barrier(0);
      f32x4 E[4][NB];
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4)
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          f32x4 acc = mma(tfr[a4 < 2 ? a4 : 2 * a4 - 2], Yb[0][b], zero4());
          if (a4 >= 2) acc = mma(tfr[2 * a4 - 1], Yb[1][b], acc);
          E[a4][b] = acc;
        }
      // (read while E forms)
      if constexpr (!SUM) load_pf(0, 0);
      load_kc(0, 0);
      __builtin_amdgcn_sched_barrier(0);
      // E: the v_new rows, or (chunks whose WY matrix carries the state-update
      // weights, SF_TF) E_w = diag(f) E, which both products below then use
      Frag<bf16> Eb[2][NB];
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int b = 0; b < NB; ++b) from_acc(Eb[s][b], E[2 * s][b], E[2 * s + 1][b]);
      if constexpr (!SUM) {
#pragma unroll
      for (int a4 = 0; a4 < OTB; ++a4) {
        if (a4 + 1 < OTB) load_pf(a4 + 1, (a4 + 1) & 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          if ((s ? tokb1 : tokb0) > 16 * a4 + 15) continue;  // P block entirely masked
#pragma unroll
          for (int b = 0; b < NB; ++b) O[b][a4] = mma(Eb[s][b], pf[a4 & 1][s], O[b][a4]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      }
      // Sst += K^T diag(f) E with f = 2^(G_last - G) rk / (lam 2^G_last) and lam *= 2^G_last,
      // unless lam would fall below LAM_MIN (then f = 2^(G_last - G) rk and Sst is
      // rescaled to lam = 1); dl = lam 2^G_last and f come from the helpers' tables
      if (!tfs) {
        const float rl = sm.scal[ts][2];
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const f32x4 f = ld4(sm.wgt[ts] + 16 * a4 + 4 * lg) * rl;
#pragma unroll
          for (int b = 0; b < NB; ++b) E[a4][b] *= f;
        }
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int b = 0; b < NB; ++b) from_acc(Eb[s][b], E[2 * s][b], E[2 * s + 1][b]);
      }
      if (!lazy) {
#pragma unroll
        for (int at = 0; at < KT16; ++at)
#pragma unroll
          for (int b = 0; b < NB; ++b) Sacc[at][b] *= dl;
      }
      // row factors of the outputs (staged after the state update, read here so
      // that their LDS reads overlap it): the q-row rstd rq_t and, on a fast token
      // chunk, lam_c scale 2^Gt_t (lam_c 2^Gt_t stays above LAM_MIN there, so the
      // product is a normal float)
      // (with LT every expanded chunk stages its own 32 tokens: rq_t and, on a fast
      // chunk, lam scale 2^G(t), which stays above LAM_MIN)
      const bool stage = !SUM && (LT || j == n - 1 || e == nexp - 1) && a.o;
      float sfac[OTB];
      if (stage) {
        if constexpr (LT) {
#pragma unroll
          for (int a4 = 0; a4 < OTB; ++a4)
            sfac[a4] = (fast ? lam_c * a.scale * fexp2(sm.gdp[ks][2 * (16 * a4 + lr)]) : 1.f) * (a.l2norm ? sm.rq[ts][16 * a4 + lr] : 1.f);
        } else {
#pragma unroll
          for (int a4 = 0; a4 < 4; ++a4) {
            const float qf = sm.qfac[qs][16 * a4 + lr], rq = sm.rq[qs][16 * a4 + lr];
            sfac[a4] = (fast ? lam_c * qf : 1.f) * (a.l2norm ? rq : 1.f);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int at = 0; at < KT16; ++at) {  // k^T fragments one step ahead
        if (at + 1 < KT16) load_kc(at + 1, (at + 1) & 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          Sacc[at][b] = mma(kc[at & 1][0], Eb[0][b], Sacc[at][b]);
          Sacc[at][b] = mma(kc[at & 1][1], Eb[1][b], Sacc[at][b]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      lam = lazy ? dl : 1.f;
      // outputs of token chunk c once its last expanded chunk is in: lane holds
      // O[t = 16 a4 + lr][16 b + 4 lg .. +3] of this wave's columns.  The q-row rstd
      // rq_t (and on a fast token chunk lam_c scale 2^Gt_t) multiplies every term of
      // row t and is applied here; the four bf16 values go straight to o (each
      // store instruction writes 32 contiguous bytes of 16 rows, and the four
      // consumer waves together cover whole rows).
      if (stage) {
        const int ntok = toks_of(c);
        const int row0 = LT ? 32 * j : 0;  // first staged row inside the token chunk
        const bool full = row0 + 16 * OTB <= ntok;
        char *ob = (char *)((bf16 *)a.o + (t0 + (int64_t)CH * c) * a.o_st + h * a.o_sh + gcol);
        const uint32_t ost = (uint32_t)a.o_st * 2u;
        // every row is packed and addressed first and the stores follow back to
        // back: a store reads its data and address registers only when the memory
        // pipeline takes it, and rewriting them before that stalls the wave.
        // With 16-byte aligned rows, lanes 16 apart swap halves (row swap), so
        // that each lane holds 8 consecutive columns and 4 lanes cover the wave's
        // 64 bytes of a row; otherwise each lane stores its two 8-byte pieces.
        const bool o16 = (((uintptr_t)a.o & 15) == 0) && (a.o_st % 8 == 0) && (a.o_sh % 8 == 0);
        if constexpr (NB == 2) if (o16) {
          uint4 pk[OTB];
          uint4 *dst[OTB];
#pragma unroll
          for (int a4 = 0; a4 < OTB; ++a4) {
            const uint2 p0 = __builtin_bit_cast(uint2, bf4(O[0][a4] * sfac[a4]));
            const uint2 p1 = __builtin_bit_cast(uint2, bf4(O[1][a4] * sfac[a4]));
            const auto rx = __builtin_amdgcn_permlane16_swap(p0.x, p1.x, false, false);
            const auto ry = __builtin_amdgcn_permlane16_swap(p0.y, p1.y, false, false);
            pk[a4] = uint4{(uint32_t)rx[0], (uint32_t)ry[0], (uint32_t)rx[1], (uint32_t)ry[1]};
            dst[a4] = (uint4 *)(ob + (uint32_t)(row0 + 16 * a4 + lr) * ost + 16 * (lg >> 1) + 32 * (lg & 1));
          }
          __builtin_amdgcn_sched_barrier(0);
          if (full) {
#pragma unroll
            for (int a4 = 0; a4 < OTB; ++a4) *dst[a4] = pk[a4];
          } else {
#pragma unroll
            for (int a4 = 0; a4 < OTB; ++a4)
              if (row0 + 16 * a4 + lr < ntok) *dst[a4] = pk[a4];
          }
        }
        if (NB != 2 || !o16) {
          uint2 pk[OTB][NB];
          uint2 *dst[OTB];
#pragma unroll
          for (int a4 = 0; a4 < OTB; ++a4) {
#pragma unroll
            for (int b = 0; b < NB; ++b) pk[a4][b] = __builtin_bit_cast(uint2, bf4(O[b][a4] * sfac[a4]));
            dst[a4] = (uint2 *)(ob + (uint32_t)(row0 + 16 * a4 + lr) * ost + 8 * lg);
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int a4 = 0; a4 < OTB; ++a4)
            if (full || row0 + 16 * a4 + lr < ntok) {
#pragma unroll
              for (int b = 0; b < NB; ++b) dst[a4][4 * b] = pk[a4][b];
            }
        }
      }
      if constexpr (!LT) {
        if (a.chunk_states && j == n - 1 && c + 1 < ntc) store_chunk_state(c + 1);
      }
      lds_barrier();
    }
    float *fdst = MP ? a.msum + state_off : (a.final_state ? a.final_state + state_off : nullptr);
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
          const int k = kap(at, lg, i), col = gcol + 16 * b + lr;
          const float x = lam * Sacc[at][b][i];
          if constexpr (MP) {  // M as a bfloat16 hi/lo pair (msum_index)
            bf16 *mb = (bf16 *)fdst;
            const bf16 hi = (bf16)x;
            mb[msum_index<K>(k, col, 0)] = hi;
            mb[msum_index<K>(k, col, 1)] = (bf16)(x - (float)hi);
          } else {
            const size_t off = (size_t)k * V + col;
            if (fdst) fdst[off] = x;
            if (cdst) cdst[off] = x;
          }
        }
  };
  if (w < NCW) {
    if ((LT && (w & 1)) || (NCW > 4 && w >= 4)) consumer(IC<1>{});
    else consumer(IC<0>{});
  } else {
    // ---------------------------------------------------------------- helpers
    // Four helper waves share the loads and the WY step.  For chunk x the WY
    // step runs as a three-stage pipeline:
    //   Gram stage   (iteration x-1, before the mid-chunk barrier): helpers 1-3
    //                form the 10 Gram tiles (row blocks 0-1, 2, 3) and the k-row
    //                rstd from the diagonal tiles;
    //   block stage  (iteration x-1, after it): helper h builds row block h of
    //                A and inverts its diagonal block by DPP row substitution;
    //   merge stage  (iteration x, before the mid-chunk barrier): helper 0 forms
    //                the blocks of T below the diagonal and writes T^T, which the
    //                consumers read after that barrier.
    // The loads are spread over the four helpers as well.
    const int hw = w - NCW;
    // In summary mode each SIMD runs two consumer waves and one helper, and the
    // WY helpers are the critical path (their Gram, block and merge stages take
    // longer than the consumers' phases): they issue first
    if constexpr (SUM) {
      if (hw != 0) __builtin_amdgcn_s_setprio(1);
    }
    const bf16 *qg = (const bf16 *)a.q + hq * a.q_sh;
    const bf16 *kg = (const bf16 *)a.k + hk * a.k_sh;
    const bf16 *vg = (const bf16 *)a.v + h * a.v_sh + vt * BV;
    const float *gg = a.g + h * a.g_sh;
    const float *bg = a.beta + h * a.b_sh;
    const uint32_t kst = (uint32_t)a.k_st * 2u, vst = (uint32_t)a.v_st * 2u, qst = (uint32_t)a.q_st * 2u;
    // lane index of the loader's address and table arithmetic; the loader loop
    // makes it opaque every chunk so that nothing derived from it is hoisted
    // out of the loop and held in registers (a spilled value reloaded between
    // direct-to-LDS loads would wait for them)
    int hl = lane;
    auto load_k = [&](int e, const TileOffs<KW, 1> &offs) {
      const char *g = (const char *)(kg + (t0 * n + (int64_t)CH * e) * a.k_st);
      if (rows_of(e) == CH) tile_load_full<KW, 1>(sm.k[e % 3], g, offs);
      else tile_load<KW, 1>(sm.k[e % 3], g, kst, rows_of(e), hl);
    };
    auto load_v = [&](int e, const TileOffs<VW> &offs) {
      const char *g = (const char *)(vg + (t0 * n + (int64_t)CH * e) * a.v_st);
      if (rows_of(e) == CH) tile_load_full<VW>(sm.v[e & 1], g, offs);
      else tile_load<VW>(sm.v[e & 1], g, vst, rows_of(e), hl);
    };
    auto load_scalars = [&](int e) {  // raw beta and decay of each sub-row of chunk e
      const int64_t s0 = (int64_t)CH * e;
      const int r = min(hl, rows_of(e) - 1);
      // token of sub-row s0 + r: the 64-bit quotient of the chunk start once per
      // wave, then a 32-bit one for the lane
      const int64_t q0 = s0 / n;
      const int r0 = (int)(s0 - q0 * n);
      const int64_t tok = q0 + (int64_t)((uint32_t)(r0 + r) / (uint32_t)n);
      scalar_load(sm.rawb[e & 1], bg + (t0 * n + s0 + r) * a.b_st);
      scalar_load(sm.rawg[e & 1], gg + (t0 + tok) * a.g_st);
    };
    auto prep_scalars = [&](int e) {  // masked betas and the base-2 decay cumsum of chunk e
      const bool valid = hl < rows_of(e);
      const int rem = (int)(((int64_t)CH * e) % n);
      const bool first = valid && (rem + hl) % n == 0;  // the decay sits on a token's first sub-row
      sm.gdp[e % 3][hl] = wave_scan(first ? sm.rawg[e & 1][hl] * LOG2E : 0.f);
      sm.beta[e % 3][hl] = valid ? sm.rawb[e & 1][hl] : 0.f;
    };
    auto load_q = [&](int c, const TileOffs<KW, 1> &offs) {  // q rows and token decays of token chunk c
      const int64_t tokbase = t0 + (int64_t)CH * c;
      const char *g = (const char *)(qg + tokbase * a.q_st);
      if (toks_of(c) == CH) tile_load_full<KW, 1>(sm.q[c & 1], g, offs);
      else tile_load<KW, 1>(sm.q[c & 1], g, qst, toks_of(c), hl);
      // with n = 1 the token decays are the sub-row decays of the scalar ring
      if (n != 1) scalar_load(sm.rawt[c & 1], gg + (tokbase + min(hl, toks_of(c) - 1)) * a.g_st);
    };
    auto tables = [&](int e) {  // token of each row of chunk e inside its token chunk, and its decay cumsum
      const int c = e / n, j = e - c * n;
      const int tk = (CH * j + hl) / n;
      const float gk = sm.gtok[c & 1][tk];
      sm.tokr[e & 1][hl] = tk;
      sm.gkr[e & 1][hl] = gk;
      sm.rkg[e & 1][hl] = sm.rk[e & 1][hl] * fexp2(-gk);  // overflow-free when qsafe
    };
    auto finish_q = [&](int c) {  // after load_q(c) has landed: token decay cumsum of token chunk c
      const int sl = c & 1, ntok = toks_of(c);
      // n = 1: token chunk c is chunk c, whose raw decays are in the scalar ring
      const float raw = n == 1 ? sm.rawg[sl][hl] : sm.rawt[sl][hl];
      const float gt = wave_scan(hl < ntok ? raw * LOG2E : 0.f);
      sm.gtok[sl][hl] = gt;
      sm.qfac[sl][hl] = a.scale * fexp2(gt);
      // the cumsum is non-increasing, so its last valid entry is its minimum
      const float gmin = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, gt), ntok - 1));
      if (hl == 0) sm.qsafe[sl] = gmin > -100.f;
    };
    // Scale scalars of chunk x (after its decay cumsum and, at a token chunk's
    // start, its token decay cumsum are in), in the order the consumers apply
    // them: lam is the lazy state scale (S = lam Sst) entering the chunk.  At a
    // token chunk's start, when lam 2^Gt_end would fall below LAM_MIN inside it,
    // the state is first rescaled to lam = 1; the token chunk is fast when lam
    // 2^Gt_end then stays at or above LAM_MIN (so no rescale happens inside it).
    // dl = lam 2^G_last; the chunk is lazy when dl >= LAM_MIN (always inside a fast
    // token chunk), and the state update's weights then carry rl = 1 / dl.
    // Summary mode has no outputs: every chunk uses the weighted WY matrix.
    auto scalars = [&](int x, float &lam_h, bool &fast_h) {
      const int cx = x / n, jx = x - cx * n;
      int fl = 0;
      if constexpr (LT) {  // per expanded chunk: its own decay decides
        const float gl = sm.gdp[x % 3][CH - 1];
        if (lam_h * fexp2(gl) < LAM_MIN && lam_h != 1.f) {
          fl |= SF_RESCALE;
          lam_h = 1.f;
        }
        fast_h = lam_h * fexp2(gl) >= LAM_MIN;
      } else if (jx == 0) {
        if constexpr (SUM) {
          fast_h = false;
        } else {
          const float gend = sm.gtok[cx & 1][CH - 1];
          if (lam_h * fexp2(gend) < LAM_MIN && lam_h != 1.f) {
            fl |= SF_RESCALE;
            lam_h = 1.f;
          }
          fast_h = lam_h * fexp2(gend) >= LAM_MIN;
        }
      }
      const float dl = lam_h * fexp2(sm.gdp[x % 3][CH - 1]);
      const bool lazy = fast_h || dl >= LAM_MIN;
      fl |= (fast_h ? SF_FAST | SF_TF : 0) | (SUM ? SF_TF : 0) | (lazy ? SF_LAZY : 0);
      if (hl == 0) {
        *(f32x4 *)sm.scal[x & 1] = f32x4{lam_h, dl, lazy ? 1.f / dl : 1.f, 0.f};
        sm.sflag[x & 1] = fl;
      }
      lam_h = lazy ? dl : 1.f;
    };
    // Gram stage of chunk x: tiles [i0, i1) of the lower triangle, with the k rows
    // of the later block as the B operand so that lane (lg, lr) of tile (ra, rb)
    // holds G[16 ra + lr][16 rb + 4 lg + i]; rstd of the rows of its diagonal tiles
    auto gram = [&](int x, int i0, int i1, int nblk) {
      const char *k = sm.k[x % 3];
      float *rk = sm.rk[x & 1];
      const int nrow = rows_of(x);
      Frag<bf16> kf[4][KS];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
        if (rt < nblk) {
#pragma unroll
          for (int s = 0; s < KS; ++s) kf[rt][s] = sw_contig<KW, 1>(k, 16 * rt + lr, 32 * s, lg);
        }
#pragma unroll
      for (int idx = 0; idx < 10; ++idx) {
        if (idx < i0 || idx >= i1) continue;
        int ra, rb;
        lower_tile(idx, ra, rb);
        f32x4 acc = zero4();
#pragma unroll
        for (int s = 0; s < KS; ++s) acc = mma(kf[rb][s], kf[ra][s], acc);
        *(f32x4 *)(sm.gram[idx] + 4 * lane) = acc;
        if (ra == rb) {  // lane with 4 lg + i == lr holds the squared norm of row 16 ra + lr
          const int i = lr & 3;
          const float dv = i == 0 ? acc[0] : (i == 1 ? acc[1] : (i == 2 ? acc[2] : acc[3]));
          if ((lr >> 2) == lg) rk[16 * ra + lr] = (16 * ra + lr < nrow) ? (a.l2norm ? frsq(dv + 1e-6f) : 1.f) : 0.f;
        }
      }
    };
    // block stage of chunk x, row block hb: A[r][c] = beta_r rk_r rk_c 2^(G_r - G_c) G[r][c]
    // for c < r, the inverse of the diagonal block, and the consumers' row weights
    auto block = [&](int x, auto hbc) {
      constexpr int hb = decltype(hbc)::value;
      const float *bt = sm.beta[x % 3], *gd = sm.gdp[x % 3], *rk = sm.rk[x & 1];
      const int r = 16 * hb + lr;
      const float fr = bt[r] * rk[r], gr = gd[r];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        if (b > hb) continue;
        const int idx = hb * (hb + 1) / 2 + b, c0 = 16 * b + 4 * lg;
        const f32x4 g = *(const f32x4 *)(sm.gram[idx] + 4 * lane);
        const f32x4 rc = ld4(rk + c0), gc = ld4(gd + c0);
        f32x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = fr * rc[i] * fexp2(gr - gc[i]) * g[i];
        if (b < hb) {
          *(bf16x4 *)(sm.alow[idx - hb] + lr * 16 + 4 * lg) = bf4(v);  // idx - hb enumerates (1,0) (2,0) (2,1) (3,0) (3,1) (3,2)
        } else {  // rows of -L of the diagonal block over the Gram tile just read: the
                  // 16-byte piece q of row lr at lr * 64 + 16 (q ^ (lr / 4 mod 4)), so that
                  // 16 lanes writing one piece of 16 rows meet distinct banks
          float *dg = sm.gram[idx];
          const int sx = (lr >> 2) & 3;
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = (c0 + i < r) ? -v[i] : 0.f;
          *(f32x4 *)(dg + lr * 16 + 4 * (lg ^ sx)) = v;
          float nl[16];
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const f32x4 u = ld4(dg + lr * 16 + 4 * (q4 ^ sx));
#pragma unroll
            for (int i = 0; i < 4; ++i) nl[4 * q4 + i] = u[i];
          }
          float tdg[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) tdg[i] = (lr == 4 * lg + i) ? 1.f : 0.f;
          subst<0>(tdg, nl);
          const bf16x4 tb = bf16x4{(bf16)tdg[0], (bf16)tdg[1], (bf16)tdg[2], (bf16)tdg[3]};
          *(bf16x4 *)(sm.tdiag[hb] + 4 * lane) = tb;
          *(bf16x4 *)(sm.tdrow[hb] + lr * 16 + 4 * lg) = tb;
        }
      }
      if (lg == 0) {  // per-row weights of the consumers' R (2^G rk) and state update (2^(G_last - G) rk)
        const float glast = gd[CH - 1];
        sm.c1[x & 1][r] = fexp2(gr) * rk[r];
        sm.wgt[x & 1][r] = fexp2(glast - gr) * rk[r];
      }
    };
    // merge stage of chunk x: the blocks of T below the diagonal, and (T diag(beta))^T
    // into the consumers' buffer (entry (r, c) of T diag(beta) at [c * LDT + r]).
    // With D = diag(T_aa) and A_off the blocks of A below the diagonal,
    // I + A = D^-1 (I + N) with N = D A_off, so T_ab = -sum_{c=b}^{a-1} N_ac T_cb:
    // the six N_ab are independent products, and the substitution that follows
    // is three products deep (T_10, then T_20, then T_30) instead of six.
    auto merge = [&](int x) {
      bf16 *tt = sm.t;
      const int tsw = 8 * ((lr >> 3) & 1);  // the T^T swizzle of this lane's rows
      // every input is read first, so that the merge waits for one LDS round trip
      bf16x4 tc[4], td[4], ab[6];
      float bcol[4];  // beta of the column this lane writes in each column block
      f32x4 w4[4];    // state-update weights of rows 16 ra + 4 lg + i
#pragma unroll
      for (int b = 0; b < 4; ++b) bcol[b] = sm.beta[x % 3][16 * b + lr];
#pragma unroll
      for (int ra = 0; ra < 4; ++ra) w4[ra] = ld4(sm.wgt[x & 1] + 16 * ra + 4 * lg);
      const float rl = sm.scal[x & 1][2];
      const int fl = sm.sflag[x & 1];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        tc[b] = tr_col4(sm.tdrow[b], 16, 4 * lg, 0, lr);      // T_b[4lg + i][lr] (B operand)
        td[b] = *(const bf16x4 *)(sm.tdiag[b] + 4 * lane);    // T_b[lr][4lg + i]
      }
#pragma unroll
      for (int i = 0; i < 6; ++i) ab[i] = tr_col4(sm.alow[i], 16, 4 * lg, 0, lr);  // A_blk[4lg + i][lr]
      // on SF_TF chunks the rows are scaled by the state-update weights f = w rl,
      // which makes the consumers' product E_w = diag(f) E directly
      const bool tf = __builtin_amdgcn_readfirstlane(fl) & SF_TF;
      const float fm = tf ? rl : 0.f, fa = tf ? 0.f : 1.f;
      f32x4 frow[4];
#pragma unroll
      for (int ra = 0; ra < 4; ++ra) frow[ra] = w4[ra] * fm + fa;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const f32x4 d = f32x4{(float)tc[b][0], (float)tc[b][1], (float)tc[b][2], (float)tc[b][3]} * (frow[b] * bcol[b]);
        *(bf16x4 *)(tt + (16 * b + lr) * LDT + 16 * b + ((4 * lg) ^ tsw)) = bf4(d);
      }
      auto put = [&](int ra, int rb, f32x4 v) {  // v: T[16 ra + 4 lg + i][16 rb + lr]; writes it times f_row beta_col
        *(bf16x4 *)(tt + (16 * rb + lr) * LDT + 16 * ra + ((4 * lg) ^ tsw)) = bf4(v * (frow[ra] * bcol[rb]));
        return bf4(v);
      };
      // -N_ab = -T_aa A_ab as an A operand: the product A_ab^T T_aa^T leaves
      // lane (lg, lr) with N_ab[lr][4lg + i]
      auto negn = [&](int i, int a_) { return bf4(-mma16(ab[i], td[a_], zero4())); };
      const bf16x4 n10 = negn(0, 1), n20 = negn(1, 2), n21 = negn(2, 2), n30 = negn(3, 3), n31 = negn(4, 3),
                   n32 = negn(5, 3);
      // distance 1
      const bf16x4 t10 = put(1, 0, mma16(n10, tc[0], zero4()));
      const bf16x4 t21 = put(2, 1, mma16(n21, tc[1], zero4()));
      put(3, 2, mma16(n32, tc[2], zero4()));
      // distance 2
      const bf16x4 t20 = put(2, 0, mma16(n21, t10, mma16(n20, tc[0], zero4())));
      put(3, 1, mma16(n32, t21, mma16(n31, tc[1], zero4())));
      // distance 3
      put(3, 0, mma16(n32, t20, mma16(n31, t10, mma16(n30, tc[0], zero4()))));
    };
    if (hw == 0) {
      // the two T^T blocks above the diagonal that the consumers' fragments cover
      // ((0,1) and (2,3) of T) stay zero; nothing else writes them (the T^T
      // swizzle keeps every 16-column group of a row in place)
      for (int u = lane; u < 2 * 16 * 2; u += 64) {
        const int blk = u >> 5, row = (u >> 1) & 15, half = u & 1;
        *(uint4 *)(sm.t + (16 + 32 * blk + row) * LDT + 32 * blk + 8 * half) = uint4{0u, 0u, 0u, 0u};
      }
    }
    // Work per helper and chunk e = (token chunk c, sub-chunk j) (WY stages for
    // chunk e+1), before || after the mid-chunk barrier:
    //   helper 0: k rows and betas/decays of chunk e+2,  || q rows of token chunk c+2
    //             v rows of chunk e+1 (per-expanded-        (per-expanded-chunk outputs:
    //             chunk outputs: and at j = 0 the q rows    the scale scalars and row
    //             of token chunk c+1)                       block 0 of chunk e+1, and no
    //                                                       loads)
    //   helper 1: merge stage                            || row block 3 of chunk e+1
    //                                                       (and otherwise the scale
    //                                                       scalars)
    //   helper 2: Gram tiles 0-4, masked betas and decay || row block 1 (and otherwise
    //             cumsum of chunk e+1, and at j = n-1 the     row block 0)
    //             q norms and token decay cumsum of token
    //             chunk c+1
    //   helper 3: Gram tiles 5-9                         || row block 2, row tables
    //                                                       of chunk e+1
    // Each row block inverts its diagonal block by a dependent chain of DPP
    // steps, which makes two of them on one wave the longest helper phase.
    // Helper 0 issues every direct-to-LDS load; the compiler makes any LDS
    // access that follows such a load in the same wave wait for it, so its
    // own LDS work comes after the barrier that follows its phase-A loads.
    // For n >= 2 it issues no load after the mid-chunk barrier (the consumers'
    // output stores would queue behind them in the vector memory path); for
    // n = 1 the q rows of token chunk c+2 follow that barrier, because the token
    // decay cumsum of token chunk c+1 is formed in the next chunk's phase A.
    // Each helper runs its own loop (the same barrier sequence as the consumers:
    // three in the prologue, two per chunk) so that its registers are its own.
    if (hw == 0) {
      // Pacing inside the group of state heads sharing q/k head hq (the group
      // shares one sequence, hence one chunk count).  Every PACE_EVERY chunks,
      // at the end of a chunk whose loads have all completed (the loader waits
      // there for the consumers anyway), a chain publishes its chunk index and
      // polls the others' counters until none is more than PACE_AHEAD chunks
      // behind, at most PACE_SPIN times, so that no chain ever waits for good.
      // The counters start at INT32_MAX (set before the launch): a chain that
      // has not started yet is never waited for.
      const int grp = a.Hv / a.Hqk, gi = h - hq * grp;
      int32_t *prog = (a.progress && grp > 1 && !a.summary) ? a.progress + (size_t)seq * a.Hv + (size_t)hq * grp : nullptr;
      auto pace = [&](int e) {
        if (lane == 0) __hip_atomic_store(prog + gi, e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        for (int i = 0; i < grp; ++i) {
          if (i == gi) continue;
          for (int it = 0; it < PACE_SPIN; ++it) {
            if (__hip_atomic_load(prog + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= e - PACE_AHEAD) break;
            __builtin_amdgcn_s_sleep(4);
          }
        }
      };
      const TileOffs<KW, 1> koffs = tile_offs<KW, 1>(kst, lane), qoffs = tile_offs<KW, 1>(qst, lane);
      const TileOffs<VW> voffs = tile_offs<VW>(vst, lane);
      float lam_h = 1.f;    // (LT) the lazy state scale, tracked as the consumers apply it
      bool fast_h = false;
      if (nexp > 0) {
        load_k(0, koffs);
        if (nexp > 1) load_k(1, koffs);
        load_v(0, voffs);
        load_scalars(0);
        if (nexp > 1) load_scalars(1);
        if constexpr (!SUM) {
          load_q(0, qoffs);
          if (ntc > 1) load_q(1, qoffs);
        }
        wait_vm();
        lds_barrier();
        lds_barrier();
        if constexpr (LT) {
          scalars(0, lam_h, fast_h);
          block(0, IC<0>{});
        }
        lds_barrier();
      }
      for (int e = 0; e < nexp; ++e) {
        const int c = e / n;
        const int j = e - c * n;
        asm volatile("" : "+v"(hl));
        // phase A: k rows and scalars of chunk e+2 (the Gram stage reads them in
        // chunk e+1), and v rows of chunk e+1 into the slot of chunk e-1 (the
        // consumers read v before the mid-chunk barrier)
        if (e + 2 < nexp) {
          load_k(e + 2, koffs);
          load_scalars(e + 2);
        }
        if (e + 1 < nexp) load_v(e + 1, voffs);
        // q rows of token chunk c+1 at the start of token chunk c, into the slot
        // of token chunk c-1, read last before the previous mid-chunk barrier
        // (the prologue loaded token chunks 0 and 1); with n >= 2 they land
        // before the chunk ends, ahead of the token decay cumsum of token chunk
        // c+1 at sub-chunk n-1 (with n = 1 that cumsum takes its decays from
        // the scalar ring, loaded a chunk earlier).  After the mid-chunk barrier
        // the consumers' output stores then share the vector memory path with
        // no q loads.
        if (!SUM && j == 0 && c >= 1 && c + 1 < ntc) load_q(c + 1, qoffs);
        lds_barrier();
        // phase B.  With per-expanded-chunk outputs the loader also takes the
        // scale scalars and row block 0 of chunk e+1 (its first LDS access waits
        // for the loads of phase A, which the next phase needs anyway).  Then
        // wait for every load: the consumers read the v rows and q rows and the
        // Gram stage the k rows of chunk e+2 after the next barrier.
        if constexpr (LT) {
          if (e + 1 < nexp) {
            scalars(e + 1, lam_h, fast_h);
            block(e + 1, IC<0>{});
          }
        }
        wait_vm();
        // nothing of this wave is in flight: the polls wait for themselves only
        if (prog && e % PACE_EVERY == 0) pace(e);
        lds_barrier();
      }
    } else if (hw == 1) {
      float lam_h = 1.f;    // the lazy state scale, tracked as the consumers apply it
      bool fast_h = false;  // the current token chunk is fast
      if (nexp > 0) {
        lds_barrier();
        lds_barrier();
        if constexpr (!LT) scalars(0, lam_h, fast_h);
        block(0, IC<3>{});
        lds_barrier();
      }
      for (int e = 0; e < nexp; ++e) {
        merge(e);
        lds_barrier();
        if (e + 1 < nexp) {
          if constexpr (!LT) scalars(e + 1, lam_h, fast_h);
          block(e + 1, IC<3>{});
        }
        lds_barrier();
      }
    } else if (hw == 2) {
      if (nexp > 0) {
        lds_barrier();
        prep_scalars(0);
        if constexpr (!SUM && !LT) finish_q(0);
        gram(0, 0, 5, 3);
        lds_barrier();
        if constexpr (!LT) block(0, IC<0>{});
        block(0, IC<1>{});
        lds_barrier();
      }
      for (int e = 0; e < nexp; ++e) {
        const int c = e / n;
        const int j = e - c * n;
        asm volatile("" : "+v"(hl));
        if (e + 1 < nexp) {
          gram(e + 1, 0, 5, 3);
          prep_scalars(e + 1);
        }
        // token chunk c+1: its token decays landed with the loads of a chunk
        // before (the q-row loads with n >= 2, the scalar ring with n = 1)
        if (!SUM && !LT && j == n - 1 && c + 1 < ntc) finish_q(c + 1);
        lds_barrier();
        if (e + 1 < nexp) {
          if constexpr (!LT) block(e + 1, IC<0>{});
          block(e + 1, IC<1>{});
        }
        lds_barrier();
      }
    } else {
      if (nexp > 0) {
        lds_barrier();
        gram(0, 5, 10, 4);
        lds_barrier();
        block(0, IC<2>{});
        if constexpr (!SUM && !LT) tables(0);
        lds_barrier();
      }
      for (int e = 0; e < nexp; ++e) {
        asm volatile("" : "+v"(hl));
        if (e + 1 < nexp) gram(e + 1, 5, 10, 4);
        lds_barrier();
        if (e + 1 < nexp) {
          block(e + 1, IC<2>{});
          if constexpr (!SUM && !LT) tables(e + 1);  // needs the k-row norms from the Gram stage
        }
        lds_barrier();
      }
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
  const int64_t wy_blocks = a.ntdp_rows * a.Hk;
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

// GDP_FUSED_OUTPUTS=token_chunk keeps the per-token-chunk output form for n = 2
// too (the tests run both forms on the same inputs)
bool fused_per_token_chunk() {
  const char *env = std::getenv("GDP_FUSED_OUTPUTS");
  return env && std::strcmp(env, "token_chunk") == 0;
}

template <int K, int V>
hipError_t launch_fused(const PrefillArgs &a, hipStream_t stream) {
  // 4 consumer waves of V/4 state columns and 4 helper waves.  8 consumer waves
  // of 16 columns (the kernel supports it) hide more latency but read every k,
  // k^T, T and P fragment twice as often, which costs more LDS time than it hides.
  constexpr int NCW = 4;
  const int64_t blocks = (int64_t)a.N * a.Hv;
  if (blocks == 0) return hipSuccess;
  if (a.n == 2 && !a.tc_outputs && !fused_per_token_chunk())
    hipLaunchKernelGGL((gdp_fused_kernel<K, V, NCW, false, 2>), dim3((unsigned)blocks), dim3(64 * (NCW + 4)), 0, stream, a);
  else
    hipLaunchKernelGGL((gdp_fused_kernel<K, V, NCW, false>), dim3((unsigned)blocks), dim3(64 * (NCW + 4)), 0, stream, a);
  return hipGetLastError();
}

template <int K, int V>
hipError_t launch_fused_summary(const PrefillArgs &a, hipStream_t stream) {
  constexpr int NCW = 8;
  const int64_t blocks = (int64_t)a.N * a.Hv;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((gdp_fused_kernel<K, V, NCW, true>), dim3((unsigned)blocks), dim3(64 * (NCW + 4)), 0, stream, a);
  return hipGetLastError();
}

// The fused kernel keeps one chain per CU busy for its whole length; it is
// chosen when there are enough chains to give every CU one.  Otherwise the
// split pair (parallel WY kernel, then the scan) spreads the WY work of few
// long chains over the whole chip.
template <typename T, int K, int V>
hipError_t launch_all(const PrefillArgs &a, int path, hipStream_t stream) {
  if (fused_chosen(sizeof(T) == 2 ? IN_BF16 : IN_F32, a.N, a.Hv, path)) {
    if constexpr (sizeof(T) == 2) return launch_fused<K, V>(a, stream);
  }
  return launch_split<T, K, V>(a, stream);
}
}  // namespace

bool fused_chosen(int dtype, int64_t N, int64_t Hv, int path) {
  return dtype == IN_BF16 && (path == PATH_FUSED || (path == PATH_AUTO && N * Hv >= 256));
}

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

hipError_t launch_fused_prefill(const PrefillArgs &a, int K, int V, hipStream_t stream) {
  if (K == 128 && V == 128) {
    PrefillArgs b = a;
    return a.summary ? launch_fused_summary<128, 128>(b, stream) : launch_fused<128, 128>(b, stream);
  }
  if (K == 64 && V == 64) {
    PrefillArgs b = a;
    return a.summary ? launch_fused_summary<64, 64>(b, stream) : launch_fused<64, 64>(b, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_descriptors(const DescArgs &a, hipStream_t stream) {
  hipLaunchKernelGGL(gdp_descriptor_kernel, dim3(1), dim3(1024), 0, stream, a);
  return hipGetLastError();
}

}  // namespace gdp
