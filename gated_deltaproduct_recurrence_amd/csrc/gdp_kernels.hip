// gdp_kernels.hip -- gfx950 (CDNA4) kernels of chunked Gated DeltaProduct prefill.
//
// Method (FlashInfer docs, "flashinfer.gdp_prefill.chunk_gated_delta_product",
// recurrence display; Megatron Core API docs, core.ssm.ops.gdp.chunk, stage list):
// per token the K x V state S decays by alpha_t, then takes n beta-gated
// Householder updates from the sub-token rows t*n..t*n+n-1, then is read out.
// The chunked form used here works on 64-row chunks of the Householder-expanded
// stream.  For an expanded chunk with start state S0, rows r, base-2 cumulative
// log decay G_r (decays sit on the first sub-row of each token, Megatron stage 1),
// and A[r,i] = beta_r 2^(G_r - G_i) k_r.k_i for i < r:
//     T = (I + A)^-1                                  (WY step, Megatron stage 2)
//     E = T (diag(beta) V - diag(beta 2^G) K S0)      (= U - W S0, the v_new rows)
//     S_end = 2^G_last S0 + K^T diag(2^(G_last - G)) E  (state sweep, stage 3)
// and for the token chunk c (n expanded chunks) with start state h_c,
//     o_t = scale (2^Gt_t q_t^T h_c + sum_{r: tok(r) <= t} 2^(Gt_t - Gt_tok(r)) (q_t.k_r) e_r)
// (output combine, stage 4), Gt being the token-stream cumulative decay.
//
// Design for CDNA4: one workgroup (4 waves) owns one (sequence, state head,
// V-tile) chain and walks its chunks in order, so S never leaves the CU.  S is
// held fp32 in MFMA accumulators; wave w owns a 16*NB-column slab of S, so the
// S-dependent products (K S, Q S) take S straight from registers as the B
// operand and the sweep needs no cross-wave exchange.  Chunk-local operands
// (K, K^T, Q, V, T, P) are staged in LDS and read as A operands.  All
// contractions run on v_mfma_f32_16x16x32_bf16 (bf16 inputs) or
// v_mfma_f32_16x16x4_f32 (f32 inputs) with fp32 accumulation; the 64 x 64
// triangular inverse is solved in fp32.

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

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

template <typename T> __device__ __forceinline__ float to_f(T x) { return (float)x; }

// ---------------------------------------------------------------- shared memory

template <typename T, int K, int NB> struct Smem {
  static constexpr int EPS = 16 / (int)sizeof(T);  // elements per 16-byte segment
  static constexpr int BV = 64 * NB;                // state columns per workgroup
  static constexpr int LDK = K + EPS;               // k, q rows
  static constexpr int LDKT = CH + EPS;             // k^T rows
  static constexpr int LDV = BV + EPS;              // v rows
  static constexpr int LDC = CH + EPS;              // T, P rows (type T)
  static constexpr int LDA = CH + 4;                // A and fp32 T rows
  static constexpr bool kTinF32 = sizeof(T) == 4;   // fp32 inputs: T is read from tf
  T k[CH * LDK];
  T kt[K * LDKT];
  T q[CH * LDK];
  T v[CH * LDV];
  float a[CH * LDA];
  float tf[CH * LDA];
  T t[kTinF32 ? 4 : CH * LDC];
  T p[CH * LDC];
  float gtok[CH], gdp[CH], beta[CH], rk[CH], rq[CH];
};

// ---------------------------------------------------------------- small helpers

__device__ __forceinline__ int64_t load_index(const void *p, int is64, int64_t i) {
  return is64 ? ((const int64_t *)p)[i] : (int64_t)((const int32_t *)p)[i];
}

union Seg16 {
  uint4 u;
  bf16 h[8];
  float f[4];
};

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

// k rows into LDS twice: row-major (sk) and transposed (skt, row = key dim).
// Each work unit is 4 rows x one 16-byte segment, so the transposed copy is
// written as 4-element runs.
template <typename T, int K, int LDK, int LDKT>
__device__ __forceinline__ void load_k_both(T *sk, T *skt, const T *src, int64_t rs, int nvalid,
                                            int tid) {
  constexpr int EPS = 16 / (int)sizeof(T), CB = K / EPS;
  for (int u = tid; u < (CH / 4) * CB; u += NTHR) {
    const int rb = u / CB, cb = u % CB;
    Seg16 x[4];
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      const int r = 4 * rb + qd;
      x[qd].u = uint4{0u, 0u, 0u, 0u};
      if (r < nvalid) x[qd].u = *(const uint4 *)(src + (int64_t)r * rs + cb * EPS);
      *(uint4 *)(sk + r * LDK + cb * EPS) = x[qd].u;
    }
#pragma unroll
    for (int e = 0; e < EPS; ++e) {
      T *d = skt + (cb * EPS + e) * LDKT + 4 * rb;
      if constexpr (sizeof(T) == 2) {
        bf16x4 w = {x[0].h[e], x[1].h[e], x[2].h[e], x[3].h[e]};
        *(bf16x4 *)d = w;
      } else {
        f32x4 w = {x[0].f[e], x[1].f[e], x[2].f[e], x[3].f[e]};
        *(f32x4 *)d = w;
      }
    }
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
// T = (I + A)^-1 for the strictly lower-triangular 64 x 64 A in sm.a, in fp32.
// Diagonal 16 x 16 blocks by forward substitution (wave 0, one lane per
// column of each block), then the off-diagonal blocks by
//     T_ab = -T_aa sum_{c=b}^{a-1} A_ac T_cb,
// one sweep per block distance a - b, on fp32 MFMA.  The result (zeros above
// the diagonal blocks) goes to sm.t (bf16) or stays in sm.tf (f32).
template <typename T, int K, int NB>
__device__ __forceinline__ void wy_inverse(Smem<T, K, NB> &sm, int tid) {
  using S = Smem<T, K, NB>;
  constexpr int LDA = S::LDA;
  const int w = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  if (w == 0) {
    const int bk = lg, j = lr;
    const float *A = sm.a + (16 * bk) * LDA + 16 * bk;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < r; ++i) s = fmaf(A[r * LDA + i], x[i], s);
      x[r] = (r == j ? 1.f : 0.f) - s;
    }
    float *Td = sm.tf + (16 * bk) * LDA + 16 * bk + j;
#pragma unroll
    for (int r = 0; r < 16; ++r) Td[r * LDA] = x[r];
  } else {
    // zero the blocks strictly above the diagonal (rows 16a.., cols 16b.., b > a)
    for (int idx = tid - 64; idx < 6 * 256; idx += NTHR - 64) {
      const int blk = idx >> 8, e = idx & 255;
      const int a = (blk < 3) ? 0 : (blk < 5 ? 1 : 2);
      const int b = (blk < 3) ? blk + 1 : (blk < 5 ? blk - 1 : 3);
      sm.tf[(16 * a + (e >> 4)) * LDA + 16 * b + (e & 15)] = 0.f;
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
          const float av = sm.a[(16 * ba + lr) * LDA + 16 * c + 4 * kk + lg];
          const float bv = sm.tf[(16 * c + 4 * kk + lg) * LDA + 16 * bb + lr];
          y = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, y, 0, 0, 0);
        }
      }
      f32x4 z = zero4();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float av = sm.tf[(16 * ba + lr) * LDA + 16 * ba + 4 * lg + i];
        z = __builtin_amdgcn_mfma_f32_16x16x4f32(av, y[i], z, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.tf[(16 * ba + 4 * lg + i) * LDA + 16 * bb + lr] = -z[i];
    }
    __syncthreads();
  }
  if constexpr (!S::kTinF32) {
    for (int idx = tid; idx < CH * CH; idx += NTHR) {
      const int r = idx >> 6, c = idx & 63;
      sm.t[r * S::LDC + c] = (bf16)sm.tf[r * LDA + c];
    }
  }
}

// ---------------------------------------------------------------- fused kernel

template <typename T, int K, int V, int NB>
__global__ void __launch_bounds__(NTHR, 1) gdp_fused_kernel(FusedArgs a) {
  using S = Smem<T, K, NB>;
  constexpr int BV = S::BV, NVT = V / BV, KT16 = K / 16, KS = K / 32;
  constexpr int LDK = S::LDK, LDKT = S::LDKT, LDV = S::LDV, LDC = S::LDC;
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
  const int wcol = w * 16 * NB;        // first column of this wave inside the tile
  const int gcol = vt * BV + wcol;     // ... and inside the head

  const T *qg = (const T *)a.q + hq * a.q_sh;
  const T *kg = (const T *)a.k + hq * a.k_sh;
  const T *vg = (const T *)a.v + h * a.v_sh + vt * BV;
  const size_t KV = (size_t)K * V;
  const size_t state_off = ((size_t)seq * a.Hv + h) * KV;

  // ---- state S (K x BV slab of this wave): fp32 accumulators
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
  Frag<T> Sb[KS][NB];
#pragma unroll
  for (int s = 0; s < KS; ++s)
#pragma unroll
    for (int b = 0; b < NB; ++b) from_acc(Sb[s][b], Sacc[2 * s][b], Sacc[2 * s + 1][b]);

  const int64_t nchunks = (L + CH - 1) / CH;
  for (int64_t c = 0; c < nchunks; ++c) {
    const int ntok = (int)((L - CH * c) < CH ? (L - CH * c) : CH);
    const int64_t tokbase = t0 + CH * c;

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
              dst[(size_t)(16 * at + 4 * lg + i) * V + gcol + 16 * b + lr] = Sacc[at][b][i];
      }
    }

    __syncthreads();  // previous chunk is done with sm.q / sm.gtok
    load_rows<T, K, LDK>(sm.q, qg + tokbase * a.q_st, a.q_st, ntok, tid);
    if (w == 0) {
      float x = (lane < ntok) ? a.g[(tokbase + lane) * a.g_st + h * a.g_sh] * LOG2E : 0.f;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off);
        if (lane >= off) x += y;
      }
      sm.gtok[lane] = x;
    }
    __syncthreads();
    if (a.l2norm) rows_rstd<T, K>(sm.q, LDK, sm.rq, tid);
    else if (tid < CH) sm.rq[tid] = 1.f;
    __syncthreads();

    // O = diag(2^Gt * rq) Q h_c
    f32x4 O[4][NB];
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4)
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        f32x4 acc = zero4();
#pragma unroll
        for (int s = 0; s < KS; ++s) acc = mma(lds_perm(sm.q, LDK, 16 * a4 + lr, 32 * s, lg), Sb[s][b], acc);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * a4 + 4 * lg + i;
          acc[i] *= exp2f(sm.gtok[r]) * sm.rq[r];
        }
        O[a4][b] = acc;
      }

    for (int j = 0; j < n; ++j) {
      const int64_t s0 = (int64_t)CH * (c * n + j);  // sub-token offset inside the sequence
      if (s0 >= nsub) break;
      const int nrow = (int)((nsub - s0) < CH ? (nsub - s0) : CH);
      // first token of the sequence whose decay lies in this expanded chunk, minus one,
      // relative to the token chunk: G of the rows before this expanded chunk
      const int64_t prev_tok = (s0 + n - 1) / n - 1 - CH * c;

      __syncthreads();  // previous expanded chunk is done with k / v / t / p
      const int64_t krow0 = t0 * n + s0;
      load_k_both<T, K, LDK, LDKT>(sm.k, sm.kt, kg + krow0 * a.k_st, a.k_st, nrow, tid);
      load_rows<T, BV, LDV>(sm.v, vg + krow0 * a.v_st, a.v_st, nrow, tid);
      if (tid < CH) {
        const int r = tid;
        const int rr = r < nrow ? r : nrow - 1;
        const int tk = (int)((s0 + rr) / n - CH * c);
        const float gp = prev_tok >= 0 ? sm.gtok[prev_tok] : 0.f;
        sm.gdp[r] = sm.gtok[tk] - gp;
        sm.beta[r] = (r < nrow) ? a.beta[(krow0 + r) * a.b_st + h * a.b_sh] : 0.f;
      }
      __syncthreads();
      if (a.l2norm) rows_rstd<T, K>(sm.k, LDK, sm.rk, tid);
      else if (tid < CH) sm.rk[tid] = 1.f;
      __syncthreads();

      // Gram K K^T -> A (strictly lower, scaled), and scores Q K^T -> P (masked, scaled)
      for (int tt = w; tt < 32; tt += 4) {
        if (tt < 16) {
          const int ra = tt >> 2, rb = tt & 3;
          if (rb > ra) continue;
          f32x4 acc = zero4();
#pragma unroll
          for (int s = 0; s < KS; ++s)
            acc = mma(lds_contig(sm.k, LDK, 16 * ra + lr, 32 * s, lg),
                      lds_contig(sm.k, LDK, 16 * rb + lr, 32 * s, lg), acc);
          const int col = 16 * rb + lr;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 16 * ra + 4 * lg + i;
            float val = 0.f;
            if (col < r)
              val = sm.beta[r] * sm.rk[r] * sm.rk[col] * exp2f(sm.gdp[r] - sm.gdp[col]) * acc[i];
            sm.a[r * S::LDA + col] = val;
          }
        } else {
          const int ta = (tt - 16) >> 2, tb = (tt - 16) & 3;
          f32x4 acc = zero4();
#pragma unroll
          for (int s = 0; s < KS; ++s)
            acc = mma(lds_contig(sm.q, LDK, 16 * ta + lr, 32 * s, lg),
                      lds_contig(sm.k, LDK, 16 * tb + lr, 32 * s, lg), acc);
          const int r = 16 * tb + lr;
          const int rr = r < nrow ? r : nrow - 1;
          const int tk = (int)((s0 + rr) / n - CH * c);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = 16 * ta + 4 * lg + i;
            float val = 0.f;
            if (r < nrow && tk <= t)
              val = sm.rq[t] * sm.rk[r] * exp2f(sm.gtok[t] - sm.gtok[tk]) * acc[i];
            sm.p[t * LDC + r] = (T)val;
          }
        }
      }

      // R = diag(beta) V - diag(beta 2^G rk) K S0   (this wave's columns)
      f32x4 R[4][NB];
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4)
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          f32x4 x = zero4();
#pragma unroll
          for (int s = 0; s < KS; ++s) x = mma(lds_perm(sm.k, LDK, 16 * a4 + lr, 32 * s, lg), Sb[s][b], x);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 16 * a4 + 4 * lg + i;
            const float bt = sm.beta[r];
            const float vv = to_f(sm.v[r * LDV + wcol + 16 * b + lr]);
            x[i] = bt * vv - bt * exp2f(sm.gdp[r]) * sm.rk[r] * x[i];
          }
          R[a4][b] = x;
        }
      __syncthreads();  // A complete

      wy_inverse<T, K, NB>(sm, tid);
      __syncthreads();  // T complete
      const T *Tm = S::kTinF32 ? (const T *)sm.tf : sm.t;
      constexpr int LDT = S::kTinF32 ? S::LDA : LDC;

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
          f32x4 e = zero4();
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            if (s == 1 && a4 < 2) continue;  // T is lower triangular
            e = mma(lds_perm(Tm, LDT, 16 * a4 + lr, 32 * s, lg), Rb[s][b], e);
          }
          E[a4][b] = e;
        }

      // O += P E
      Frag<T> Eb[2][NB];
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int b = 0; b < NB; ++b) from_acc(Eb[s][b], E[2 * s][b], E[2 * s + 1][b]);
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4)
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int s = 0; s < 2; ++s)
            O[a4][b] = mma(lds_perm(sm.p, LDC, 16 * a4 + lr, 32 * s, lg), Eb[s][b], O[a4][b]);

      // S = 2^G_last S + K^T diag(2^(G_last - G) rk) E
      const float glast = sm.gdp[CH - 1];
      const float dlast = exp2f(glast);
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4)
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 16 * a4 + 4 * lg + i;
            E[a4][b][i] *= exp2f(glast - sm.gdp[r]) * sm.rk[r];
          }
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int b = 0; b < NB; ++b) from_acc(Eb[s][b], E[2 * s][b], E[2 * s + 1][b]);
#pragma unroll
      for (int at = 0; at < KT16; ++at)
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          f32x4 acc = Sacc[at][b] * dlast;
#pragma unroll
          for (int s = 0; s < 2; ++s) acc = mma(lds_perm(sm.kt, LDKT, 16 * at + lr, 32 * s, lg), Eb[s][b], acc);
          Sacc[at][b] = acc;
        }
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int b = 0; b < NB; ++b) from_acc(Sb[s][b], Sacc[2 * s][b], Sacc[2 * s + 1][b]);
    }

    // o rows of this token chunk
    T *og = (T *)a.o + h * a.o_sh + gcol;
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * a4 + 4 * lg + i;
        if (t < ntok) {
#pragma unroll
          for (int b = 0; b < NB; ++b) og[(tokbase + t) * a.o_st + 16 * b + lr] = (T)(O[a4][b][i] * a.scale);
        }
      }
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
        if (fdst) fdst[off] = Sacc[at][b][i];
        if (cdst) cdst[off] = Sacc[at][b][i];
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
hipError_t launch_one(const FusedArgs &a, hipStream_t stream) {
  constexpr int NVT = V / (64 * NB);
  const int64_t blocks = (int64_t)a.N * a.Hv * NVT;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((gdp_fused_kernel<T, K, V, NB>), dim3((unsigned)blocks), dim3(NTHR), 0, stream, a);
  return hipGetLastError();
}

// Wider V-tiles when there are enough chains to fill the chip; narrower ones
// otherwise, so that few long chains still spread over more CUs.
template <typename T, int K, int V>
hipError_t launch_v(const FusedArgs &a, hipStream_t stream) {
  if constexpr (V == 128 && sizeof(T) == 2) {
    if ((int64_t)a.N * a.Hv * 2 > 256) return launch_one<T, K, V, 2>(a, stream);
  }
  return launch_one<T, K, V, 1>(a, stream);
}
}  // namespace

bool fused_supported(int dtype, int K, int V) {
  const bool kv = (K == 64 || K == 128) && (V == 64 || V == 128);
  if (dtype == IN_BF16) return kv;
  if (dtype == IN_F32) return kv && K == 64;
  return false;
}

hipError_t launch_fused(const FusedArgs &a, int dtype, int K, int V, hipStream_t stream) {
  if (dtype == IN_BF16) {
    if (K == 128 && V == 128) return launch_v<bf16, 128, 128>(a, stream);
    if (K == 128 && V == 64) return launch_v<bf16, 128, 64>(a, stream);
    if (K == 64 && V == 128) return launch_v<bf16, 64, 128>(a, stream);
    if (K == 64 && V == 64) return launch_v<bf16, 64, 64>(a, stream);
  } else if (dtype == IN_F32) {
    if (K == 64 && V == 64) return launch_v<float, 64, 64>(a, stream);
    if (K == 64 && V == 128) return launch_v<float, 64, 128>(a, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_descriptors(const DescArgs &a, hipStream_t stream) {
  hipLaunchKernelGGL(gdp_descriptor_kernel, dim3(1), dim3(1024), 0, stream, a);
  return hipGetLastError();
}

}  // namespace gdp
