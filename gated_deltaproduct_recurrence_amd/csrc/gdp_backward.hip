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
// (k and q here are the L2-normalised rows when the in-kernel norm is on: a
// pre-pass stores each row's norm factor, which scales the products with the
// stored row; a last kernel maps the q and k gradients back to the raw rows.)
//
// The states S_{t-1} are recomputed: the forward pass leaves the state entering
// every 64-token chunk (return_chunk_states); per chunk this kernel re-runs the
// recurrence once to keep the state entering every 8th token in LDS, and once
// per 8-token block to hold the 8 token states in registers, then walks the
// block backwards.  One wave owns one (sequence, state head, V tile of VT
// columns): VT = 4 for K = 128 and 8 for K = 64, with 64 / VT row groups of 8
// state rows; lane = (64 / VT) c + rg holds rows 8 rg .. 8 rg + 7 of column c.
// A column dot over K (on the recurrence's critical path) is then a sum over
// the adjacent lanes of one column, done with DPP moves.  Sums over the tile's
// columns stay in the VALU too: the 8 row entries of a dq or dk partial are
// reduce-scattered over the column lanes with the gfx950 half-wave and row
// swaps (and, for 8 columns, a DPP row rotation), so that each lane ends with
// finished entries.  Gradients shared by several waves (dq, dk: all V tiles and
// the state heads of a q/k head; dbeta, dg_log: all V tiles) go to per-wave LDS
// slots; every few tokens the workgroup (four adjacent V tiles of one chain)
// sums the four waves' slots after a barrier and adds the sums to the zeroed
// output buffers with one float atomic per element.  dv is stored there too,
// coalesced over the workgroup's columns.  A workgroup stays within half the
// CU's LDS and, for n <= 2 with bfloat16 inputs, 256 registers, so two run per
// CU and each SIMD has a second wave to cover stalls.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdp_launch.h"

namespace gdp {
namespace {

constexpr int CH = 64;     // token chunk of the forward pass's chunk states
constexpr int BLK = 8;     // tokens per register block (checkpoint spacing)
constexpr int NMAX = 5;    // Householder rows per token served
constexpr int RKL = 8;     // state rows per lane
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
template <int CTRL> __device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
// sum over the RG lanes of an aligned group (the row groups of one column), in
// every lane, with DPP only: swap neighbours, swap pairs, the two quads of the
// half row, then (RG = 16) the two halves of the row
template <int RG> __device__ __forceinline__ float col_sum(float x) {
  static_assert(RG == 8 || RG == 16, "8 or 16 row groups");
  x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_mov<0x141>(x);  // row_half_mirror
  if constexpr (RG == 16) x += dpp_mov<0x140>(x);  // row_mirror
  return x;
}
// x + the value of the lane whose index differs in bit 5 (W32) or bit 4, for
// the pair (x, y): the half-wave (row) swap leaves (own x, partner's x) in the
// lanes with the bit clear and (partner's y, own y) in the others
template <bool W32> __device__ __forceinline__ float swap_add(float x, float y) {
  const uint32_t ux = __builtin_bit_cast(uint32_t, x), uy = __builtin_bit_cast(uint32_t, y);
  uint32_t r0, r1;
  if constexpr (W32) {
    const auto r = __builtin_amdgcn_permlane32_swap(ux, uy, false, false);
    r0 = r[0];
    r1 = r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane16_swap(ux, uy, false, false);
    r0 = r[0];
    r1 = r[1];
  }
  return __builtin_bit_cast(float, r0) + __builtin_bit_cast(float, r1);
}
// sum over the VT columns of the tile (lane bits 3 .. 5 for 8 columns, 4 .. 5
// for 4), in every lane
template <int VT> __device__ __forceinline__ float row_all(float x) {
  x = swap_add<true>(x, x);
  x = swap_add<false>(x, x);
  if constexpr (VT == 8) x += dpp_mov<0x128>(x);  // row_ror:8, i.e. the lane with bit 3 flipped
  return x;
}
// Reduce-scatter over the VT columns: v holds the lane's R row entries of one
// column; afterwards out[p] is, in lane (c, rg), the sum over the columns of
// entry (R / VT) c + p.  Each stage halves the entries: the lanes with the
// stage's lane bit clear keep the lower half, the others the upper half.
template <int R, int VT> __device__ __forceinline__ void row_scatter(const float (&v)[R], float (&out)[R / VT], bool bit3) {
  static_assert(VT == 4 || VT == 8, "4 or 8 columns");
  float a[R / 2], b[R / 4];
#pragma unroll
  for (int p = 0; p < R / 2; ++p) a[p] = swap_add<true>(v[p], v[p + R / 2]);
#pragma unroll
  for (int p = 0; p < R / 4; ++p) b[p] = swap_add<false>(a[p], a[p + R / 4]);
  if constexpr (VT == 4) {
#pragma unroll
    for (int p = 0; p < R / 4; ++p) out[p] = b[p];
  } else {
#pragma unroll
    for (int p = 0; p < R / 8; ++p) {
      const float keep = bit3 ? b[p + R / 8] : b[p], send = bit3 ? b[p] : b[p + R / 8];
      out[p] = keep + dpp_mov<0x128>(send);
    }
  }
}

template <typename T, int K, int V, int NH> struct Bwd {
  // a wave owns VT columns (4 for K = 128, 8 for K = 64) with RG row groups of
  // RK = 8 rows each: lane = RG c + rg
  static constexpr int VT = K == 128 ? 4 : 8, RG = 64 / VT, RK = K / RG;
  static_assert(RK == RKL, "eight state rows per lane");
  static constexpr int RW = RK * (int)sizeof(T) / 16;  // 16-byte words holding them
  static_assert(RW >= 1, "at least one 16-byte word per lane");
  // the inputs of one token (loaded a token ahead of their use), all as loaded
  // (converted where used, so that the loads stay in flight): the lane's RK
  // entries of the token's k rows (and q row), the rows' L2-norm factors (1
  // without the norm), its beta, log decay, v and output gradient
  struct In {
    uint4 k[NH][RW];
    uint4 q[RW];
    float rk[NH], rq, b[NH], g;
    T v[NH], dov;
  };
  const BwdArgs &a;
  int seq, h, hq, hk, vt, lane, rg, c, col;
  __device__ Bwd(const BwdArgs &args) : a(args) {}

  // the loads of one token, issued where called: the scheduling barrier keeps
  // the compiler from sinking them towards their use, which would undo the
  // prefetch
  __device__ __forceinline__ void load(In &x, int64_t t, bool with_q) const {
    load_(x, t, with_q);
    __builtin_amdgcn_sched_barrier(0);
  }
  __device__ __forceinline__ void load_(In &x, int64_t t, bool with_q) const {
    x.g = a.g[t * a.g_st + (int64_t)h * a.g_sh];
#pragma unroll
    for (int j = 0; j < NH; ++j) {
      if (j < NH) {
        const int64_t r = t * NH + j;
        const uint4 *p = (const uint4 *)((const T *)a.k + r * a.k_st + (int64_t)hk * a.k_sh + RK * rg);
#pragma unroll
        for (int i = 0; i < RW; ++i) x.k[j][i] = p[i];
        x.b[j] = a.beta[r * a.b_st + (int64_t)h * a.b_sh];
        x.rk[j] = a.rk[r * a.rk_st + (int64_t)hk * a.rk_sh];
        x.v[j] = ((const T *)a.v)[r * a.v_st + (int64_t)h * a.v_sh + col];
      }
    }
    if (with_q) {
      const uint4 *p = (const uint4 *)((const T *)a.q + t * a.q_st + (int64_t)hq * a.q_sh + RK * rg);
#pragma unroll
      for (int i = 0; i < RW; ++i) x.q[i] = p[i];
      x.dov = ((const T *)a.dout)[t * a.do_st + (int64_t)h * a.do_sh + col];
      x.rq = a.rq[t * a.rq_st + (int64_t)hq * a.rq_sh];
    }
  }
  // the lane's entries of a row in float, as stored (the norm factor is
  // applied to the products with the row)
  __device__ __forceinline__ void row(float (&o)[RK], const uint4 (&x)[RW]) const {
#pragma unroll
    for (int i = 0; i < RK; ++i) {
      constexpr int PER = 16 / (int)sizeof(T);  // elements per word
      const uint4 wd = x[i / PER];
      const int e = i % PER;
      const uint32_t u32 = (sizeof(T) == 4) ? (e == 0 ? wd.x : e == 1 ? wd.y : e == 2 ? wd.z : wd.w)
                                            : (e / 2 == 0 ? wd.x : e / 2 == 1 ? wd.y : e / 2 == 2 ? wd.z : wd.w);
      o[i] = (sizeof(T) == 4) ? __builtin_bit_cast(float, u32)
                              : __builtin_bit_cast(float, (e & 1) ? (u32 & 0xFFFF0000u) : (u32 << 16));
    }
  }
  // one token forward on the lane's part of S
  __device__ __forceinline__ static float decay(const In &x) { return __builtin_amdgcn_exp2f(x.g * LOG2E_B); }
  __device__ __forceinline__ void step(float (&S)[RK], const In &x) const {
    const float al = decay(x);
#pragma unroll
    for (int i = 0; i < RK; ++i) S[i] *= al;
#pragma unroll
    for (int j = 0; j < NH; ++j) {
      if (j < NH) {
        float kv[RK];
        row(kv, x.k[j]);
        float part = 0.f;
#pragma unroll
        for (int i = 0; i < RK; ++i) part = fmaf(S[i], kv[i], part);
        const float e = x.b[j] * ((float)x.v[j] - x.rk[j] * col_sum<RG>(part));
        const float ek = e * x.rk[j];
#pragma unroll
        for (int i = 0; i < RK; ++i) S[i] = fmaf(kv[i], ek, S[i]);
      }
    }
  }
};

template <typename T, int K, int V, int NH>
__global__ void __launch_bounds__(256, (NH <= 2 && sizeof(T) == 2) ? 2 : 1) gdp_backward_kernel(BwdArgs a) {
  using B = Bwd<T, K, V, NH>;
  using In = typename B::In;
  constexpr int RK = B::RK, VT = B::VT, RG = B::RG, NVT = V / VT;
  // tokens in flight in the forward passes (two where the rows take more registers)
  constexpr int PF = RK * NH > 32 ? 2 : 4;
  // per wave: the state entering each 8-token block of the chunk (64 tokens)
  __shared__ float ck[4][CH / BLK][RK * 64];
  // per token of the current group of F tokens: each wave's finished entries of
  // the dq row (slot 0) and the dk rows (slot 1 + j), summed over the four waves
  // when the group is flushed (sized so that the checkpoints and these fit in LDS)
  // F: the largest of 8, 4, 2, 1 tokens whose slots fit beside the other arrays
  // in half the CU's LDS (two workgroups per CU)
  constexpr int LDS_HALF = 80 * 1024;
  constexpr int FIXED = 4 * (CH / BLK) * RK * 64 * 4 + BLK * (NH + 1) * 4 * 4 + BLK * NH * 4 * VT * 4;
  constexpr int SLOT = (NH + 1) * 4 * K * 4;
  constexpr int F = FIXED + 8 * SLOT <= LDS_HALF ? 8 : FIXED + 4 * SLOT <= LDS_HALF ? 4 : FIXED + 2 * SLOT <= LDS_HALF ? 2 : 1;
  static_assert(FIXED + F * SLOT <= LDS_HALF, "two workgroups per CU");
  __shared__ float wsl[F][NH + 1][4][K];
  // per token of the block and wave, the wave's dg_log (slot 0) and dbeta
  // (slot 1 + j) partials, summed over the waves at the flush
  __shared__ float scal[BLK][NH + 1][4];
  // per token of the block, dv of the workgroup's 4 x 8 columns (written by
  // the wave owning the column, stored with its group's flush)
  __shared__ float dvs[BLK][NH][4 * VT];
  B s(a);
  const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);  // uniform per wave: the chain and its addresses stay scalar
  s.lane = threadIdx.x & 63;
  s.rg = s.lane % RG;
  s.c = s.lane / RG;
  const int64_t wid = (int64_t)blockIdx.x * 4 + w;
  const int64_t nw = (int64_t)a.N * a.Hv * NVT;
  if (wid >= nw) return;  // never taken: the grid holds exactly nw waves (V / 8 is a multiple of 4)
  s.vt = (int)(wid % NVT);
  s.h = (int)((wid / NVT) % a.Hv);
  s.seq = (int)(wid / ((int64_t)NVT * a.Hv));
  s.hq = s.h / (a.Hv / a.Hqk);
  s.hk = s.h / (a.Hv / a.Hk);
  s.col = VT * s.vt + s.c;
  int64_t t0 = idx_at(a.cu, a.cu_is64, s.seq), t1 = idx_at(a.cu, a.cu_is64, s.seq + 1);
  t0 = t0 < 0 ? 0 : (t0 > a.T ? a.T : t0);
  t1 = t1 < t0 ? t0 : (t1 > a.T ? a.T : t1);
  const int ntc = (int)((t1 - t0 + CH - 1) / CH);
  const size_t KV = (size_t)K * V;
  const size_t hoff = (size_t)s.h * KV + (size_t)(RK * s.rg) * V + s.col;  // within one [Hv, K, V] state; + i * V
  const size_t soff = (size_t)s.seq * a.Hv * KV + hoff;
  float *my_ck = &ck[w][0][0];
  const bool bit3 = (s.lane >> 3) & 1;  // (8 columns: the last reduce-scatter stage)

  float dS[RK];
#pragma unroll
  for (int i = 0; i < RK; ++i) dS[i] = a.dfinal ? a.dfinal[soff + (size_t)i * V] : 0.f;

  // the backward walk's token inputs, double-buffered: the next token's are
  // loaded while the current one is used (compile-time buffer indices)
  In buf[2];
  for (int cc = ntc - 1; cc >= 0; --cc) {
    const int64_t tb = t0 + (int64_t)CH * cc;
    const int ntok = (int)((t1 - tb) < CH ? (t1 - tb) : CH);
    const int nblk = (ntok + BLK - 1) / BLK;
    // the state entering the chunk, then the state entering every 8th token
    // (the row comes from descriptors built on cu_seqlens; contents that are not
    // monotone can place it outside the buffer, and then no state is read)
    float S[RK];
    const int64_t csrow = (int64_t)a.chunk_offsets[s.seq] + cc;
    const bool csok = csrow >= 0 && csrow < a.cs_rows;
    const float *src = a.chunk_states + (size_t)(csok ? csrow : 0) * a.Hv * KV + hoff;
#pragma unroll
    for (int i = 0; i < RK; ++i) S[i] = csok ? src[(size_t)i * V] : 0.f;
    const int nstep = BLK * (nblk - 1);  // tokens before the last block's start (a multiple of 8)
    // (block 0's entry is stored before the loop, so that the loop waits for no
    // state load)
#pragma unroll
    for (int i = 0; i < RK; ++i) my_ck[i * 64 + s.lane] = S[i];
    // One forward token is shorter than a load's latency: the forward passes
    // keep the inputs of the next PF tokens in flight, in a ring of registers
    // indexed by compile-time constants.  Every load is issued (past the end of
    // the range, the sequence's or the block's last token is loaded again and not
    // used) and only the arithmetic depends on run-time counts: with no load under
    // a run-time condition the compiler can count the loads in flight exactly.
    const int64_t tseq = t1 - 1;
    In fb[PF];
#pragma unroll
    for (int d = 0; d < PF; ++d) s.load(fb[d], tb + d < tseq ? tb + d : tseq, false);
    for (int m0 = 0; m0 < nstep; m0 += BLK) {
      if (m0 > 0) {
#pragma unroll
        for (int i = 0; i < RK; ++i) my_ck[((m0 / BLK) * RK + i) * 64 + s.lane] = S[i];
      }
#pragma unroll
      for (int i = 0; i < BLK; ++i) {
        s.step(S, fb[i % PF]);
        const int64_t tn = tb + m0 + i + PF;
        s.load(fb[i % PF], tn < tseq ? tn : tseq, false);
      }
    }
#pragma unroll
    for (int i = 0; i < RK; ++i) my_ck[((nblk - 1) * RK + i) * 64 + s.lane] = S[i];
    // blocks backwards
    for (int b = nblk - 1; b >= 0; --b) {
      const int nb = (ntok - BLK * b) < BLK ? (ntok - BLK * b) : BLK;
      const int64_t tbb = tb + BLK * b, tlast = tbb + nb - 1;
      // the backward walk's first token (with q and the output gradient), in buf[1]
      s.load(buf[1], tbb + BLK - 1 < tlast ? tbb + BLK - 1 : tlast, true);
      float ST[BLK][RK];  // state entering token m of the block
#pragma unroll
      for (int i = 0; i < RK; ++i) ST[0][i] = my_ck[(b * RK + i) * 64 + s.lane];
      // token m - 1 of the block moves ST[m-1] to ST[m]; its inputs sit in fb[(m - 1) % PF]
#pragma unroll
      for (int d = 0; d < PF; ++d) s.load(fb[d], tbb + d < tlast ? tbb + d : tlast, false);
#pragma clang loop unroll(full)
      for (int m = 1; m < BLK; ++m) {
        if (m < nb) {
#pragma unroll
          for (int i = 0; i < RK; ++i) ST[m][i] = ST[m - 1][i];
          s.step(ST[m], fb[(m - 1) % PF]);
        }
        if (m - 1 + PF < BLK - 1) {  // token m - 1 + PF is one of the tokens stepped (0 .. BLK - 2)
          const int64_t tn = tbb + m - 1 + PF;
          s.load(fb[(m - 1) % PF], tn < tlast ? tn : tlast, false);
        }
      }
      // backwards over the block: token m's inputs (with q and the output
      // gradient) in buf[m & 1], token m - 1's loaded meanwhile
#pragma clang loop unroll(full)
      for (int m = BLK - 1; m >= 0; --m) {
        const int64_t t = tbb + m;
        In &cur = buf[m & 1];
        if (m > 0) s.load(buf[(m - 1) & 1], t - 1 < tlast ? t - 1 : tlast, true);
        if (m >= nb) continue;
        // recompute the token's sub-states S^j and u_j, e_j
        const float al = B::decay(cur);
        float Sj[NH][RK], u[NH], e[NH];
        float st[RK];
#pragma unroll
        for (int i = 0; i < RK; ++i) st[i] = al * ST[m][i];
#pragma unroll
        for (int j = 0; j < NH; ++j) {
          if (j < NH) {
            float kv[RK];
            s.row(kv, cur.k[j]);
            float part = 0.f;
#pragma unroll
            for (int i = 0; i < RK; ++i) {
              Sj[j][i] = st[i];
              part = fmaf(st[i], kv[i], part);
            }
            u[j] = (float)cur.v[j] - cur.rk[j] * col_sum<RG>(part);
            e[j] = cur.b[j] * u[j];
            const float ek = e[j] * cur.rk[j];
#pragma unroll
            for (int i = 0; i < RK; ++i) st[i] = fmaf(kv[i], ek, st[i]);
          }
        }
        // readout: o_t = scale S_t^T q_t
        float(*wm)[4][K] = wsl[m % F];
        const int el0 = RK * s.rg + (RK / VT) * s.c;  // the row entries this lane finishes
        {
          const float dov = (float)cur.dov * a.scale, dovq = dov * cur.rq;
          float qv[RK], pq[RK], oq[RK / VT];
          s.row(qv, cur.q);
#pragma unroll
          for (int i = 0; i < RK; ++i) {
            pq[i] = st[i] * dov;
            dS[i] = fmaf(qv[i], dovq, dS[i]);
          }
          row_scatter<RK, VT>(pq, oq, bit3);
#pragma unroll
          for (int p = 0; p < RK / VT; ++p) wm[0][w][el0 + p] = oq[p];
        }
#pragma unroll
        for (int j = NH - 1; j >= 0; --j) {
          if (j < NH) {
            float kv[RK];
            s.row(kv, cur.k[j]);
            float part = 0.f;
#pragma unroll
            for (int i = 0; i < RK; ++i) part = fmaf(dS[i], kv[i], part);
            const float de = cur.rk[j] * col_sum<RG>(part);  // equal in the column's RG lanes
            const float du = cur.b[j] * de, duk = du * cur.rk[j];
            dvs[m][j][VT * w + s.c] = du;
            const float db = row_all<VT>(de * u[j]);
            if (s.lane == 0) scal[m][1 + j][w] = db;
            float pk[RK], ok[RK / VT];
#pragma unroll
            for (int i = 0; i < RK; ++i) {
              pk[i] = fmaf(dS[i], e[j], -Sj[j][i] * du);
              dS[i] = fmaf(-kv[i], duk, dS[i]);
            }
            row_scatter<RK, VT>(pk, ok, bit3);
#pragma unroll
            for (int p = 0; p < RK / VT; ++p) wm[1 + j][w][el0 + p] = ok[p];
          }
        }
        // decay
        float part = 0.f;
#pragma unroll
        for (int i = 0; i < RK; ++i) part = fmaf(dS[i], ST[m][i], part);
        const float dal = row_all<VT>(col_sum<RG>(part));
        if (s.lane == 0) scal[m][0][w] = dal * al;
#pragma unroll
        for (int i = 0; i < RK; ++i) dS[i] *= al;
        // the group of tokens m .. m + F - 1 is done: the sums over the four waves,
        // then one float atomic per element (the other contributions: the state
        // heads sharing a q/k head, and the other workgroups of this chain's V tiles)
        if (m % F == 0 && m < nb) {
          __syncthreads();
          const int ng = (nb - m) < F ? (nb - m) : F;  // tokens m .. m + ng - 1 of the block
          // rows (token mm, slot) of the group, EPT at a time over the 256 threads;
          // a wave's 64 threads share one row, so every branch is wave-uniform.
          // All LDS reads are issued before the first atomic.
          constexpr int EPT = 256 / K, NP = F * (NH + 1), IT = (NP + EPT - 1) / EPT;
          const int el = threadIdx.x % K;
          const int sub = __builtin_amdgcn_readfirstlane((int)threadIdx.x / K);  // uniform per wave (K >= 64)
          float sums[IT];
#pragma unroll
          for (int it = 0; it < IT; ++it) {
            const int p = it * EPT + sub, mm = p / (NH + 1), slot = p - mm * (NH + 1);
            sums[it] = p < NP ? (wsl[mm][slot][0][el] + wsl[mm][slot][1][el]) + (wsl[mm][slot][2][el] + wsl[mm][slot][3][el])
                              : 0.f;
          }
#pragma unroll
          for (int it = 0; it < IT; ++it) {
            const int p = it * EPT + sub, mm = p / (NH + 1), slot = p - mm * (NH + 1);
            if (p < NP && mm < ng) {
              const int64_t t = tbb + m + mm;
              if (slot == 0) atomicAdd(a.dq + t * a.dq_st + (int64_t)s.hq * a.dq_sh + el, sums[it]);
              else atomicAdd(a.dk + (t * NH + slot - 1) * a.dk_st + (int64_t)s.hk * a.dk_sh + el, sums[it]);
            }
          }
          if ((int)threadIdx.x < ng * (NH + 1)) {  // dg_log (slot 0) and dbeta (slot 1 + j)
            const int mm = threadIdx.x / (NH + 1), slot = threadIdx.x - mm * (NH + 1);
            const float *sc = scal[m + mm][slot];
            const float sum = (sc[0] + sc[1]) + (sc[2] + sc[3]);
            const int64_t t = tbb + m + mm;
            if (slot == 0) atomicAdd(a.dg + t * a.dg_st + (int64_t)s.h * a.dg_sh, sum);
            else atomicAdd(a.dbeta + (t * NH + slot - 1) * a.db_st + (int64_t)s.h * a.db_sh, sum);
          }
          const int64_t col0 = (int64_t)VT * (s.vt - w);  // the workgroup's first column
          for (int x = threadIdx.x; x < ng * NH * 4 * VT; x += 256) {
            const int mm = x / (NH * 4 * VT), rem = x - mm * (NH * 4 * VT), j = rem / (4 * VT), cc = rem - j * (4 * VT);
            a.dv[((tbb + m + mm) * NH + j) * a.dv_st + (int64_t)s.h * a.dv_sh + col0 + cc] = dvs[m + mm][j][cc];
          }
          __syncthreads();  // before the next group's partials overwrite the slots
        }
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

// The L2-norm factor (|x|^2 + 1e-6)^(-1/2) of each [rows, heads, K] row, into
// a dense [rows, heads] float32 array (g, g_st = heads, g_sh = 1).  One wave per row.
template <typename T, int K>
__global__ void __launch_bounds__(256) gdp_row_norm_kernel(NormGradArgs a) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= a.rows) return;
  const int64_t r = row / a.heads, hh = row % a.heads;
  const T *x = (const T *)a.x + r * a.x_st + hh * a.x_sh;
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < K / 64; ++i) {
    const float xv = (float)x[lane + 64 * i];
    ss = fmaf(xv, xv, ss);
  }
  ss = xsum<1, 32>(ss);
  if (lane == 0) a.g[r * a.g_st + hh * a.g_sh] = __builtin_amdgcn_rsqf(ss + 1e-6f);
}

// Zero the rows of a [T*n, heads, D] float32 tensor (row stride st, head stride
// sh, elements contiguous) that no sequence covers: sub-rows before cu[0]*n and
// from cu[N]*n on (bounds clamped to [0, T] as the other kernels clamp them).
// The backward kernel writes every other row of dv.
__global__ void __launch_bounds__(256) gdp_zero_outside_kernel(ZeroOutsideArgs a) {
  int64_t lo = idx_at(a.cu, a.cu_is64, 0), hi = idx_at(a.cu, a.cu_is64, a.N);
  lo = lo < 0 ? 0 : (lo > a.T ? a.T : lo);
  hi = hi < lo ? lo : (hi > a.T ? a.T : hi);
  lo *= a.n;
  hi *= a.n;
  const int64_t R = a.T * a.n, per_row = (int64_t)a.heads * a.D;
  const int64_t total = (lo + (R - hi)) * per_row;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    int64_t r = i / per_row;
    const int64_t rem = i - r * per_row;
    const int hh = (int)(rem / a.D), d = (int)(rem - (int64_t)hh * a.D);
    if (r >= lo) r += hi - lo;
    a.p[r * a.st + hh * a.sh + d] = 0.f;
  }
}

template <typename T, int K, int V, int NH> hipError_t launch_bwd_n(const BwdArgs &a, hipStream_t stream) {
  constexpr int VT = Bwd<T, K, V, NH>::VT;
  static_assert((V / VT) % 4 == 0, "a workgroup holds four V tiles of one chain");
  const int64_t waves = (int64_t)a.N * a.Hv * (V / VT);
  if (waves == 0) return hipSuccess;
  hipLaunchKernelGGL((gdp_backward_kernel<T, K, V, NH>), dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, stream, a);
  return hipGetLastError();
}
// the number of Householder rows is a template parameter: the per-token loads
// are then unconditional and stay in flight across the token they are hidden by
template <typename T, int K, int V> hipError_t launch_bwd(const BwdArgs &a, hipStream_t stream) {
  switch (a.n) {
    case 1: return launch_bwd_n<T, K, V, 1>(a, stream);
    case 2: return launch_bwd_n<T, K, V, 2>(a, stream);
    case 3: return launch_bwd_n<T, K, V, 3>(a, stream);
    case 4: return launch_bwd_n<T, K, V, 4>(a, stream);
    case 5: return launch_bwd_n<T, K, V, 5>(a, stream);
    default: return hipErrorInvalidValue;
  }
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
  } else if (dtype == IN_F32) {  // the float32 forward serves K = 64
    if (K == 64 && V == 128) return launch_bwd<float, 64, 128>(a, stream);
    if (K == 64 && V == 64) return launch_bwd<float, 64, 64>(a, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_zero_outside(const ZeroOutsideArgs &a, hipStream_t stream) {
  if (a.T * a.n == 0) return hipSuccess;
  hipLaunchKernelGGL(gdp_zero_outside_kernel, dim3(256), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_row_norm(const NormGradArgs &a, int dtype, int K, hipStream_t stream) {
  if (a.rows == 0) return hipSuccess;
  const dim3 grid((unsigned)((a.rows + 3) / 4));
  if (dtype == IN_BF16 && K == 128) hipLaunchKernelGGL((gdp_row_norm_kernel<__bf16, 128>), grid, dim3(256), 0, stream, a);
  else if (dtype == IN_BF16 && K == 64) hipLaunchKernelGGL((gdp_row_norm_kernel<__bf16, 64>), grid, dim3(256), 0, stream, a);
  else if (dtype == IN_F32 && K == 128) hipLaunchKernelGGL((gdp_row_norm_kernel<float, 128>), grid, dim3(256), 0, stream, a);
  else if (dtype == IN_F32 && K == 64) hipLaunchKernelGGL((gdp_row_norm_kernel<float, 64>), grid, dim3(256), 0, stream, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
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
