// gdp_segments.hip -- gfx950 kernels of the segmented (chunk-parallel) prefill
// for workloads with few (sequence, state head) chains.
//
// A chain's state after a run of tokens is an affine map of the state before
// it, S -> M S + B (blog page "Attention Cache and Sequence Parallelism",
// section "GDN: pass the state, not the KV": each chunk forms an
// input-state -> output-state transition summary, combined by a scan).  Long
// sequences are cut into segments of whole 64-token chunks; the summaries
// (M, B) of all segments are formed in parallel by the fused prefill kernel
// (one workgroup per segment: B from a zero state with the real values, M from
// the identity with zero values, on the same WY matrices), combined in order
// per chain here, and the segments are then run again from their true start
// states.
//
//   gdp_segment_kernel   one workgroup: segment boundaries (as a cu_seqlens of
//                        segments), the first segment of every sequence and
//                        the chunk-state row offset of every segment
//   gdp_combine_kernel   one workgroup per (sequence, state head, 16-column
//                        tile): S = s0; per segment: record S as the segment's
//                        start state, S = M S + B (split-precision bf16 MFMA,
//                        M read straight into the operand registers); final
//                        state and cache slot at the end

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdp_launch.h"

namespace gdp {
namespace {

__device__ __forceinline__ int64_t seg_index_at(const void *p, int is64, int64_t i) {
  return is64 ? ((const int64_t *)p)[i] : (int64_t)((const int32_t *)p)[i];
}

// exclusive block scan of one value per thread (1024 threads); returns the
// prefix and writes the total to *total
__device__ int64_t block_exclusive_scan(int64_t x, int64_t *ws, int64_t *total) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  int64_t v = x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int64_t y = __shfl_up(v, d, 64);
    if (lane >= d) v += y;
  }
  if (lane == 63) ws[w] = v;
  __syncthreads();
  if (w == 0) {
    int64_t u = lane < 16 ? ws[lane] : 0;
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) {
      const int64_t y = __shfl_up(u, d, 64);
      if (lane >= d) u += y;
    }
    if (lane < 16) ws[16 + lane] = u;
  }
  __syncthreads();
  const int64_t before = (w > 0 ? ws[16 + w - 1] : 0) + v - x;
  *total = ws[16 + 15];
  __syncthreads();
  return before;
}

__global__ void __launch_bounds__(1024) gdp_segment_kernel(SegArgs a) {
  __shared__ int64_t ws[32];
  const int t = threadIdx.x;
  // pass 1: first segment of every sequence (ceil(L / Lseg) segments each)
  int64_t carry = 0;
  for (int64_t base = 0; base < a.N; base += 1024) {
    const int64_t i = base + t;
    int64_t cnt = 0;
    if (i < a.N) {
      int64_t t0 = seg_index_at(a.cu, a.cu_is64, i), t1 = seg_index_at(a.cu, a.cu_is64, i + 1);
      t0 = t0 < 0 ? 0 : (t0 > a.T ? a.T : t0);
      t1 = t1 < t0 ? t0 : (t1 > a.T ? a.T : t1);
      cnt = (t1 - t0 + a.Lseg - 1) / a.Lseg;
    }
    int64_t total;
    const int64_t pre = block_exclusive_scan(cnt, ws, &total);
    if (i < a.N) a.seg_first[i] = (int32_t)min(carry + pre, a.ns_cap);
    carry += total;
  }
  if (t == 0) a.seg_first[a.N] = (int32_t)min(carry, a.ns_cap);
  __syncthreads();
  // pass 2: every segment row finds its sequence by binary search
  const int64_t nreal = min(carry, a.ns_cap);
  for (int64_t s = t; s <= a.ns_cap; s += 1024) {
    if (s >= nreal) {  // the end of the last real segment, then zero-length padding
      a.cu_seg[s] = (int32_t)a.T;
      if (s < a.ns_cap) a.seg_cs_off[s] = 0;
      continue;
    }
    int64_t lo = 0, hi = a.N - 1;  // last i with seg_first[i] <= s
    while (lo < hi) {
      const int64_t mid = (lo + hi + 1) / 2;
      if (a.seg_first[mid] <= s) lo = mid; else hi = mid - 1;
    }
    int64_t t0 = seg_index_at(a.cu, a.cu_is64, lo);
    t0 = t0 < 0 ? 0 : (t0 > a.T ? a.T : t0);
    const int64_t k = s - a.seg_first[lo];
    a.cu_seg[s] = (int32_t)min(t0 + k * a.Lseg, a.T);
    a.seg_cs_off[s] = (a.chunk_offsets ? a.chunk_offsets[lo] : 0) + (int32_t)(k * (a.Lseg / 64));
  }
}

// Longest-first order of the fused kernel's chains.  The dispatcher deals
// workgroup b to XCD b mod 8 as that XCD's (b / 8)-th workgroup, and a CU runs
// one fused workgroup at a time, so starting the longest chains first (longest
// processing time first) shortens the tail of mixed-length batches.  Units are
// the groups of grp state heads sharing a q/k head (grp = Hv / Hqk, when the
// grid splits evenly into 8 XCD lists of whole groups; else single heads) in
// decreasing sequence length (ties by index); XCD x takes units x, x + 8, ...
// so that each XCD gets an even mix and a unit's heads share that XCD's L2.
__global__ void __launch_bounds__(1024) gdp_order_kernel(OrderArgs a) {
  __shared__ int32_t len[ORDER_MAX_SEQ];
  __shared__ int32_t by_rank[ORDER_MAX_SEQ];
  const int t = threadIdx.x;
  for (int64_t i = t; i < a.N; i += 1024) {
    int64_t t0 = seg_index_at(a.cu, a.cu_is64, i), t1 = seg_index_at(a.cu, a.cu_is64, i + 1);
    t0 = t0 < 0 ? 0 : (t0 > a.T ? a.T : t0);
    t1 = t1 < t0 ? t0 : (t1 > a.T ? a.T : t1);
    len[i] = (int32_t)(t1 - t0);
  }
  __syncthreads();
  for (int64_t i = t; i < a.N; i += 1024) {
    int32_t r = 0;
    const int32_t li = len[i];
    for (int64_t j = 0; j < a.N; ++j) r += (len[j] > li) || (len[j] == li && j < i);
    by_rank[r] = (int32_t)i;
  }
  __syncthreads();
  const int64_t G = a.N * a.Hv;
  int grp = a.Hv / a.Hqk;
  if (G % (8 * grp) != 0) grp = 1;
  const int64_t units_per_seq = a.Hv / grp;
  for (int64_t b = t; b < G; b += 1024) {
    const int64_t x = b % 8, slot = b / 8;
    const int64_t u = x + 8 * (slot / grp), c = slot % grp;  // unit and head within it
    const int64_t seq = by_rank[u / units_per_seq];
    const int64_t h = (u % units_per_seq) * grp + c;
    a.order[b] = (int32_t)(seq * a.Hv + h);
  }
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Workgroup barrier for LDS only: this wave's LDS accesses are complete, but
// its global loads and stores may still be in flight (__syncthreads waits for
// them too, which would stall every step on the next segment's prefetch).  The
// combine's barriers order LDS traffic only; a register loaded from global
// memory is waited for where it is used.
__device__ __forceinline__ void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// S = M S + B per segment, on a 16-column tile of the state.  Wave w computes
// rows 16 w .. 16 w + 15 of the new tile on bf16 16x16x32 MFMA in three products
// per 32-deep block (split precision: with x_hi = bf16(x) and x_lo = bf16(x -
// x_hi), M S = M_hi S_hi + M_hi S_lo + M_lo S_hi up to the M_lo S_lo term, about
// 2^-16 relative, with fp32 accumulation).  The summary kernel stores M_hi and
// M_lo in the order these A operands are read (msum_index), so they come straight
// into registers, a kilobyte per wave and load, two segments ahead (no workgroup
// ever stages M); only the tile of S goes through LDS, transposed (St[c][k], rows
// padded by four floats so that 16 lanes reading 16-byte pieces of 16 rows meet
// distinct banks) and double buffered, so each segment takes one barrier.  Each
// lane splits its 8 S values of a block into the two bfloat16 parts itself.
template <int K, int V>
__global__ void __launch_bounds__(4 * K) gdp_combine_kernel(CombineArgs a) {
  static_assert(K == 128 || K == 64, "K of 64 or 128");
  constexpr int CT = 16, NCT = V / CT, NU = K / 32, LDR = K + 4;
  __shared__ __attribute__((aligned(16))) float St[2][CT * LDR];
  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Workgroups are dealt to the 8 XCDs round-robin; remap so that each XCD takes
  // a contiguous range of tiles, which keeps the column tiles of one chain (all
  // reading the same M) on one XCD's L2
  const int64_t G = gridDim.x, b0 = blockIdx.x;
  const int64_t bid = (G % 8 == 0) ? (b0 % 8) * (G / 8) + b0 / 8 : b0;
  const int ct = (int)(bid % NCT);
  const int h = (int)((bid / NCT) % a.Hv);
  const int64_t i = bid / ((int64_t)NCT * a.Hv);
  const size_t KV = (size_t)K * V, KK = (size_t)K * K;
  const int c0 = ct * CT, row0 = 16 * w + 4 * lg;  // lane entries: rows row0 .. row0 + 3, column c0 + lr
  f32x4 s;
#pragma unroll
  for (int e = 0; e < 4; ++e) s[e] = a.s0 ? a.s0[((size_t)i * a.Hv + h) * KV + (size_t)(row0 + e) * V + c0 + lr] : 0.f;
  const int64_t s_lo = a.seg_first[i], s_hi = a.seg_first[i + 1];
  // M operands and B entries of three segments in flight: segment sg uses
  // buffer sg mod 3 and issues the loads of segment sg + 2.  The loop runs whole
  // rounds of three steps, and no global load or store in it is conditional, so
  // that the compiler's waits count exactly and a step waits only for its own
  // loads: a step past the last segment loads the last segment again, keeps the
  // tile and stores the last segment's start state again (the same values).
  struct Ops {
    uint4 m[NU][2];  // [block][hi, lo]
    f32x4 b;
  };
  Ops o0, o1, o2;
  auto load = [&](Ops &o, int64_t sg) {
    const uint4 *M = (const uint4 *)(a.msum + ((size_t)sg * a.Hv + h) * KK) + (size_t)w * NU * 2 * 64 + lane;
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int p = 0; p < 2; ++p) o.m[u][p] = M[(2 * u + p) * 64];
    const float *B = a.bsum + ((size_t)sg * a.Hv + h) * KV + c0 + lr;
#pragma unroll
    for (int e = 0; e < 4; ++e) o.b[e] = B[(size_t)(row0 + e) * V];
  };
  f32x4 sin = s;  // the tile entering the last segment stepped through
  auto step = [&](const Ops &o, Ops &onext2, int64_t sg) {
    const bool real = sg < s_hi;
    load(onext2, min(sg + 2, s_hi - 1));  // into the buffer segment sg - 1 used
    if (real) sin = s;
    float *buf = St[sg & 1];
    *(f32x4 *)&buf[lr * LDR + row0] = s;
    float *init = a.seg_init + ((size_t)(real ? sg : s_hi - 1) * a.Hv + h) * KV + c0 + lr;
#pragma unroll
    for (int e = 0; e < 4; ++e) init[(size_t)(row0 + e) * V] = sin[e];
    // every wave's rows are in; the barrier also orders this segment's writes of
    // the other buffer after every wave's reads of it in the segment before
    lds_sync();
    f32x4 acc[3];
    acc[0] = o.b;
    acc[1] = acc[2] = f32x4{0.f, 0.f, 0.f, 0.f};
    const float *sr = &buf[lr * LDR + 8 * lg];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const f32x4 x0 = *(const f32x4 *)(sr + 32 * u), x1 = *(const f32x4 *)(sr + 32 * u + 4);
      bf16x8_t shi, slo;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float x = j < 4 ? x0[j] : x1[j - 4];
        const __bf16 hx = (__bf16)x;
        shi[j] = hx;
        slo[j] = (__bf16)(x - (float)hx);
      }
      const bf16x8_t mhi = __builtin_bit_cast(bf16x8_t, o.m[u][0]), mlo = __builtin_bit_cast(bf16x8_t, o.m[u][1]);
      acc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mhi, shi, acc[0], 0, 0, 0);
      acc[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mhi, slo, acc[1], 0, 0, 0);
      acc[2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mlo, shi, acc[2], 0, 0, 0);
    }
    if (real) s = acc[0] + (acc[1] + acc[2]);
  };
  if (s_lo < s_hi) {
    // the start tile has landed before the prefetches are issued (a wait for it
    // inside the loop would cover every load in flight)
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    load(o0, s_lo);
    load(o1, min(s_lo + 1, s_hi - 1));
    for (int64_t sg = s_lo; sg < s_hi; sg += 3) {
      step(o0, o2, sg);
      step(o1, o0, sg + 1);
      step(o2, o1, sg + 2);
    }
  }
  float *fdst = a.final_state ? a.final_state + ((size_t)i * a.Hv + h) * KV + c0 + lr : nullptr;
  float *cdst = nullptr;
  if (a.cache) {
    const int64_t slot = seg_index_at(a.slots, a.slots_is64, i);
    if (slot >= 0 && slot < a.num_slots) cdst = a.cache + ((size_t)slot * a.Hv + h) * KV + c0 + lr;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (fdst) fdst[(size_t)(row0 + e) * V] = s[e];
    if (cdst) cdst[(size_t)(row0 + e) * V] = s[e];
  }
}

}  // namespace

hipError_t launch_segments(const SegArgs &a, hipStream_t stream) {
  hipLaunchKernelGGL(gdp_segment_kernel, dim3(1), dim3(1024), 0, stream, a);
  return hipGetLastError();
}

// every entry of p[0 .. n) set to v (a kernel, not a memset, so that the call
// stays safe to capture in a graph)
__global__ void __launch_bounds__(256) gdp_fill_kernel(int32_t *p, int64_t n, int32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = v;
}

hipError_t launch_fill(int32_t *p, int64_t n, int32_t v, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024;
  hipLaunchKernelGGL(gdp_fill_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n, v);
  return hipGetLastError();
}

hipError_t launch_order(const OrderArgs &a, hipStream_t stream) {
  if (a.N < 1 || a.N > ORDER_MAX_SEQ) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gdp_order_kernel, dim3(1), dim3(1024), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs &a, int K, int V, hipStream_t stream) {
  const int64_t blocks = (int64_t)a.N * a.Hv * (V / 16);
  if (blocks == 0) return hipSuccess;
  if (K == 128 && V == 128) hipLaunchKernelGGL((gdp_combine_kernel<128, 128>), dim3((unsigned)blocks), dim3(512), 0, stream, a);
  else if (K == 64 && V == 64) hipLaunchKernelGGL((gdp_combine_kernel<64, 64>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace gdp
