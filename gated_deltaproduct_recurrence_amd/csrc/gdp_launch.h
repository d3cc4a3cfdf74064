// gdp_launch.h -- internal interface between the C ABI (gdp_api.cpp) and the
// gfx950 kernels (gdp_kernels.hip).  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdp {

// Arguments of the descriptor builder (both chunkings).
struct DescArgs {
  const void *cu;  // [N+1] int32 or int64
  int cu_is64;
  int64_t N;
  int n;
  int64_t nt_cap, ntdp_cap;
  int32_t *chunk_indices, *chunk_indices_dp, *chunk_offsets, *chunk_offsets_dp;
};

// Arguments shared by the WY kernel and the scan/output kernel.  Strides are
// in elements.
struct PrefillArgs {
  const void *q; int64_t q_st, q_sh;
  const void *k; int64_t k_st, k_sh;
  const void *v; int64_t v_st, v_sh;
  const float *g; int64_t g_st, g_sh;
  const float *beta; int64_t b_st, b_sh;
  const void *cu; int cu_is64;
  int64_t T;
  int N, n, Hqk, Hv;
  int Hk;                // k heads: Hqk or Hv (state head h reads k head h / (Hv / Hk))
  float scale;
  int l2norm;
  const float *s0;       // [N, Hv, K, V] or null
  float *final_state;    // [N, Hv, K, V] or null
  float *cache;          // [num_slots, Hv, K, V] or null
  const void *slots; int slots_is64; int64_t num_slots;
  float *chunk_states;   // [cs_rows, Hv, K, V] or null
  int64_t cs_rows;
  const int32_t *chunk_offsets;     // [N+1]
  const int32_t *chunk_indices_dp;  // [ntdp_rows, 2]
  const int32_t *chunk_offsets_dp;  // [N+1]
  int64_t ntdp_rows;                // rows of chunk_indices_dp (WY grid)
  void *tws;                        // WY matrices: [tws_rows, Hv, 64*64] input dtype, fragment order
  int64_t tws_rows;
  void *o; int64_t o_st, o_sh;      // null: no outputs (the segment summaries of the fused kernel)
  // Segment summaries (fused kernel only, K == V): one workgroup per chain
  // forms both maps.  Its B waves run from a zero state with the real values
  // and write their final state (B of the segment's map S -> M S + B) to
  // final_state; its M waves run from the identity with zero values and write
  // their final state (M) to msum as a bfloat16 hi/lo pair, in the msum_index
  // order.
  int summary;
  float *msum;                      // [N, Hv, K * K]
  // fused kernel, n = 2: outputs per token chunk instead of per expanded chunk
  // (the backward's forward pass asks for it: its chunk states then come from
  // the per-token-chunk decay logic, whose rounding its decay gradients were
  // checked against)
  int tc_outputs;
  // fused kernel: chain run by workgroup b (longest sequences first, spread over
  // the XCDs), or null for the plain XCD-grouped order
  const int32_t *order;             // [N * Hv]
  // fused kernel: chunk progress of every chain, or null.  The state heads of
  // one q/k head read the same k/q rows; a chain more than a few chunks ahead of
  // another of its group waits (bounded) so that the group shares those rows
  // through its XCD's L2 instead of fetching them once per head.
  int32_t *progress;                // [N * Hv]
};

// Longest-first order of the fused kernel's chains (one workgroup).
struct OrderArgs {
  const void *cu; int cu_is64;
  int64_t N, T;
  int Hqk, Hv;
  int32_t *order;                   // [N * Hv]
};

enum InDtype { IN_F32 = 0, IN_BF16 = 1 };

// Arguments of the single-token decode step (strides in elements).
struct DecodeArgs {
  const void *q; int64_t q_st, q_sh;      // [N, Hqk, K]
  const void *k; int64_t k_st, k_sh;      // [N*n, Hk, K]
  const void *v; int64_t v_st, v_sh;      // [N*n, Hv, V]
  const float *g; int64_t g_st, g_sh;     // [N, Hv]
  const float *beta; int64_t b_st, b_sh;  // [N*n, Hv]
  int N, n, Hqk, Hv;
  int Hk;                                 // k heads: Hqk or Hv
  float scale;
  int l2norm;
  float *cache; int64_t num_slots;        // [num_slots, Hv, K, V], read and written in place
  const void *slots; int slots_is64;      // [N]
  void *o; int64_t o_st, o_sh;            // [N, Hv, V]
};

// Kernel path: AUTO picks the fused single kernel for bf16 when there are at
// least 256 (sequence, state head) chains, the segmented path (fused kernel on
// segments of long sequences) for bf16 with fewer chains and long sequences,
// else the WY kernel + scan kernel pair.
enum Path { PATH_AUTO = 0, PATH_FUSED = 1, PATH_SPLIT = 2, PATH_SEGMENTED = 3 };

bool prefill_supported(int dtype, int K, int V);
// Bytes of the WY-matrix buffer for `rows` expanded chunks and Hv heads.
size_t wy_buffer_bytes(int dtype, int64_t rows, int64_t Hv);
hipError_t launch_prefill(const PrefillArgs &a, int dtype, int K, int V, int path, hipStream_t stream);
hipError_t launch_descriptors(const DescArgs &a, hipStream_t stream);
// Segmented prefill: segment boundaries of every sequence (segments of Lseg
// tokens, a multiple of 64), padded to ns_cap zero-length segments at T.
struct SegArgs {
  const void *cu; int cu_is64;
  int64_t N, T, Lseg, ns_cap;
  const int32_t *chunk_offsets;  // [N+1] token-chunk offsets of the sequences
  int32_t *cu_seg;               // [ns_cap+1] segment boundaries (a cu_seqlens of segments)
  int32_t *seg_first;            // [N+1] first segment of every sequence
  int32_t *seg_cs_off;           // [ns_cap] chunk-state row of every segment's first chunk
};
// Layout of one K x K summary M in the msum buffer (K * K floats' room): M is
// kept as a pair of bfloat16 matrices, M_hi = bf16(M) and M_lo = bf16(M - M_hi),
// in the order the combine kernel reads its MFMA A operands, so that each of its
// loads is one contiguous kilobyte per wave.  Wave w of the combine computes rows
// 16 w .. 16 w + 15; for the 32-deep reduction block u its lane (lg, lr) holds
// M[16 w + lr][32 u + 8 lg .. + 7] of part p (0: hi, 1: lo) as one 16-byte piece.
// msum_index gives the bfloat16 element index of entry (k, c) of part p.
template <int K> __host__ __device__ constexpr int msum_index(int k, int c, int p) {
  return (((((k >> 4) * (K / 32) + (c >> 5)) * 2 + p) * 64 + 16 * ((c >> 3) & 3) + (k & 15)) << 3) + (c & 7);
}
// Segmented prefill: the in-order combination of the segment summaries.
struct CombineArgs {
  int N, Hv;
  const int32_t *seg_first;      // [N+1]
  const float *msum, *bsum;      // [ns, Hv, K, K] and [ns, Hv, K, V]
  float *seg_init;               // [ns, Hv, K, V] start state of every segment (written)
  const float *s0;               // [N, Hv, K, V] or null
  float *final_state;            // [N, Hv, K, V] or null
  float *cache; const void *slots; int slots_is64; int64_t num_slots;
};
// whether launch_prefill runs the fused kernel (else the split pair) for this
// input dtype, grid and path
bool fused_chosen(int dtype, int64_t N, int64_t Hv, int path);
hipError_t launch_segments(const SegArgs &a, hipStream_t stream);
// sequences the ordering kernel can rank (LDS-resident lengths)
constexpr int64_t ORDER_MAX_SEQ = 4096;
hipError_t launch_order(const OrderArgs &a, hipStream_t stream);

// Gradients of the prefill (recurrent reverse pass; gdp_backward.hip).
struct BwdArgs {
  const void *q; int64_t q_st, q_sh;        // [T, Hqk, K]
  const void *k; int64_t k_st, k_sh;        // [T*n, Hk, K]
  const void *v; int64_t v_st, v_sh;        // [T*n, Hv, V]
  const float *g; int64_t g_st, g_sh;       // [T, Hv] log decays
  const float *beta; int64_t b_st, b_sh;    // [T*n, Hv]
  const void *cu; int cu_is64;
  int64_t T;
  int N, n, Hqk, Hv, Hk;
  float scale;
  // the rows' L2-norm factors, [T, Hqk] and [T*n, Hk] float32; without the norm
  // a single 1 with zero strides
  const float *rq; int64_t rq_st, rq_sh;
  const float *rk; int64_t rk_st, rk_sh;
  const float *chunk_states;                // [cs_rows, Hv, K, V]: state entering each token chunk
  int64_t cs_rows;                          // rows of chunk_states; a row index outside [0, cs_rows)
                                            // (bad cu_seqlens contents) reads a zero state instead
  const int32_t *chunk_offsets;             // [N+1]
  const void *dout; int64_t do_st, do_sh;   // [T, Hv, V], the inputs' dtype
  const float *dfinal;                      // [N, Hv, K, V] or null
  // outputs (float32): dq, dk, dbeta, dg accumulate into zeroed buffers
  float *dq; int64_t dq_st, dq_sh;
  float *dk; int64_t dk_st, dk_sh;
  float *dv; int64_t dv_st, dv_sh;
  float *dg; int64_t dg_st, dg_sh;
  float *dbeta; int64_t db_st, db_sh;
  float *ds0;                               // [N, Hv, K, V] or null
};
bool backward_supported(int K, int V, int n);

// Chunked gradients on the matrix cores (gdp_bwd_chunk.hip): prep, reverse
// state-gradient scan and per-chunk gradient kernels.  bf16 inputs; q, k, v and
// d_o rows 16-byte aligned.
struct BwdChunkArgs {
  const void *q; int64_t q_st, q_sh;        // [T, Hqk, K]
  const void *k; int64_t k_st, k_sh;        // [T*n, Hk, K]
  const void *v; int64_t v_st, v_sh;        // [T*n, Hv, V]
  const float *g; int64_t g_st, g_sh;       // [T, Hv] log decays
  const float *beta; int64_t b_st, b_sh;    // [T*n, Hv]
  const void *cu; int cu_is64;
  int64_t T;
  int N, n, Hqk, Hv, Hk;
  float scale;
  int l2norm;
  const int32_t *chunk_indices_dp;          // [ntdp_rows, 2]
  const int32_t *chunk_offsets_dp;          // [N+1]
  int64_t ntdp_rows;
  char *bundle;                             // [ntdp_rows, Hv] x bwd_bundle_bytes(n): prep output
  const float *s0;                          // [N, Hv, K, V] initial states or null
  char *states;                             // [ntdp_rows, Hv] x bwd_state_record_bytes(K, V): W = K S0 and
                                            // S0 (bf16) of the state entering each expanded chunk
  float *dstates;                           // [ntdp_rows, Hv, K, V] dL/d(state leaving each expanded chunk)
  const void *dout; int64_t do_st, do_sh;   // [T, Hv, V]
  const float *dfinal;                      // [N, Hv, K, V] or null
  float *ds0;                               // [N, Hv, K, V] or null
  // outputs (float32), each entry inside the sequences stored once (dq and dk
  // through the L2-norm gradient when the in-kernel norm is on)
  float *dq; int64_t dq_st, dq_sh;
  float *dk; int64_t dk_st, dk_sh;
  float *dv; int64_t dv_st, dv_sh;
  float *dg; int64_t dg_st, dg_sh;
  float *dbeta; int64_t db_st, db_sh;
};
size_t bwd_bundle_bytes(int n);
size_t bwd_state_record_bytes(int K, int V);
bool bwd_chunked_supported(int dtype, int K, int V, int n);
hipError_t launch_bwd_chunked(const BwdChunkArgs &a, int K, int V, hipStream_t stream);
hipError_t launch_backward(const BwdArgs &a, int dtype, int K, int V, hipStream_t stream);

// Zero fill of the rows of a strided [T*n, heads, D] float32 tensor that lie
// outside [cu[0]*n, cu[N]*n) (the rows no sequence covers).
struct ZeroOutsideArgs {
  float *p; int64_t st, sh;
  const void *cu; int cu_is64;
  int64_t T; int N, n, heads, D;
};
hipError_t launch_zero_outside(const ZeroOutsideArgs &a, hipStream_t stream);

// Gradient with respect to raw rows from the one with respect to their L2-normalised
// versions, in place (rows = R * heads rows of a [R, heads, K] tensor).
struct NormGradArgs {
  const void *x; int64_t x_st, x_sh;
  float *g; int64_t g_st, g_sh;
  int64_t rows; int heads;
};
hipError_t launch_l2norm_grad(const NormGradArgs &a, int dtype, int K, hipStream_t stream);
// the norm factors of the rows of x into g (dense [rows, heads]: g_st = heads, g_sh = 1)
hipError_t launch_row_norm(const NormGradArgs &a, int dtype, int K, hipStream_t stream);

// Element types of the front end's conversion kernels.
enum ElType { EL_F32 = 0, EL_BF16 = 1, EL_F16 = 2 };

// Gates in the prefill kernels' form: g_log [T, Hv] = ln(alpha) (0 without
// alpha), beta32 [T*n, Hv] (1 without beta); both contiguous float32.
struct GateArgs {
  const void *alpha; int alpha_dtype; int64_t a_st, a_sh;  // [T, Hv] or null
  const void *beta; int beta_dtype; int64_t b_st, b_sh;    // [T*n, Hv] or null
  int64_t T; int n, Hv;
  float *g_log, *beta32;
};
hipError_t launch_gates(const GateArgs &a, hipStream_t stream);

// State layout change of `mats` contiguous K x V states: V-major (state_dtype)
// to K-major float32, or K-major float32 to V-major (state_dtype).  K and V
// multiples of 64.
struct StateArgs {
  const void *src; void *dst;
  int64_t mats; int K, V;
  int state_dtype;
};
hipError_t launch_state_transpose(const StateArgs &a, bool to_k_major, hipStream_t stream);

// float16 <-> bfloat16 copy of a [R, H, D] tensor whose rows (st) and heads (sh)
// may be strided on the float16 side; the bfloat16 side is contiguous.
struct HalfCopyArgs {
  const void *src; void *dst;
  int64_t R; int H, D;
  int64_t st, sh;
};
hipError_t launch_half_copy(const HalfCopyArgs &a, bool to_bf16, hipStream_t stream);
hipError_t launch_fill(int32_t *p, int64_t n, int32_t v, hipStream_t stream);

// Opt-in checks of the data-dependent arguments (GDP_DEBUG_VALIDATE=1): the
// bits GDP_DBG_* of include/gdp.h are ORed into one device-global word per device.
struct ValidateArgs {
  const void *cu; int cu_is64; int64_t N, T;                    // cu_seqlens [N+1], or null
  const void *slots; int slots_is64; int64_t nslots_given, num_slots;  // state indices, or null
  uint32_t *word;                                               // set by launch_validate
};
hipError_t launch_validate(ValidateArgs a, hipStream_t stream);
// device address of the static scratch array of the current device (the
// workspace of gdp_chunk_prefill_noalloc), looked up once per device
hipError_t noalloc_scratch(void **out);
// device address of the current device's word
hipError_t debug_word_ptr(uint32_t **out);
hipError_t launch_combine(const CombineArgs &a, int K, int V, hipStream_t stream);
// launches the fused kernel regardless of the chain count (bf16 only)
hipError_t launch_fused_prefill(const PrefillArgs &a, int K, int V, hipStream_t stream);

bool decode_supported(int K, int V);
hipError_t launch_decode(const DecodeArgs &a, int dtype, int K, int V, hipStream_t stream);

}  // namespace gdp
