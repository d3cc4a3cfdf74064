/*
 * gdp.h -- C ABI of the MI355X (gfx950) chunked Gated DeltaProduct prefill library.
 *
 * The operation (FlashInfer docs, "flashinfer.gdp_prefill.chunk_gated_delta_product",
 * the recurrence display): for every sequence and every state head, per real
 * token t the K x V state S is first scaled by alpha_t = exp(g_log_t); then for
 * j = 0..n-1 on sub-token row r = t*n + j
 *     v_new_r = beta_r * (v_r - S^T k_r),   S += k_r v_new_r^T;
 * and after the last update o_t = scale * S^T q_t.  n = 1 is the gated delta rule.
 * The argument list follows the Megatron Core API docs, core.ssm.ops.gdp.chunk,
 * chunk_gated_delta_product_varlen (parameter list and the graph-capture note
 * after it), with outputs, workspace and stream appended.
 *
 * Conventions shared by every entry point
 *   - Every data pointer is DEVICE memory owned by the caller.  The library
 *     never allocates, frees or synchronises, never reads device memory on
 *     the host, and launches only on the stream it is given (a hipStream_t
 *     passed as void*; NULL is the default stream).  A call is therefore
 *     capturable into a HIP graph.
 *   - Return value: GDP_OK (0) or a negative gdp_status.  No exception ever
 *     crosses the ABI.  On failure gdp_last_error() returns a message (per
 *     calling thread).  Errors are detected from shapes, dtypes, strides and
 *     pointer ranges only; the contents of cu_seqlens, state_indices and
 *     caller-built descriptors are not checked (that would need a device to
 *     host read).  The kernels clamp what they index with them: sequence
 *     bounds to [0, T], cache slots outside [0, S) and chunk-state rows past
 *     the buffer are skipped, so bad contents give wrong numbers, never an
 *     out-of-bounds access.
 *   - Chunk size is fixed at 64 (Megatron Core page, the two-chunkings
 *     paragraph and the chunk_states description).
 */
#ifndef GDP_H
#define GDP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types of gdp_tensor. */
enum gdp_dtype { GDP_F32 = 0, GDP_BF16 = 1, GDP_I32 = 2, GDP_I64 = 3, GDP_F16 = 4 };

/* Return codes. */
enum gdp_status {
  GDP_OK = 0,
  GDP_EINVAL = -1,       /* bad shape, dtype, stride, n < 1, Hv % Hqk != 0, missing argument */
  GDP_EUNSUPPORTED = -2, /* valid request this build does not serve (head dims, dtype mix) */
  GDP_EALIAS = -3,       /* an output overlaps an input or another output */
  GDP_EWORKSPACE = -4,   /* workspace missing or smaller than gdp_workspace_bytes() */
  GDP_EHIP = -5          /* a HIP launch failed; message from hipGetErrorString */
};

/* A strided view of device memory.  data == NULL means "absent" (None).
 * shape/stride hold ndim valid entries; strides are in ELEMENTS.  The
 * innermost dimension must be contiguous (stride 1). */
typedef struct gdp_tensor {
  void *data;
  int32_t dtype;
  int32_t ndim;
  int64_t shape[4];
  int64_t stride[4];
} gdp_tensor;

/* Chunk descriptors of the two chunkings (Megatron Core page: chunk_indices,
 * chunk_indices_dp, chunk_offsets).  Sequence i of length L_i has
 * ceil(L_i/64) token chunks and ceil(n*L_i/64) expanded chunks.
 *   chunk_indices    [nt_cap, 2]   int32 rows (i, c), sequence-major, c ascending,
 *                                  rows past the real count hold (-1, -1)
 *   chunk_indices_dp [ntdp_cap, 2] the same for the expanded stream
 *   chunk_offsets    [N+1]         int32 exclusive prefix sums of token-chunk counts
 *   chunk_offsets_dp [N+1]         the same for expanded-chunk counts
 * All four arrays are device memory owned by the caller. */
typedef struct gdp_descriptors {
  int32_t *chunk_indices;
  int32_t *chunk_indices_dp;
  int32_t *chunk_offsets;
  int32_t *chunk_offsets_dp;
  int64_t nt_cap;
  int64_t ntdp_cap;
} gdp_descriptors;

/* Host-only.  Capacities that bound the descriptor row counts for any
 * cu_seqlens with N sequences and T real tokens:
 *   nt_cap = floor((T + 63 N) / 64),  ntdp_cap = floor((n T + 63 N) / 64).
 * Padding to these makes every grid depend on (T, N, n) only (Megatron Core
 * page, the graph-capture note).  Returns GDP_EINVAL for negative sizes or n < 1. */
int gdp_descriptor_capacity(int64_t T, int64_t N, int32_t num_householder,
                            int64_t *nt_cap, int64_t *ntdp_cap);

/* Device.  Builds the descriptors of cu_seqlens ([N+1], int32 or int64,
 * device, contiguous) into out->*, padded to out->nt_cap / out->ntdp_cap, with
 * one kernel launch on `stream`.  T is the caller's real-token count; the
 * capacities must be at least gdp_descriptor_capacity(T, N, n) (GDP_EINVAL
 * otherwise).  Capturable; "built once per step" in the Megatron Core
 * page's words. */
int gdp_build_descriptors(const gdp_tensor *cu_seqlens, int32_t num_householder, int64_t T,
                          const gdp_descriptors *out, void *stream);

/* Host-only.  Workspace bytes gdp_chunk_prefill needs for T real tokens, N
 * sequences, n Householder rows per token, Hv state heads and input dtype
 * (GDP_BF16 or GDP_F32): the per-chunk WY matrices (64 x 64 per expanded
 * chunk and state head, at the input precision) or the buffers of the
 * segmented (chunk-parallel) path for few long sequences (bf16, K == V: per
 * segment of at least 256 tokens an f32 K x K map and two K x V states per
 * head), whichever is larger; plus room for the descriptors when the caller
 * passes none; plus an int32 work order of N x Hv entries when N x Hv > 256 and
 * N <= 4096; plus an int32 chunk counter per (sequence, state head) when
 * Hv > Hqk (the fused kernel paces the state heads that share a q/k head).
 * The size depends on host-known shapes only, so one allocation serves every
 * call of a captured batch shape, as the fixed-length descriptors do (Megatron
 * Core page, core.ssm.ops.gdp.chunk, the note on the descriptor arguments and
 * graph capture).  Returns 0 for invalid sizes or dtypes. */
size_t gdp_workspace_bytes(int64_t T, int64_t N, int32_t num_householder, int32_t Hqk,
                           int32_t Hv, int32_t K, int32_t V, int32_t dtype);

/* Device.  The chunked GDP prefill forward pass.
 *
 * Inputs (T real tokens, N sequences, n = num_householder, Hqk q/k heads,
 * Hv state heads = v/g/beta/output heads, head dims K and V):
 *   q            [T, Hqk, K]      bf16 or f32; rows may be strided
 *   k            [T*n, Hk, K]     same dtype as q; rows t*n..t*n+n-1 belong to token t;
 *                                 Hk = Hqk, or Hk = Hv (one k head per state head;
 *                                 FlashInfer page, k: num_k_heads equals the q or the
 *                                 v head count).  State head h reads q head
 *                                 h / (Hv / Hqk) and k head h / (Hv / Hk)
 *   v            [T*n, Hv, V]     same dtype as q
 *   g_log        [T, Hv]          f32 log decays (alpha_t = exp(g_log_t))
 *   beta         [T*n, Hv]        f32
 *   cu_seqlens   [N+1]            int32 or int64, contiguous, required
 *   scale        readout scale; 0 means K^-1/2 (FlashInfer page, scale)
 *   initial_state [N, Hv, K, V]   f32 contiguous, or data == NULL for zeros
 *   output_final_state            write final_state when nonzero
 *   use_qk_l2norm                 divide every q row and k sub-token row by
 *                                 sqrt(sum x^2 + 1e-6) inside the kernel
 *   state_cache  [S, Hv, K, V]    f32 contiguous, or NULL; when given, the final
 *                                 state of sequence i is written in place at
 *                                 slot state_indices[i]; -1 writes nothing
 *   state_indices [N]             int32 or int64; required with state_cache
 *   return_chunk_states           write chunk_states when nonzero
 * Outputs (caller-allocated device memory):
 *   o            [T, Hv, V]       same dtype as q; rows may be strided
 *   final_state  [N, Hv, K, V]    f32 contiguous; required iff output_final_state
 *   chunk_states [R, Hv, K, V]    f32 contiguous, R >= gdp_descriptor_capacity's
 *                                 nt_cap; row chunk_offsets[i] + c is the state of
 *                                 sequence i entering its token chunk c, i.e. after
 *                                 its first 64*c tokens (Megatron Core page,
 *                                 return_chunk_states).  Rows past the real count
 *                                 are left untouched.
 *   desc         caller-built descriptors (gdp_build_descriptors) or NULL; when
 *                NULL they are built into the workspace on `stream`.  Their
 *                capacities must be at least gdp_descriptor_capacity(T, N, n)
 *                (GDP_EINVAL otherwise: descriptors built for a smaller T or a
 *                different n would leave chunks out of the grids)
 *   workspace    device scratch, 256-byte aligned, of workspace_bytes >=
 *                gdp_workspace_bytes(...) (required: it holds the per-chunk WY
 *                matrices between the two kernels of the call)
 * Ownership/aliasing: no output may overlap an input or another output; in
 * particular final_state must not alias initial_state, because one sequence's
 * state is split over several workgroups (FlashInfer page, output_state).
 * Supported today: K, V in {64, 128}; f32 inputs need K = 64 (GDP_EUNSUPPORTED
 * otherwise).  Calls that overlap on one stream are ordered; calls on
 * different streams sharing an output race. */
int gdp_chunk_prefill(const gdp_tensor *q, const gdp_tensor *k, const gdp_tensor *v,
                      const gdp_tensor *g_log, const gdp_tensor *beta,
                      int32_t num_householder, const gdp_tensor *cu_seqlens, float scale,
                      const gdp_tensor *initial_state, int32_t output_final_state,
                      int32_t use_qk_l2norm, const gdp_tensor *state_cache,
                      const gdp_tensor *state_indices, int32_t return_chunk_states,
                      const gdp_tensor *o, const gdp_tensor *final_state,
                      const gdp_tensor *chunk_states, const gdp_descriptors *desc,
                      void *workspace, size_t workspace_bytes, void *stream);

/* Size of the static scratch array of gdp_chunk_prefill_noalloc, per GPU. */
#define GDP_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* Device.  gdp_chunk_prefill without a workspace argument, for callers that
 * cannot allocate device memory: code under graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Arguments, results and errors are
 * those of gdp_chunk_prefill; the workspace is a file-scope device array of
 * GDP_NOALLOC_SCRATCH_BYTES (64 MiB) that every GPU the library runs on holds
 * until the process ends.  The call allocates nothing.  A call whose workspace
 * need exceeds the array returns GDP_EWORKSPACE with the size it needs.  The
 * fused path needs only the descriptors (when desc is NULL), the work order and
 * the pacing counters: 16 bytes per chunk row plus 8 per (sequence, state
 * head), under 1 MiB up to tens of millions of tokens; the split path's WY
 * matrices take 8 KiB (bf16) or 16 KiB (f32) per expanded chunk and state head,
 * and the segmented path 12 K V bytes per segment and state head.  All calls on one GPU share its array:
 * calls that overlap on one GPU (for instance on two streams) race; calls on
 * one stream are ordered.  No call depends on what an earlier one left in the
 * array. */
int gdp_chunk_prefill_noalloc(const gdp_tensor *q, const gdp_tensor *k, const gdp_tensor *v,
                              const gdp_tensor *g_log, const gdp_tensor *beta, int32_t num_householder,
                              const gdp_tensor *cu_seqlens, float scale, const gdp_tensor *initial_state,
                              int32_t output_final_state, int32_t use_qk_l2norm,
                              const gdp_tensor *state_cache, const gdp_tensor *state_indices,
                              int32_t return_chunk_states, const gdp_tensor *o,
                              const gdp_tensor *final_state, const gdp_tensor *chunk_states,
                              const gdp_descriptors *desc, void *stream);

/* Device.  The single-token recurrent decode step on the state cache, in place.
 *
 * The decode step of the blog page "Attention Cache and Sequence Parallelism"
 * (section "GDN: fixed state instead of a per-token cache": Sbar = lambda S,
 * vhat = Sbar^T k, e = beta (v - vhat), S = Sbar + k e^T, r = q^T S), with the
 * n Householder rows per token of the FlashInfer recurrence display and the
 * slot convention of the Megatron Core page (state / state_indices).  For
 * every entry i and state head h with slot = state_indices[i] in [0, S):
 *     S = state_cache[slot, h];  S *= exp(g_log[i, h]);
 *     for j = 0..n-1, r = i*n + j:  e = beta[r,h] (v[r,h] - S^T k[r]);  S += k[r] e^T;
 *     o[i, h] = scale * S^T q[i];  state_cache[slot, h] = S.
 * Entries whose index is negative (padding, -1) or past the cache get a zero
 * output row and leave the cache untouched.
 *   q [N, Hqk, K], k [N*n, Hk, K], v [N*n, Hv, V]    bf16 or f32 (one dtype); rows may be strided;
 *                                                    Hk = Hqk or Hv, as for gdp_chunk_prefill
 *   g_log [N, Hv], beta [N*n, Hv]                    f32 (log decays; alpha = exp(g_log))
 *   scale                                            0 means K^-1/2
 *   use_qk_l2norm                                    as for gdp_chunk_prefill
 *   state_cache [S, Hv, K, V]                        f32 contiguous, K-major states, read and written
 *   state_indices [N]                                int32 or int64
 *   o [N, Hv, V]                                     q's dtype, written
 * Two entries naming the same slot race (caller error; not checked: that needs
 * a device read).  o and the cache may not overlap the inputs or each other
 * (GDP_EALIAS).  K, V in {64, 128}.  One kernel launch on `stream`; nothing is
 * allocated, so the call is capturable. */
int gdp_recurrent_decode(const gdp_tensor *q, const gdp_tensor *k, const gdp_tensor *v,
                         const gdp_tensor *g_log, const gdp_tensor *beta, int32_t num_householder,
                         float scale, int32_t use_qk_l2norm, const gdp_tensor *state_cache,
                         const gdp_tensor *state_indices, const gdp_tensor *o, void *stream);

/* Host-only.  Workspace bytes gdp_chunk_prefill_backward needs, the larger of
 * its two paths' needs.  The chunked path: the descriptors, then per expanded
 * 64-row chunk and state head the float32 entering state and end-of-chunk state
 * gradient (2 x ntdp_cap x Hv x K x V floats) and a prep bundle (T^T and the
 * decayed scores in bfloat16, per-row factors).  The recurrent path: the
 * descriptors, the float32 state entering every token chunk (nt_cap x Hv x K x V),
 * an output buffer of the forward pass it reruns, the float32 L2-norm factors of
 * the q and k rows (T x Hqk and T*n x Hv at most), and that pass's workspace
 * (gdp_workspace_bytes).  Returns 0 for invalid sizes or dtypes. */
size_t gdp_backward_workspace_bytes(int64_t T, int64_t N, int32_t num_householder, int32_t Hqk, int32_t Hv,
                                    int32_t K, int32_t V, int32_t dtype);

/* Device.  Gradients of the prefill: with L = <o, d_o> + <final_state,
 * d_final_state>, writes dL/dq, dL/dk, dL/dv, dL/dg_log, dL/dbeta and (when
 * d_initial_state is given) dL/dinitial_state, for the same inputs and
 * conventions as gdp_chunk_prefill (no state cache, no chunk states).
 *
 * The pages give no backward formulas (the blog page "Attention Cache and
 * Sequence Parallelism", section "GDN: pass the state, not the KV", notes only
 * that the dependencies run in reverse); these are the gradients of the
 * recurrence itself, by reverse-mode differentiation.  Two paths give them:
 *   chunked (bfloat16 inputs, q/k/v/d_o 16-byte aligned with row and head
 *   strides multiples of 8): per
 *   64-row expanded chunk, a prep kernel forms the chunk's WY inverse and decayed
 *   scores, a forward walk stores each chunk's entering state and a reverse walk
 *   each chunk's end-of-chunk state gradient (both float32), and a gradient
 *   kernel forms every gradient of a chunk with matrix-core products;
 *   recurrent (everything else, or GDP_BACKWARD_PATH=recurrent in the
 *   environment): reruns the forward pass to obtain the state entering every
 *   64-token chunk, then walks each chain backwards token by token, recomputing
 *   the states in between.
 *   d_o            [T, Hv, V]      q's dtype, rows may be strided
 *   d_final_state  [N, Hv, K, V]   float32 contiguous, or data == NULL (zero)
 *   dq [T, Hqk, K], dk [T*n, Hk, K], dg_log [T, Hv], dbeta [T*n, Hv]
 *                                  float32, contiguous: the recurrent path
 *                                  accumulates them with float atomics over state
 *                                  heads and V tiles, so their last bits depend on
 *                                  the order of the adds; the chunked path stores
 *                                  each entry once
 *   dv [T*n, Hv, V]                float32, rows may be strided; the sub-rows no
 *                                  sequence covers (before cu_seqlens[0]*n or from
 *                                  cu_seqlens[N]*n on) are written as zeros, like
 *                                  the other gradients' rows there
 *   d_initial_state [N, Hv, K, V]  float32 contiguous, or data == NULL
 *   workspace      at least gdp_backward_workspace_bytes(...), 256-byte aligned
 * No gradient may overlap an input or another gradient (GDP_EALIAS).  K, V in
 * {64, 128}, num_householder <= 5 (GDP_EUNSUPPORTED otherwise).  Everything
 * runs on `stream` with no allocation and no host read of device memory. */
int gdp_chunk_prefill_backward(const gdp_tensor *q, const gdp_tensor *k, const gdp_tensor *v,
                               const gdp_tensor *g_log, const gdp_tensor *beta, int32_t num_householder,
                               const gdp_tensor *cu_seqlens, float scale, const gdp_tensor *initial_state,
                               int32_t use_qk_l2norm, const gdp_tensor *d_o, const gdp_tensor *d_final_state,
                               const gdp_tensor *dq, const gdp_tensor *dk, const gdp_tensor *dv,
                               const gdp_tensor *dg_log, const gdp_tensor *dbeta,
                               const gdp_tensor *d_initial_state, void *workspace, size_t workspace_bytes,
                               void *stream);

/* Host-only.  Workspace bytes gdp_chunk_gated_delta_product needs: the gates
 * restated as float32 log decays and betas (4 (1 + n) T Hv bytes; the betas are
 * used only when they are not float32 already), a float32
 * K-major copy of each state it converts (4 N Hv d^2 bytes each, when an
 * initial state is given and when the final state is requested), and the
 * workspace of the prefill it runs (gdp_workspace_bytes); with float16 inputs
 * also bfloat16 copies of q, k, v and the output.  dtype is q's (GDP_BF16 or
 * GDP_F16).  Returns 0 for invalid sizes or dtypes. */
size_t gdp_fi_workspace_bytes(int64_t T, int64_t N, int32_t num_householder, int32_t Hq, int32_t Hv,
                              int32_t head_size, int32_t dtype, int32_t with_initial_state,
                              int32_t output_final_state);

/* Device.  The chunked GDP prefill in the FlashInfer convention (FlashInfer docs,
 * "flashinfer.gdp_prefill.chunk_gated_delta_product": its recurrence display and
 * parameter list, in the same order, with workspace and stream appended).
 * It computes what gdp_chunk_prefill computes; only the operands are stated
 * differently:
 *   q  [T, Hq, d], k [T*n, Hk, d] (Hk = Hq or Hv), v [T*n, Hv, d]   bfloat16 or
 *                  float16, rows may be strided; Hv a multiple of Hq (more q than v
 *                  heads is GDP_EUNSUPPORTED), d in {64, 128}.  float16 inputs
 *                  are copied to bfloat16 operands in the workspace (row and head
 *                  strides must be multiples of 8) and the output, formed in
 *                  bfloat16, is converted to float16
 *   g    [T, Hv]   the decay alpha itself (in (0, 1]), float32, bfloat16 or float16,
 *                  or data == NULL for no decay (alpha = 1)
 *   beta [T*n, Hv] float32 (read in place, strides honoured) or q's dtype, or
 *                  data == NULL for all ones
 *   scale          0 means d^-1/2
 *   initial_state  [N, Hv, d, d] V-major (entry [v][k]), float32 or bfloat16,
 *                  contiguous, or data == NULL for zero states
 *   output_final_state  write output_state when nonzero
 *   cu_seqlens     [N+1] int32 or int64, required
 *   use_qk_l2norm_in_kernel   as gdp_chunk_prefill's use_qk_l2norm
 *   output         [T, Hv, d] q's dtype, written
 *   output_state   [N, Hv, d, d] V-major, float32 or bfloat16, contiguous; required
 *                  iff output_final_state; it may not overlap initial_state or any
 *                  input (GDP_EALIAS; FlashInfer page, output_state)
 *   workspace      device scratch of at least gdp_fi_workspace_bytes(...), 256-byte
 *                  aligned
 * Everything runs on `stream` (conversion kernels, then the prefill), with no
 * host read of device memory and no allocation, so the call is capturable. */
int gdp_chunk_gated_delta_product(const gdp_tensor *q, const gdp_tensor *k, const gdp_tensor *v,
                                  const gdp_tensor *g, const gdp_tensor *beta, int32_t num_householder,
                                  float scale, const gdp_tensor *initial_state, int32_t output_final_state,
                                  const gdp_tensor *cu_seqlens, int32_t use_qk_l2norm_in_kernel,
                                  const gdp_tensor *output, const gdp_tensor *output_state, void *workspace,
                                  size_t workspace_bytes, void *stream);

/* Debug validation of the data-dependent arguments.  These are not checked by
 * default, because checking them needs a read of device data.  A bad value stays
 * in bounds (every kernel clamps sequence ranges to [0, T] and skips slots
 * outside the cache), but the results are then undefined.  With the environment
 * variable GDP_DEBUG_VALIDATE=1, gdp_chunk_prefill (and the entries built on it)
 * and gdp_recurrent_decode first launch a check on their stream.  The check ORs
 * these bits into a word kept per device:
 *   GDP_DBG_CU    cu_seqlens decreases somewhere, or an entry lies outside [0, T]
 *                 (Megatron Core page, chunk_gated_delta_product_varlen: the
 *                 cumulative sequence boundaries)
 *   GDP_DBG_SLOT  a state index below -1 or not below the number of cache slots
 *   GDP_DBG_DUP   two sequences (decode entries) share a non-negative state
 *                 index (same page, the state-cache arguments: -1 means no write)
 * The duplicate check is quadratic in the number of sequences: it is a
 * debugging aid, not for production steps. */
enum gdp_debug_bits { GDP_DBG_CU = 1, GDP_DBG_SLOT = 2, GDP_DBG_DUP = 4 };

/* Host-side: reads the current device's debug word into *word (host memory)
 * after the work queued on `stream` so far, then, if clear != 0, queues its
 * reset to 0 on `stream`.  Synchronises `stream`.  GDP_EINVAL if word is NULL,
 * GDP_EHIP on a runtime failure. */
int gdp_debug_status(uint32_t *word, int32_t clear, void *stream);

/* Message of the last failed call on this thread ("" if none).  A request the
 * library does not serve is declined with GDP_EUNSUPPORTED and its reason left
 * here rather than aborting the caller, the way the FlashInfer page
 * (flashinfer.gdp_prefill.chunk_gated_delta_product, requirements note) has an
 * engine decline a graph it cannot serve and log why. */
const char *gdp_last_error(void);

/* Library version string.  Informational; no passage of the pages defines it. */
const char *gdp_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDP_H */
