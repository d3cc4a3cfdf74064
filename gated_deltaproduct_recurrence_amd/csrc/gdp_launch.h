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
  void *o; int64_t o_st, o_sh;
};

enum InDtype { IN_F32 = 0, IN_BF16 = 1 };

// Arguments of the single-token decode step (strides in elements).
struct DecodeArgs {
  const void *q; int64_t q_st, q_sh;      // [N, Hqk, K]
  const void *k; int64_t k_st, k_sh;      // [N*n, Hqk, K]
  const void *v; int64_t v_st, v_sh;      // [N*n, Hv, V]
  const float *g; int64_t g_st, g_sh;     // [N, Hv]
  const float *beta; int64_t b_st, b_sh;  // [N*n, Hv]
  int N, n, Hqk, Hv;
  float scale;
  int l2norm;
  float *cache; int64_t num_slots;        // [num_slots, Hv, K, V], read and written in place
  const void *slots; int slots_is64;      // [N]
  void *o; int64_t o_st, o_sh;            // [N, Hv, V]
};

// Kernel path: AUTO picks the fused single kernel for bf16 when there are at
// least 256 (sequence, state head) chains, else the WY kernel + scan kernel pair.
enum Path { PATH_AUTO = 0, PATH_FUSED = 1, PATH_SPLIT = 2 };

bool prefill_supported(int dtype, int K, int V);
// Bytes of the WY-matrix buffer for `rows` expanded chunks and Hv heads.
size_t wy_buffer_bytes(int dtype, int64_t rows, int64_t Hv);
hipError_t launch_prefill(const PrefillArgs &a, int dtype, int K, int V, int path, hipStream_t stream);
hipError_t launch_descriptors(const DescArgs &a, hipStream_t stream);
bool decode_supported(int K, int V);
hipError_t launch_decode(const DecodeArgs &a, int dtype, int K, int V, hipStream_t stream);

}  // namespace gdp
