// gdp_api.cpp -- C ABI of the chunked Gated DeltaProduct prefill library
// (declared in include/gdp.h).  Host-side validation reads shapes, dtypes,
// strides and pointer ranges only -- never device memory -- then launches on
// the caller's stream.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include "gdp.h"
#include "gdp_launch.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

bool present(const gdp_tensor *t) { return t != nullptr && t->data != nullptr; }

// GDP_DEBUG_VALIDATE=1: launch the device checks of cu_seqlens and the state indices
bool debug_validate() {
  const char *s = std::getenv("GDP_DEBUG_VALIDATE");
  return s != nullptr && s[0] == '1' && s[1] == '\0';
}

int elem_size(int32_t dt) {
  switch (dt) {
    case GDP_F32: return 4;
    case GDP_BF16: return 2;
    case GDP_I32: return 4;
    case GDP_I64: return 8;
    case GDP_F16: return 2;
    default: return 0;
  }
}

// Checks ndim, the exact shape and that the innermost stride is 1.
int check_shape(const gdp_tensor *t, const char *name, int ndim, const int64_t *shape) {
  if (t->ndim != ndim) return fail(GDP_EINVAL, "%s: expected %d dims, got %d", name, ndim, t->ndim);
  for (int d = 0; d < ndim; ++d)
    if (shape[d] >= 0 && t->shape[d] != shape[d])
      return fail(GDP_EINVAL, "%s: dim %d is %lld, expected %lld", name, d, (long long)t->shape[d],
                  (long long)shape[d]);
  if (ndim > 0 && t->stride[ndim - 1] != 1)
    return fail(GDP_EINVAL, "%s: innermost dimension must be contiguous", name);
  return GDP_OK;
}

bool contiguous(const gdp_tensor *t) {
  int64_t expect = 1;
  for (int d = t->ndim - 1; d >= 0; --d) {
    if (t->shape[d] != 1 && t->stride[d] != expect) return false;
    expect *= t->shape[d];
  }
  return true;
}

// [lo, hi) byte range a tensor may touch (strides are non-negative here).
struct Range { uintptr_t lo, hi; const char *name; };

Range range_of(const gdp_tensor *t, const char *name) {
  Range r{0, 0, name};
  if (!present(t)) return r;
  int64_t last = 0;
  for (int d = 0; d < t->ndim; ++d) {
    if (t->shape[d] == 0) return r;
    last += (t->shape[d] - 1) * t->stride[d];
  }
  r.lo = (uintptr_t)t->data;
  r.hi = r.lo + (uintptr_t)((last + 1) * elem_size(t->dtype));
  return r;
}

bool overlap(const Range &a, const Range &b) { return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi; }

bool nonneg_strides(const gdp_tensor *t) {
  for (int d = 0; d < t->ndim; ++d)
    if (t->stride[d] < 0) return false;
  return true;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t desc_bytes(int64_t N, int64_t nt_cap, int64_t ntdp_cap) {
  return align256((size_t)nt_cap * 8) + align256((size_t)ntdp_cap * 8) + 2 * align256((size_t)(N + 1) * 4);
}

// Segmented prefill plan (host-known sizes only, so the call stays capturable):
// bf16 inputs, K == V, fewer than 256 (sequence, state head) chains and
// sequences long enough to cut into segments of whole 64-token chunks such that
// the segment chains fill the 256 compute units.
struct SegPlan {
  bool use = false;
  int64_t Lseg = 0, ns_cap = 0;
};

SegPlan seg_plan(int64_t T, int64_t N, int64_t Hv, int64_t K, int64_t V, int32_t dtype, int path) {
  SegPlan p;
  if (dtype != GDP_BF16 || K != V || !(K == 64 || K == 128) || N < 1 || T < 0) return p;
  if (path == gdp::PATH_FUSED || path == gdp::PATH_SPLIT) return p;
  if (path != gdp::PATH_SEGMENTED && N * Hv >= 256) return p;
  const int64_t avg = (T + N - 1) / N;
  const int64_t target = std::max<int64_t>(2, 256 / (N * Hv));  // segments per sequence
  int64_t L = (avg + target - 1) / target;
  L = std::max<int64_t>(256, (L + 63) / 64 * 64);
  if (path != gdp::PATH_SEGMENTED && avg < 2 * L) return p;
  p.use = true;
  p.Lseg = L;
  p.ns_cap = (T + (L - 1) * N) / L;
  return p;
}

size_t seg_bytes(const SegPlan &p, int64_t N, int64_t Hv, int64_t K, int64_t V) {
  if (!p.use) return 0;
  return align256((size_t)(p.ns_cap + 1) * 4) + align256((size_t)(N + 1) * 4) + align256((size_t)p.ns_cap * 4) +
         align256((size_t)p.ns_cap * Hv * K * K * 4) + 2 * align256((size_t)p.ns_cap * Hv * K * V * 4);
}

// the fused kernel's longest-first chain order: for grids of more than one round
// of workgroups (one per CU) and at most ORDER_MAX_SEQ sequences; the workspace
// reserves it whenever the grid qualifies, the call builds it only when the
// fused kernel runs
bool order_grid(int64_t N, int64_t Hv) { return N * Hv > 256 && N <= gdp::ORDER_MAX_SEQ; }
size_t order_bytes(int64_t N, int64_t Hv) { return order_grid(N, Hv) ? align256((size_t)N * Hv * 4) : 0; }
// the fused kernel's chunk progress per chain (pacing of state heads that share
// a q/k head)
size_t progress_bytes(int64_t N, int64_t Hv, int64_t Hqk) { return Hv > Hqk ? align256((size_t)N * Hv * 4) : 0; }

int env_path() {
  // GDP_PREFILL_PATH=fused|split|segmented overrides the automatic kernel
  // choice (tests use it to run every path on the same inputs)
  if (const char *env = std::getenv("GDP_PREFILL_PATH")) {
    if (std::strcmp(env, "fused") == 0) return gdp::PATH_FUSED;
    if (std::strcmp(env, "split") == 0) return gdp::PATH_SPLIT;
    if (std::strcmp(env, "segmented") == 0) return gdp::PATH_SEGMENTED;
  }
  return gdp::PATH_AUTO;
}

}  // namespace

extern "C" {

const char *gdp_last_error(void) { return g_last_error.c_str(); }

namespace {
int el_type(int32_t dt) { return dt == GDP_F32 ? gdp::EL_F32 : (dt == GDP_BF16 ? gdp::EL_BF16 : gdp::EL_F16); }

// Workspace of the FlashInfer-convention front end, in order: the gates in the
// prefill kernels' form, the K-major initial and final states, then the
// prefill's own workspace.
struct FiLayout {
  size_t glog = 0, beta = 0, s0 = 0, fin = 0, q = 0, k = 0, v = 0, o = 0, inner = 0, total = 0;
};
// float16 inputs add bfloat16 copies of q, k, v and the output (k sized for Hk = Hv)
static FiLayout fi_layout(int64_t T, int64_t N, int32_t n, int32_t Hq, int32_t Hv, int32_t d, int32_t dtype,
                   bool with_initial, bool with_final) {
  FiLayout L;
  const size_t st = align256((size_t)N * Hv * d * d * 4);
  const bool half = dtype == GDP_F16;
  L.glog = 0;
  L.beta = L.glog + align256((size_t)T * Hv * 4);
  L.s0 = L.beta + align256((size_t)T * n * Hv * 4);
  L.fin = L.s0 + (with_initial ? st : 0);
  L.q = L.fin + (with_final ? st : 0);
  L.k = L.q + (half ? align256((size_t)T * Hq * d * 2) : 0);
  L.v = L.k + (half ? align256((size_t)T * n * Hv * d * 2) : 0);
  L.o = L.v + (half ? align256((size_t)T * n * Hv * d * 2) : 0);
  L.inner = L.o + (half ? align256((size_t)T * Hv * d * 2) : 0);
  const size_t ws = gdp_workspace_bytes(T, N, n, Hq, Hv, d, d, GDP_BF16);
  L.total = ws ? L.inner + ws : 0;
  return L;
}
}  // namespace

size_t gdp_fi_workspace_bytes(int64_t T, int64_t N, int32_t n, int32_t Hq, int32_t Hv, int32_t d, int32_t dtype,
                              int32_t with_initial_state, int32_t output_final_state) {
  if (T < 0 || N < 0 || n < 1 || Hq < 1 || Hv < 1 || d < 1) return 0;
  if (dtype != GDP_BF16 && dtype != GDP_F16) return 0;
  return fi_layout(T, N, n, Hq, Hv, d, dtype, with_initial_state != 0, output_final_state != 0).total;
}

int gdp_chunk_gated_delta_product(const gdp_tensor *q, const gdp_tensor *k, const gdp_tensor *v,
                                  const gdp_tensor *g, const gdp_tensor *beta, int32_t n, float scale,
                                  const gdp_tensor *initial_state, int32_t output_final_state,
                                  const gdp_tensor *cu_seqlens, int32_t use_qk_l2norm_in_kernel,
                                  const gdp_tensor *output, const gdp_tensor *output_state, void *workspace,
                                  size_t workspace_bytes, void *stream) {
  g_last_error.clear();
  if (!present(q) || !present(k) || !present(v) || !present(output))
    return fail(GDP_EINVAL, "q, k, v and output are required");
  if (!present(cu_seqlens)) return fail(GDP_EINVAL, "cu_seqlens is required (varlen input only)");
  if (n < 1) return fail(GDP_EINVAL, "num_householder must be >= 1, got %d", n);
  if (q->ndim != 3 || k->ndim != 3 || v->ndim != 3 || cu_seqlens->ndim != 1)
    return fail(GDP_EINVAL, "q, k, v must be 3-d and cu_seqlens 1-d");
  const int64_t T = q->shape[0], Hq = q->shape[1], d = q->shape[2], Hv = v->shape[1];
  const int64_t N = cu_seqlens->shape[0] - 1;
  if (N < 0) return fail(GDP_EINVAL, "cu_seqlens must have N+1 >= 1 entries");
  if (Hq < 1 || Hv < 1) return fail(GDP_EINVAL, "head counts must be positive");
  if (Hq > Hv) return fail(GDP_EUNSUPPORTED, "more q heads than v heads is not served (Hq %lld, Hv %lld)",
                           (long long)Hq, (long long)Hv);
  if (v->shape[2] != d) return fail(GDP_EINVAL, "q, k and v share one head size");
  if (q->dtype != GDP_BF16 && q->dtype != GDP_F16) return fail(GDP_EUNSUPPORTED, "q, k and v must be bfloat16 or float16");
  if (d != 64 && d != 128) return fail(GDP_EUNSUPPORTED, "head size must be 64 or 128");
  int rc;
  const int64_t Hk = k->shape[1];
  if (Hk != Hq && Hk != Hv) return fail(GDP_EINVAL, "k must have Hq or Hv heads, got %lld", (long long)Hk);
  if (Hv % Hq != 0) return fail(GDP_EINVAL, "Hv (%lld) must be a multiple of Hq (%lld)", (long long)Hv, (long long)Hq);
  if (k->dtype != q->dtype || v->dtype != q->dtype || output->dtype != q->dtype)
    return fail(GDP_EUNSUPPORTED, "q, k, v and output must share one dtype");
  const int64_t sk[3] = {T * n, Hk, d}, sv[3] = {T * n, Hv, d}, so[3] = {T, Hv, d};
  if ((rc = check_shape(k, "k", 3, sk)) || (rc = check_shape(v, "v", 3, sv)) || (rc = check_shape(output, "output", 3, so)))
    return rc;
  if (q->dtype == GDP_F16 &&
      ((q->stride[0] | q->stride[1] | k->stride[0] | k->stride[1] | v->stride[0] | v->stride[1] | output->stride[0] |
        output->stride[1]) & 7))
    return fail(GDP_EUNSUPPORTED, "float16 q/k/v/output need row and head strides that are multiples of 8");
  const int64_t sg[2] = {T, Hv}, sb[2] = {T * n, Hv}, sst[4] = {N, Hv, d, d};
  if (present(g)) {
    if ((rc = check_shape(g, "g", 2, sg))) return rc;
    if (g->dtype != GDP_F32 && g->dtype != GDP_BF16 && g->dtype != GDP_F16)
      return fail(GDP_EUNSUPPORTED, "g must be float32, bfloat16 or float16");
    if (!nonneg_strides(g)) return fail(GDP_EINVAL, "negative strides are not supported");
  }
  if (present(beta)) {
    if ((rc = check_shape(beta, "beta", 2, sb))) return rc;
    if (beta->dtype != GDP_F32 && beta->dtype != q->dtype) return fail(GDP_EUNSUPPORTED, "beta must be float32 or q's dtype");
    if (!nonneg_strides(beta)) return fail(GDP_EINVAL, "negative strides are not supported");
  }
  if (present(initial_state)) {
    if ((rc = check_shape(initial_state, "initial_state", 4, sst))) return rc;
    if (!contiguous(initial_state)) return fail(GDP_EINVAL, "initial_state must be contiguous");
    if (initial_state->dtype != GDP_F32 && initial_state->dtype != GDP_BF16)
      return fail(GDP_EUNSUPPORTED, "initial_state must be float32 or bfloat16");
  }
  if (output_final_state) {
    if (!present(output_state)) return fail(GDP_EINVAL, "output_state is required when output_final_state is set");
    if ((rc = check_shape(output_state, "output_state", 4, sst))) return rc;
    if (!contiguous(output_state)) return fail(GDP_EINVAL, "output_state must be contiguous");
    if (output_state->dtype != GDP_F32 && output_state->dtype != GDP_BF16)
      return fail(GDP_EUNSUPPORTED, "output_state must be float32 or bfloat16");
    // the page's ownership rule (FlashInfer docs, output_state)
    if (overlap(range_of(output_state, "output_state"), range_of(initial_state, "initial_state")))
      return fail(GDP_EALIAS, "output_state overlaps initial_state");
    for (const Range &ri : {range_of(q, "q"), range_of(k, "k"), range_of(v, "v"), range_of(g, "g"),
                            range_of(beta, "beta"), range_of(cu_seqlens, "cu_seqlens"), range_of(output, "output")})
      if (overlap(range_of(output_state, "output_state"), ri)) return fail(GDP_EALIAS, "output_state overlaps %s", ri.name);
  }
  const FiLayout L = fi_layout(T, N, n, (int32_t)Hq, (int32_t)Hv, (int32_t)d, q->dtype, present(initial_state),
                               output_final_state != 0);
  if (L.total == 0) return fail(GDP_EINVAL, "bad sizes");
  if (!workspace || workspace_bytes < L.total)
    return fail(GDP_EWORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes, L.total);
  if ((uintptr_t)workspace & 255) return fail(GDP_EWORKSPACE, "workspace must be 256-byte aligned");
  char *ws = (char *)workspace;

  hipError_t e;
  gdp::GateArgs ga;
  ga.alpha = present(g) ? g->data : nullptr;
  ga.alpha_dtype = present(g) ? el_type(g->dtype) : 0;
  ga.a_st = present(g) ? g->stride[0] : 0; ga.a_sh = present(g) ? g->stride[1] : 0;
  ga.beta = present(beta) ? beta->data : nullptr;
  ga.beta_dtype = present(beta) ? el_type(beta->dtype) : 0;
  ga.b_st = present(beta) ? beta->stride[0] : 0; ga.b_sh = present(beta) ? beta->stride[1] : 0;
  ga.T = T; ga.n = n; ga.Hv = (int)Hv;
  // a float32 beta is read in place by the prefill; otherwise it is restated
  const bool beta_direct = present(beta) && beta->dtype == GDP_F32;
  ga.g_log = (float *)(ws + L.glog); ga.beta32 = beta_direct ? nullptr : (float *)(ws + L.beta);
  if ((e = gdp::launch_gates(ga, (hipStream_t)stream)) != hipSuccess)
    return fail(GDP_EHIP, "gate launch: %s", hipGetErrorString(e));
  if (present(initial_state)) {
    gdp::StateArgs sa;
    sa.src = initial_state->data; sa.dst = ws + L.s0; sa.mats = N * Hv; sa.K = (int)d; sa.V = (int)d;
    sa.state_dtype = el_type(initial_state->dtype);
    if ((e = gdp::launch_state_transpose(sa, true, (hipStream_t)stream)) != hipSuccess)
      return fail(GDP_EHIP, "state launch: %s", hipGetErrorString(e));
  }
  // float16 inputs: bfloat16 copies of q, k, v (and an output buffer)
  const bool half = q->dtype == GDP_F16;
  gdp_tensor hq_t, hk_t, hv_t, ho_t;
  const gdp_tensor *pq = q, *pk = k, *pv = v, *po = output;
  if (half) {
    struct { const gdp_tensor *t; size_t off; int64_t R, H; gdp_tensor *dst; } cp[3] = {
        {q, L.q, T, Hq, &hq_t}, {k, L.k, T * n, Hk, &hk_t}, {v, L.v, T * n, Hv, &hv_t}};
    for (auto &c : cp) {
      gdp::HalfCopyArgs ha{c.t->data, ws + c.off, c.R, (int)c.H, (int)d, c.t->stride[0], c.t->stride[1]};
      if ((e = gdp::launch_half_copy(ha, true, (hipStream_t)stream)) != hipSuccess)
        return fail(GDP_EHIP, "input copy launch: %s", hipGetErrorString(e));
      *c.dst = gdp_tensor{ws + c.off, GDP_BF16, 3, {c.R, c.H, d}, {c.H * d, d, 1}};
    }
    ho_t = gdp_tensor{ws + L.o, GDP_BF16, 3, {T, Hv, d}, {Hv * d, d, 1}};
    pq = &hq_t; pk = &hk_t; pv = &hv_t; po = &ho_t;
  }
  // the prefill in the Megatron Core convention on the restated operands
  gdp_tensor tg{ws + L.glog, GDP_F32, 2, {T, Hv}, {Hv, 1}};
  const gdp_tensor tb = beta_direct ? *beta : gdp_tensor{ws + L.beta, GDP_F32, 2, {T * n, Hv}, {Hv, 1}};
  gdp_tensor ts0{present(initial_state) ? ws + L.s0 : nullptr, GDP_F32, 4, {N, Hv, d, d}, {Hv * d * d, d * d, d, 1}};
  gdp_tensor tfin{output_final_state ? ws + L.fin : nullptr, GDP_F32, 4, {N, Hv, d, d}, {Hv * d * d, d * d, d, 1}};
  if ((rc = gdp_chunk_prefill(pq, pk, pv, &tg, &tb, n, cu_seqlens, scale, &ts0, output_final_state,
                              use_qk_l2norm_in_kernel, nullptr, nullptr, 0, po, &tfin, nullptr, nullptr,
                              ws + L.inner, workspace_bytes - L.inner, stream)) != GDP_OK)
    return rc;
  if (half) {
    gdp::HalfCopyArgs ha{ws + L.o, output->data, T, (int)Hv, (int)d, output->stride[0], output->stride[1]};
    if ((e = gdp::launch_half_copy(ha, false, (hipStream_t)stream)) != hipSuccess)
      return fail(GDP_EHIP, "output copy launch: %s", hipGetErrorString(e));
  }
  if (output_final_state) {
    gdp::StateArgs sa;
    sa.src = ws + L.fin; sa.dst = output_state->data; sa.mats = N * Hv; sa.K = (int)d; sa.V = (int)d;
    sa.state_dtype = el_type(output_state->dtype);
    if ((e = gdp::launch_state_transpose(sa, false, (hipStream_t)stream)) != hipSuccess)
      return fail(GDP_EHIP, "state launch: %s", hipGetErrorString(e));
  }
  return GDP_OK;
}

int gdp_debug_status(uint32_t *word, int32_t clear, void *stream) {
  g_last_error.clear();
  if (!word) return fail(GDP_EINVAL, "word is required");
  uint32_t *p = nullptr;
  hipError_t e = gdp::debug_word_ptr(&p);
  if (e == hipSuccess) e = hipMemcpyAsync(word, p, sizeof(uint32_t), hipMemcpyDeviceToHost, (hipStream_t)stream);
  if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
  if (e == hipSuccess && clear) e = gdp::launch_fill((int32_t *)p, 1, 0, (hipStream_t)stream);
  if (e != hipSuccess) return fail(GDP_EHIP, "debug status: %s", hipGetErrorString(e));
  return GDP_OK;
}

const char *gdp_version(void) { return "gdp-mi355x 0.1.0 (gfx950)"; }

int gdp_descriptor_capacity(int64_t T, int64_t N, int32_t n, int64_t *nt_cap, int64_t *ntdp_cap) {
  if (T < 0 || N < 0 || n < 1) return fail(GDP_EINVAL, "descriptor capacity: bad sizes");
  if (nt_cap) *nt_cap = (T + 63 * N) / 64;
  if (ntdp_cap) *ntdp_cap = (n * T + 63 * N) / 64;
  return GDP_OK;
}

size_t gdp_workspace_bytes(int64_t T, int64_t N, int32_t n, int32_t Hqk, int32_t Hv, int32_t K, int32_t V,
                           int32_t dtype) {
  int64_t ct, cd;
  if (Hv < 1 || (dtype != GDP_F32 && dtype != GDP_BF16)) return 0;
  if (gdp_descriptor_capacity(T, N, n, &ct, &cd) != GDP_OK) return 0;
  const size_t wy = align256(gdp::wy_buffer_bytes(dtype == GDP_BF16 ? gdp::IN_BF16 : gdp::IN_F32, cd, Hv));
  // the segmented path (forced or automatic) needs its own buffers instead of the WY matrices
  const SegPlan forced = seg_plan(T, N, Hv, K, V, dtype, gdp::PATH_SEGMENTED);
  return std::max(wy, seg_bytes(forced, N, Hv, K, V)) + desc_bytes(N, ct, cd) + order_bytes(N, Hv) +
         progress_bytes(N, Hv, Hqk);
}

int gdp_build_descriptors(const gdp_tensor *cu_seqlens, int32_t n, int64_t T, const gdp_descriptors *out,
                          void *stream) {
  if (!present(cu_seqlens) || !out) return fail(GDP_EINVAL, "build_descriptors: cu_seqlens and out are required");
  if (cu_seqlens->ndim != 1 || cu_seqlens->shape[0] < 1 || cu_seqlens->stride[0] != 1)
    return fail(GDP_EINVAL, "cu_seqlens must be a contiguous [N+1] vector");
  if (cu_seqlens->dtype != GDP_I32 && cu_seqlens->dtype != GDP_I64)
    return fail(GDP_EINVAL, "cu_seqlens must be int32 or int64");
  if (n < 1) return fail(GDP_EINVAL, "num_householder must be >= 1");
  const int64_t N = cu_seqlens->shape[0] - 1;
  int64_t ct, cd;
  if (gdp_descriptor_capacity(T, N, n, &ct, &cd) != GDP_OK) return GDP_EINVAL;
  if (out->nt_cap < ct || out->ntdp_cap < cd)
    return fail(GDP_EINVAL, "descriptor capacities (%lld, %lld) below the bound (%lld, %lld)",
                (long long)out->nt_cap, (long long)out->ntdp_cap, (long long)ct, (long long)cd);
  if (!out->chunk_indices || !out->chunk_indices_dp || !out->chunk_offsets || !out->chunk_offsets_dp)
    return fail(GDP_EINVAL, "descriptor arrays must all be given");
  gdp::DescArgs a;
  a.cu = cu_seqlens->data;
  a.cu_is64 = cu_seqlens->dtype == GDP_I64;
  a.N = N;
  a.n = n;
  a.nt_cap = out->nt_cap;
  a.ntdp_cap = out->ntdp_cap;
  a.chunk_indices = out->chunk_indices;
  a.chunk_indices_dp = out->chunk_indices_dp;
  a.chunk_offsets = out->chunk_offsets;
  a.chunk_offsets_dp = out->chunk_offsets_dp;
  hipError_t e = gdp::launch_descriptors(a, (hipStream_t)stream);
  if (e != hipSuccess) return fail(GDP_EHIP, "descriptor launch: %s", hipGetErrorString(e));
  return GDP_OK;
}

// The prefill behind both entry points.  noalloc: the workspace is the static
// scratch array of the current device (gdp_chunk_prefill_noalloc), after a
// check that the call fits in it.
static int prefill_impl(const gdp_tensor *q, const gdp_tensor *k, const gdp_tensor *v, const gdp_tensor *g_log,
                        const gdp_tensor *beta, int32_t n, const gdp_tensor *cu_seqlens, float scale,
                        const gdp_tensor *initial_state, int32_t output_final_state, int32_t use_qk_l2norm,
                        const gdp_tensor *state_cache, const gdp_tensor *state_indices, int32_t return_chunk_states,
                        const gdp_tensor *o, const gdp_tensor *final_state, const gdp_tensor *chunk_states,
                        const gdp_descriptors *desc, void *workspace, size_t workspace_bytes, void *stream,
                        bool noalloc, bool tc_outputs = false) {
  g_last_error.clear();
  if (!present(q) || !present(k) || !present(v) || !present(g_log) || !present(beta) || !present(o))
    return fail(GDP_EINVAL, "q, k, v, g_log, beta and o are required");
  if (!present(cu_seqlens)) return fail(GDP_EINVAL, "cu_seqlens is required (varlen input only)");
  if (n < 1) return fail(GDP_EINVAL, "num_householder must be >= 1, got %d", n);
  if (q->ndim != 3) return fail(GDP_EINVAL, "q must be [T, Hqk, K]");
  if (k->ndim != 3) return fail(GDP_EINVAL, "k must be [T*n, Hk, K]");
  if (v->ndim != 3) return fail(GDP_EINVAL, "v must be [T*n, Hv, V]");
  const int64_t T = q->shape[0], Hqk = q->shape[1], K = q->shape[2];
  const int64_t Hv = v->shape[1], V = v->shape[2], Hk = k->shape[1];
  if (cu_seqlens->ndim != 1 || cu_seqlens->shape[0] < 1 || cu_seqlens->stride[0] != 1)
    return fail(GDP_EINVAL, "cu_seqlens must be a contiguous [N+1] vector");
  if (cu_seqlens->dtype != GDP_I32 && cu_seqlens->dtype != GDP_I64)
    return fail(GDP_EINVAL, "cu_seqlens must be int32 or int64");
  const int64_t N = cu_seqlens->shape[0] - 1;
  if (Hqk < 1 || Hv < 1 || K < 1 || V < 1) return fail(GDP_EINVAL, "head counts and dims must be positive");
  if (Hv % Hqk != 0) return fail(GDP_EINVAL, "Hv (%lld) must be a multiple of Hqk (%lld)", (long long)Hv, (long long)Hqk);
  if (Hk != Hqk && Hk != Hv) return fail(GDP_EINVAL, "k must have Hqk or Hv heads, got %lld", (long long)Hk);
  if (N > INT32_MAX || Hv > 65535) return fail(GDP_EINVAL, "too many sequences or heads");

  const int32_t dt = q->dtype;
  if (dt != GDP_F32 && dt != GDP_BF16) return fail(GDP_EUNSUPPORTED, "q must be float32 or bfloat16");
  if (k->dtype != dt || v->dtype != dt || o->dtype != dt)
    return fail(GDP_EUNSUPPORTED, "q, k, v and o must share one dtype");
  if (g_log->dtype != GDP_F32 || beta->dtype != GDP_F32)
    return fail(GDP_EUNSUPPORTED, "g_log and beta must be float32");

  int rc;
  const int64_t sq[3] = {T, Hqk, K}, sk[3] = {T * n, Hk, K}, sv[3] = {T * n, Hv, V};
  const int64_t sg[2] = {T, Hv}, sb[2] = {T * n, Hv}, so[3] = {T, Hv, V};
  if ((rc = check_shape(q, "q", 3, sq)) || (rc = check_shape(k, "k", 3, sk)) || (rc = check_shape(v, "v", 3, sv)) ||
      (rc = check_shape(g_log, "g_log", 2, sg)) || (rc = check_shape(beta, "beta", 2, sb)) ||
      (rc = check_shape(o, "o", 3, so)))
    return rc;
  for (const gdp_tensor *t : {q, k, v, g_log, beta, o})
    if (!nonneg_strides(t)) return fail(GDP_EINVAL, "negative strides are not supported");

  const int64_t st_shape[4] = {N, Hv, K, V};
  if (present(initial_state)) {
    if (initial_state->dtype != GDP_F32) return fail(GDP_EUNSUPPORTED, "initial_state must be float32");
    if ((rc = check_shape(initial_state, "initial_state", 4, st_shape))) return rc;
    if (!contiguous(initial_state)) return fail(GDP_EINVAL, "initial_state must be contiguous");
  }
  if (output_final_state) {
    if (!present(final_state)) return fail(GDP_EINVAL, "output_final_state needs a final_state buffer");
    if (final_state->dtype != GDP_F32) return fail(GDP_EUNSUPPORTED, "final_state must be float32");
    if ((rc = check_shape(final_state, "final_state", 4, st_shape))) return rc;
    if (!contiguous(final_state)) return fail(GDP_EINVAL, "final_state must be contiguous");
  }
  if (present(state_cache) != present(state_indices))
    return fail(GDP_EINVAL, "state_cache and state_indices go together");
  int64_t num_slots = 0;
  if (present(state_cache)) {
    if (state_cache->dtype != GDP_F32) return fail(GDP_EUNSUPPORTED, "state_cache must be float32");
    const int64_t cs[4] = {-1, Hv, K, V};
    if ((rc = check_shape(state_cache, "state_cache", 4, cs))) return rc;
    if (!contiguous(state_cache)) return fail(GDP_EINVAL, "state_cache must be contiguous");
    num_slots = state_cache->shape[0];
    if (state_indices->dtype != GDP_I32 && state_indices->dtype != GDP_I64)
      return fail(GDP_EINVAL, "state_indices must be int32 or int64");
    const int64_t si[1] = {N};
    if ((rc = check_shape(state_indices, "state_indices", 1, si))) return rc;
  }
  int64_t nt_cap, ntdp_cap;
  gdp_descriptor_capacity(T, N, n, &nt_cap, &ntdp_cap);
  if (return_chunk_states) {
    if (!present(chunk_states)) return fail(GDP_EINVAL, "return_chunk_states needs a chunk_states buffer");
    if (chunk_states->dtype != GDP_F32) return fail(GDP_EUNSUPPORTED, "chunk_states must be float32");
    const int64_t cs[4] = {-1, Hv, K, V};
    if ((rc = check_shape(chunk_states, "chunk_states", 4, cs))) return rc;
    if (!contiguous(chunk_states)) return fail(GDP_EINVAL, "chunk_states must be contiguous");
    if (chunk_states->shape[0] < nt_cap)
      return fail(GDP_EINVAL, "chunk_states has %lld rows; %lld needed", (long long)chunk_states->shape[0],
                  (long long)nt_cap);
  }
  if (!gdp::prefill_supported(dt == GDP_BF16 ? gdp::IN_BF16 : gdp::IN_F32, (int)K, (int)V))
    return fail(GDP_EUNSUPPORTED, "head dims K=%lld V=%lld with %s inputs are not served", (long long)K,
                (long long)V, dt == GDP_BF16 ? "bf16" : "f32");

  // 16-byte vector loads of q/k/v rows need aligned bases and row strides;
  // the kernels address the 64 rows of a chunk with 32-bit byte offsets.
  const int es = elem_size(dt), eps = 16 / es;
  for (const gdp_tensor *t : {q, k, v})
    if (((uintptr_t)t->data & 15) || (t->stride[0] % eps) || (t->stride[1] % eps))
      return fail(GDP_EUNSUPPORTED, "q/k/v need 16-byte aligned data and row/head strides");
  if (((uintptr_t)o->data & 7) || (o->stride[0] % 4) || (o->stride[1] % 4))
    return fail(GDP_EUNSUPPORTED, "o needs 8-byte aligned data and row/head strides that are multiples of 4");
  for (const gdp_tensor *t : {q, k, v, o, g_log, beta})
    if (t->stride[0] * 64 * elem_size(t->dtype) >= ((int64_t)1 << 31))
      return fail(GDP_EUNSUPPORTED, "row strides above 2^31 / 64 bytes are not served");

  // aliasing: outputs must not overlap inputs or each other
  Range ins[] = {range_of(q, "q"), range_of(k, "k"), range_of(v, "v"), range_of(g_log, "g_log"),
                 range_of(beta, "beta"), range_of(cu_seqlens, "cu_seqlens"),
                 range_of(initial_state, "initial_state"), range_of(state_indices, "state_indices")};
  Range outs[] = {range_of(o, "o"), output_final_state ? range_of(final_state, "final_state") : Range{0, 0, ""},
                  present(state_cache) ? range_of(state_cache, "state_cache") : Range{0, 0, ""},
                  return_chunk_states ? range_of(chunk_states, "chunk_states") : Range{0, 0, ""}};
  for (const Range &ro : outs) {
    for (const Range &ri : ins)
      if (overlap(ro, ri)) return fail(GDP_EALIAS, "%s overlaps input %s", ro.name, ri.name);
  }
  for (int i = 0; i < 4; ++i)
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outs[j])) return fail(GDP_EALIAS, "%s overlaps %s", outs[i].name, outs[j].name);

  // workspace: the WY matrices (or, on the segmented path, the segment buffers),
  // then (when the caller passes none) the descriptors
  const int idt = dt == GDP_BF16 ? gdp::IN_BF16 : gdp::IN_F32;
  const int path = env_path();
  const SegPlan plan = seg_plan(T, N, Hv, K, V, dt, path);
  if (path == gdp::PATH_SEGMENTED && !plan.use)
    return fail(GDP_EUNSUPPORTED, "the segmented path needs bf16 inputs with K == V in {64, 128}");
  // (the fused kernel keeps its WY matrices in LDS: the region is empty then)
  const bool fused_run = !plan.use && gdp::fused_chosen(idt, N, Hv, path);
  const size_t wy_bytes = plan.use ? seg_bytes(plan, N, Hv, K, V)
                                   : (fused_run ? 0 : align256(gdp::wy_buffer_bytes(idt, ntdp_cap, Hv)));
  const size_t tail0 = wy_bytes + (desc ? 0 : desc_bytes(N, nt_cap, ntdp_cap));
  const size_t need = tail0 + order_bytes(N, Hv) + progress_bytes(N, Hv, Hqk);
  if (noalloc) {
    if (need > GDP_NOALLOC_SCRATCH_BYTES)
      return fail(GDP_EWORKSPACE,
                  "gdp_chunk_prefill_noalloc: this call needs %zu bytes of scratch, more than the %zu bytes of "
                  "its static scratch array; call gdp_chunk_prefill with a workspace instead",
                  need, (size_t)GDP_NOALLOC_SCRATCH_BYTES);
    void *p = nullptr;
    hipError_t e = gdp::noalloc_scratch(&p);
    if (e != hipSuccess) return fail(GDP_EHIP, "scratch array address: %s", hipGetErrorString(e));
    workspace = p;
    workspace_bytes = GDP_NOALLOC_SCRATCH_BYTES;
  }
  if (!workspace || workspace_bytes < need)
    return fail(GDP_EWORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes, need);
  if ((uintptr_t)workspace & 255) return fail(GDP_EWORKSPACE, "workspace must be 256-byte aligned");
  gdp_descriptors local;
  const gdp_descriptors *d = desc;
  if (!d) {
    char *p = (char *)workspace + wy_bytes;
    local.chunk_indices = (int32_t *)p;
    p += align256((size_t)nt_cap * 8);
    local.chunk_indices_dp = (int32_t *)p;
    p += align256((size_t)ntdp_cap * 8);
    local.chunk_offsets = (int32_t *)p;
    p += align256((size_t)(N + 1) * 4);
    local.chunk_offsets_dp = (int32_t *)p;
    local.nt_cap = nt_cap;
    local.ntdp_cap = ntdp_cap;
    gdp_tensor cu = *cu_seqlens;
    if ((rc = gdp_build_descriptors(&cu, n, T, &local, stream)) != GDP_OK) return rc;
    d = &local;
  } else {
    if (!d->chunk_indices_dp || !d->chunk_offsets || !d->chunk_offsets_dp)
      return fail(GDP_EINVAL, "caller descriptors need chunk_indices_dp, chunk_offsets and chunk_offsets_dp");
    if (d->nt_cap < nt_cap || d->ntdp_cap < ntdp_cap)
      return fail(GDP_EINVAL, "caller descriptors hold capacities %lld / %lld, below the bounds %lld / %lld for (T, N, n)",
                  (long long)d->nt_cap, (long long)d->ntdp_cap, (long long)nt_cap, (long long)ntdp_cap);
  }

  gdp::PrefillArgs a;
  std::memset(&a, 0, sizeof a);
  a.q = q->data; a.q_st = q->stride[0]; a.q_sh = q->stride[1];
  a.k = k->data; a.k_st = k->stride[0]; a.k_sh = k->stride[1];
  a.v = v->data; a.v_st = v->stride[0]; a.v_sh = v->stride[1];
  a.g = (const float *)g_log->data; a.g_st = g_log->stride[0]; a.g_sh = g_log->stride[1];
  a.beta = (const float *)beta->data; a.b_st = beta->stride[0]; a.b_sh = beta->stride[1];
  a.cu = cu_seqlens->data; a.cu_is64 = cu_seqlens->dtype == GDP_I64;
  a.T = T; a.N = (int)N; a.n = n; a.Hqk = (int)Hqk; a.Hv = (int)Hv; a.Hk = (int)Hk;
  a.scale = (scale == 0.0f) ? (float)(1.0 / std::sqrt((double)K)) : scale;
  a.l2norm = use_qk_l2norm ? 1 : 0;
  a.s0 = present(initial_state) ? (const float *)initial_state->data : nullptr;
  a.final_state = output_final_state ? (float *)final_state->data : nullptr;
  if (present(state_cache)) {
    a.cache = (float *)state_cache->data;
    a.slots = state_indices->data;
    a.slots_is64 = state_indices->dtype == GDP_I64;
    a.num_slots = num_slots;
  }
  if (return_chunk_states) {
    a.chunk_states = (float *)chunk_states->data;
    a.cs_rows = chunk_states->shape[0];
  }
  a.chunk_offsets = d->chunk_offsets;
  a.chunk_indices_dp = d->chunk_indices_dp;
  a.chunk_offsets_dp = d->chunk_offsets_dp;
  a.ntdp_rows = d->ntdp_cap;
  a.tws = workspace;
  a.tws_rows = ntdp_cap;
  a.o = o->data; a.o_st = o->stride[0]; a.o_sh = o->stride[1];
  a.tc_outputs = tc_outputs ? 1 : 0;
  hipError_t e;
  if (debug_validate()) {
    gdp::ValidateArgs va;
    std::memset(&va, 0, sizeof va);
    va.cu = cu_seqlens->data; va.cu_is64 = a.cu_is64; va.N = N; va.T = T;
    if (a.cache) {
      va.slots = a.slots; va.slots_is64 = a.slots_is64; va.nslots_given = N; va.num_slots = a.num_slots;
    }
    if ((e = gdp::launch_validate(va, (hipStream_t)stream)) != hipSuccess)
      return fail(GDP_EHIP, "validation launch: %s", hipGetErrorString(e));
  }
  if (plan.use) {
    // segmented: segment boundaries, summaries (M, B) of every segment, their
    // in-order combination per chain, then every segment from its start state
    char *p = (char *)workspace;
    int32_t *cu_seg = (int32_t *)p; p += align256((size_t)(plan.ns_cap + 1) * 4);
    int32_t *seg_first = (int32_t *)p; p += align256((size_t)(N + 1) * 4);
    int32_t *seg_cs_off = (int32_t *)p; p += align256((size_t)plan.ns_cap * 4);
    float *msum = (float *)p; p += align256((size_t)plan.ns_cap * Hv * K * K * 4);
    float *bsum = (float *)p; p += align256((size_t)plan.ns_cap * Hv * K * V * 4);
    float *seg_init = (float *)p;
    gdp::SegArgs sa;
    sa.cu = cu_seqlens->data; sa.cu_is64 = a.cu_is64; sa.N = N; sa.T = T; sa.Lseg = plan.Lseg;
    sa.ns_cap = plan.ns_cap; sa.chunk_offsets = d->chunk_offsets;
    sa.cu_seg = cu_seg; sa.seg_first = seg_first; sa.seg_cs_off = seg_cs_off;
    if ((e = gdp::launch_segments(sa, (hipStream_t)stream)) != hipSuccess)
      return fail(GDP_EHIP, "segment launch: %s", hipGetErrorString(e));
    gdp::PrefillArgs s1 = a;
    s1.cu = cu_seg; s1.cu_is64 = 0; s1.N = (int)plan.ns_cap;
    s1.s0 = nullptr; s1.final_state = bsum; s1.msum = msum; s1.summary = 1; s1.o = nullptr;
    s1.cache = nullptr; s1.chunk_states = nullptr;
    if ((e = gdp::launch_fused_prefill(s1, (int)K, (int)V, (hipStream_t)stream)) != hipSuccess)
      return fail(GDP_EHIP, "segment summary launch: %s", hipGetErrorString(e));
    gdp::CombineArgs ca;
    ca.N = (int)N; ca.Hv = (int)Hv; ca.seg_first = seg_first; ca.msum = msum; ca.bsum = bsum;
    ca.seg_init = seg_init; ca.s0 = a.s0; ca.final_state = a.final_state;
    ca.cache = a.cache; ca.slots = a.slots; ca.slots_is64 = a.slots_is64; ca.num_slots = a.num_slots;
    if ((e = gdp::launch_combine(ca, (int)K, (int)V, (hipStream_t)stream)) != hipSuccess)
      return fail(GDP_EHIP, "segment combine launch: %s", hipGetErrorString(e));
    gdp::PrefillArgs s3 = a;
    s3.cu = cu_seg; s3.cu_is64 = 0; s3.N = (int)plan.ns_cap;
    s3.s0 = seg_init; s3.final_state = nullptr; s3.cache = nullptr; s3.chunk_offsets = seg_cs_off;
    if ((e = gdp::launch_fused_prefill(s3, (int)K, (int)V, (hipStream_t)stream)) != hipSuccess)
      return fail(GDP_EHIP, "segment prefill launch: %s", hipGetErrorString(e));
    return GDP_OK;
  }
  if (progress_bytes(N, Hv, Hqk) > 0 && gdp::fused_chosen(idt, N, Hv, path)) {  // after the work order
    a.progress = (int32_t *)((char *)workspace + tail0 + order_bytes(N, Hv));
    if ((e = gdp::launch_fill(a.progress, N * Hv, INT32_MAX, (hipStream_t)stream)) != hipSuccess)
      return fail(GDP_EHIP, "progress fill launch: %s", hipGetErrorString(e));
  }
  if (order_grid(N, Hv) && gdp::fused_chosen(idt, N, Hv, path)) {  // after the WY region and the descriptors
    int32_t *order = (int32_t *)((char *)workspace + tail0);
    gdp::OrderArgs oa;
    oa.cu = cu_seqlens->data; oa.cu_is64 = a.cu_is64; oa.N = N; oa.T = T; oa.Hqk = (int)Hqk; oa.Hv = (int)Hv;
    oa.order = order;
    if ((e = gdp::launch_order(oa, (hipStream_t)stream)) != hipSuccess)
      return fail(GDP_EHIP, "order launch: %s", hipGetErrorString(e));
    a.order = order;
  }
  e = gdp::launch_prefill(a, idt, (int)K, (int)V, path, (hipStream_t)stream);
  if (e != hipSuccess) return fail(GDP_EHIP, "prefill launch: %s", hipGetErrorString(e));
  return GDP_OK;
}

int gdp_chunk_prefill(const gdp_tensor *q, const gdp_tensor *k, const gdp_tensor *v, const gdp_tensor *g_log,
                      const gdp_tensor *beta, int32_t n, const gdp_tensor *cu_seqlens, float scale,
                      const gdp_tensor *initial_state, int32_t output_final_state, int32_t use_qk_l2norm,
                      const gdp_tensor *state_cache, const gdp_tensor *state_indices, int32_t return_chunk_states,
                      const gdp_tensor *o, const gdp_tensor *final_state, const gdp_tensor *chunk_states,
                      const gdp_descriptors *desc, void *workspace, size_t workspace_bytes, void *stream) {
  return prefill_impl(q, k, v, g_log, beta, n, cu_seqlens, scale, initial_state, output_final_state, use_qk_l2norm,
                      state_cache, state_indices, return_chunk_states, o, final_state, chunk_states, desc, workspace,
                      workspace_bytes, stream, false);
}

int gdp_chunk_prefill_noalloc(const gdp_tensor *q, const gdp_tensor *k, const gdp_tensor *v,
                              const gdp_tensor *g_log, const gdp_tensor *beta, int32_t n,
                              const gdp_tensor *cu_seqlens, float scale, const gdp_tensor *initial_state,
                              int32_t output_final_state, int32_t use_qk_l2norm, const gdp_tensor *state_cache,
                              const gdp_tensor *state_indices, int32_t return_chunk_states, const gdp_tensor *o,
                              const gdp_tensor *final_state, const gdp_tensor *chunk_states,
                              const gdp_descriptors *desc, void *stream) {
  return prefill_impl(q, k, v, g_log, beta, n, cu_seqlens, scale, initial_state, output_final_state, use_qk_l2norm,
                      state_cache, state_indices, return_chunk_states, o, final_state, chunk_states, desc, nullptr, 0,
                      stream, true);
}

namespace {
// Workspace of the backward call.  Recurrent path: descriptors, the state
// entering every token chunk, the forward's outputs, the rows' norm factors,
// the forward's own workspace.  Chunked path: descriptors, the state entering
// and the state gradient leaving every expanded chunk, the prep bundles.  The
// size is the larger of the two for inputs the chunked path serves, so either
// path runs in it.
struct BwdLayout {
  size_t desc = 0, cs = 0, o = 0, rn = 0, fwd = 0, total = 0;
  size_t xs = 0, xd = 0, xb = 0, xtotal = 0;  // chunked path
  int64_t nt_cap = 0, ntdp_cap = 0;
};
static BwdLayout bwd_layout(int64_t T, int64_t N, int32_t n, int32_t Hqk, int32_t Hv, int32_t K, int32_t V, int32_t dtype) {
  BwdLayout L;
  if (gdp_descriptor_capacity(T, N, n, &L.nt_cap, &L.ntdp_cap) != GDP_OK) return L;
  const size_t fwd = gdp_workspace_bytes(T, N, n, Hqk, Hv, K, V, dtype);
  if (!fwd) return L;
  L.desc = 0;
  L.cs = L.desc + desc_bytes(N, L.nt_cap, L.ntdp_cap);
  L.o = L.cs + align256((size_t)(L.nt_cap > 0 ? L.nt_cap : 1) * Hv * K * V * 4);
  L.rn = L.o + align256((size_t)T * Hv * V * elem_size(dtype));
  // the rows' norm factors: q [T, Hqk], k [T*n, Hk <= Hv], then one float 1
  L.fwd = L.rn + align256((size_t)T * Hqk * 4) + align256((size_t)T * n * Hv * 4) + 256;
  L.total = L.fwd + fwd;
  if (gdp::bwd_chunked_supported(dtype == GDP_BF16 ? gdp::IN_BF16 : gdp::IN_F32, K, V, n)) {
    const size_t rows = (size_t)(L.ntdp_cap > 0 ? L.ntdp_cap : 1);
    L.xs = L.cs;  // after the descriptors
    L.xd = L.xs + align256(rows * Hv * gdp::bwd_state_record_bytes((int)K, (int)V));
    L.xb = L.xd + align256(rows * Hv * K * V * 4);
    L.xtotal = L.xb + align256(rows * Hv * gdp::bwd_bundle_bytes(n));
  }
  return L;
}
// GDP_BACKWARD_PATH=recurrent keeps the per-token kernel for inputs the chunked
// path serves (for comparison); any other value or none picks the chunked path.
static bool env_backward_recurrent() {
  const char *s = std::getenv("GDP_BACKWARD_PATH");
  return s && std::strcmp(s, "recurrent") == 0;
}
}  // namespace

// The backward's last steps: zero rows of dv outside every sequence, and (with
// the in-kernel norm, on the recurrent path; the chunked gradient kernel applies
// it itself) the gradients by the raw q and k rows from those by their
// normalised rows.
// Zeroes the rows of a float32 gradient [T * per_token, heads, D] (D = 1 for a
// 2-d [T * per_token, heads] one) that no sequence covers: before cu[0] or from
// cu[N] on.
static int zero_rows_outside(const gdp_tensor *t, const gdp_tensor *cu_seqlens, int64_t T, int64_t N,
                             int32_t per_token, int64_t heads, int64_t D, void *stream) {
  gdp::ZeroOutsideArgs z;
  z.p = (float *)t->data; z.st = t->stride[0]; z.sh = t->ndim > 1 ? t->stride[1] : 0;
  z.cu = cu_seqlens->data; z.cu_is64 = cu_seqlens->dtype == GDP_I64;
  z.T = T; z.N = (int)N; z.n = per_token; z.heads = (int)heads; z.D = (int)D;
  const hipError_t e = gdp::launch_zero_outside(z, (hipStream_t)stream);
  return e == hipSuccess ? GDP_OK : fail(GDP_EHIP, "zero fill launch: %s", hipGetErrorString(e));
}

static int bwd_finish(const gdp_tensor *q, const gdp_tensor *k, const gdp_tensor *dq, const gdp_tensor *dk,
                      const gdp_tensor *dv, const gdp_tensor *cu_seqlens, int64_t T, int64_t N, int32_t n, int64_t Hqk,
                      int64_t Hk, int64_t Hv, int64_t K, int64_t V, int idt, int32_t use_qk_l2norm, void *stream) {
  hipError_t e;
  int rc;
  if ((rc = zero_rows_outside(dv, cu_seqlens, T, N, n, Hv, V, stream)) != GDP_OK) return rc;
  if (use_qk_l2norm) {
    gdp::NormGradArgs na;
    na.x = q->data; na.x_st = q->stride[0]; na.x_sh = q->stride[1];
    na.g = (float *)dq->data; na.g_st = dq->stride[0]; na.g_sh = dq->stride[1];
    na.rows = T * Hqk; na.heads = (int)Hqk;
    if ((e = gdp::launch_l2norm_grad(na, idt, (int)K, (hipStream_t)stream)) != hipSuccess)
      return fail(GDP_EHIP, "norm gradient launch: %s", hipGetErrorString(e));
    na.x = k->data; na.x_st = k->stride[0]; na.x_sh = k->stride[1];
    na.g = (float *)dk->data; na.g_st = dk->stride[0]; na.g_sh = dk->stride[1];
    na.rows = T * n * Hk; na.heads = (int)Hk;
    if ((e = gdp::launch_l2norm_grad(na, idt, (int)K, (hipStream_t)stream)) != hipSuccess)
      return fail(GDP_EHIP, "norm gradient launch: %s", hipGetErrorString(e));
  }
  return GDP_OK;
}

size_t gdp_backward_workspace_bytes(int64_t T, int64_t N, int32_t n, int32_t Hqk, int32_t Hv, int32_t K, int32_t V,
                                    int32_t dtype) {
  if (T < 0 || N < 0 || n < 1 || Hqk < 1 || Hv < 1 || K < 1 || V < 1) return 0;
  if (dtype != GDP_F32 && dtype != GDP_BF16) return 0;
  const BwdLayout L = bwd_layout(T, N, n, Hqk, Hv, K, V, dtype);
  return std::max(L.total, L.xtotal);
}

int gdp_chunk_prefill_backward(const gdp_tensor *q, const gdp_tensor *k, const gdp_tensor *v, const gdp_tensor *g_log,
                               const gdp_tensor *beta, int32_t n, const gdp_tensor *cu_seqlens, float scale,
                               const gdp_tensor *initial_state, int32_t use_qk_l2norm, const gdp_tensor *d_o,
                               const gdp_tensor *d_final_state, const gdp_tensor *dq, const gdp_tensor *dk,
                               const gdp_tensor *dv, const gdp_tensor *dg_log, const gdp_tensor *dbeta,
                               const gdp_tensor *d_initial_state, void *workspace, size_t workspace_bytes,
                               void *stream) {
  g_last_error.clear();
  if (!present(q) || !present(k) || !present(v) || !present(g_log) || !present(beta) || !present(d_o))
    return fail(GDP_EINVAL, "q, k, v, g_log, beta and d_o are required");
  if (!present(dq) || !present(dk) || !present(dv) || !present(dg_log) || !present(dbeta))
    return fail(GDP_EINVAL, "dq, dk, dv, dg_log and dbeta are required");
  if (!present(cu_seqlens)) return fail(GDP_EINVAL, "cu_seqlens is required (varlen input only)");
  if (n < 1) return fail(GDP_EINVAL, "num_householder must be >= 1, got %d", n);
  if (q->ndim != 3 || k->ndim != 3 || v->ndim != 3 || cu_seqlens->ndim != 1)
    return fail(GDP_EINVAL, "q, k, v must be 3-d and cu_seqlens 1-d");
  const int64_t T = q->shape[0], Hqk = q->shape[1], K = q->shape[2];
  const int64_t Hk = k->shape[1], Hv = v->shape[1], V = v->shape[2];
  const int64_t N = cu_seqlens->shape[0] - 1;
  if (N < 0 || Hqk < 1 || Hv < 1 || Hk < 1) return fail(GDP_EINVAL, "bad sizes");
  if (Hv % Hqk != 0 || (Hk != Hqk && Hk != Hv)) return fail(GDP_EINVAL, "head counts: Hv a multiple of Hqk, Hk = Hqk or Hv");
  if (!gdp::backward_supported((int)K, (int)V, n))
    return fail(GDP_EUNSUPPORTED, "backward needs K, V in {64, 128} and num_householder <= 5");
  const int32_t dt = q->dtype;
  if (dt != GDP_F32 && dt != GDP_BF16) return fail(GDP_EUNSUPPORTED, "q must be float32 or bfloat16");
  if (d_o->dtype != dt) return fail(GDP_EUNSUPPORTED, "d_o must have q's dtype");
  int rc;
  const int64_t sdo[3] = {T, Hv, V}, sq[3] = {T, Hqk, K}, sk[3] = {T * n, Hk, K}, sv[3] = {T * n, Hv, V};
  const int64_t sg[2] = {T, Hv}, sb[2] = {T * n, Hv}, sst[4] = {N, Hv, K, V};
  if ((rc = check_shape(d_o, "d_o", 3, sdo)) || (rc = check_shape(dq, "dq", 3, sq)) || (rc = check_shape(dk, "dk", 3, sk)) ||
      (rc = check_shape(dv, "dv", 3, sv)) || (rc = check_shape(dg_log, "dg_log", 2, sg)) ||
      (rc = check_shape(dbeta, "dbeta", 2, sb)))
    return rc;
  for (const gdp_tensor *t : {dq, dk, dv, dg_log, dbeta})
    if (t->dtype != GDP_F32) return fail(GDP_EUNSUPPORTED, "gradients are float32");
  for (const gdp_tensor *t : {dq, dk, dg_log, dbeta})
    if (!contiguous(t)) return fail(GDP_EINVAL, "dq, dk, dg_log and dbeta must be contiguous (they are accumulated)");
  if (!nonneg_strides(d_o) || !nonneg_strides(dv)) return fail(GDP_EINVAL, "negative strides are not supported");
  if (present(d_final_state)) {
    if ((rc = check_shape(d_final_state, "d_final_state", 4, sst))) return rc;
    if (d_final_state->dtype != GDP_F32 || !contiguous(d_final_state))
      return fail(GDP_EUNSUPPORTED, "d_final_state must be contiguous float32");
  }
  if (present(d_initial_state)) {
    if ((rc = check_shape(d_initial_state, "d_initial_state", 4, sst))) return rc;
    if (d_initial_state->dtype != GDP_F32 || !contiguous(d_initial_state))
      return fail(GDP_EUNSUPPORTED, "d_initial_state must be contiguous float32");
  }
  // gradients may not overlap inputs or each other
  Range ins[] = {range_of(q, "q"), range_of(k, "k"), range_of(v, "v"), range_of(g_log, "g_log"),
                 range_of(beta, "beta"), range_of(cu_seqlens, "cu_seqlens"), range_of(initial_state, "initial_state"),
                 range_of(d_o, "d_o"), range_of(d_final_state, "d_final_state")};
  Range outs[] = {range_of(dq, "dq"), range_of(dk, "dk"), range_of(dv, "dv"), range_of(dg_log, "dg_log"),
                  range_of(dbeta, "dbeta"), range_of(d_initial_state, "d_initial_state")};
  for (const Range &ro : outs)
    for (const Range &ri : ins)
      if (overlap(ro, ri)) return fail(GDP_EALIAS, "%s overlaps input %s", ro.name, ri.name);
  for (int i = 0; i < 6; ++i)
    for (int j = i + 1; j < 6; ++j)
      if (overlap(outs[i], outs[j])) return fail(GDP_EALIAS, "%s overlaps %s", outs[i].name, outs[j].name);
  const BwdLayout L = bwd_layout(T, N, n, (int32_t)Hqk, (int32_t)Hv, (int32_t)K, (int32_t)V, dt);
  if (!L.total) return fail(GDP_EINVAL, "bad sizes");
  const size_t need = std::max(L.total, L.xtotal);
  if (!workspace || workspace_bytes < need)
    return fail(GDP_EWORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes, need);
  bool chunked = L.xtotal > 0 && !env_backward_recurrent();
  // (the chunked kernels read q, k, v and d_o rows in 16-byte pieces)
  for (const gdp_tensor *t : {q, k, v, d_o})
    if (((uintptr_t)t->data & 15) || (t->stride[0] % 8) || (t->stride[1] % 8)) chunked = false;
  if ((uintptr_t)workspace & 255) return fail(GDP_EWORKSPACE, "workspace must be 256-byte aligned");
  char *ws = (char *)workspace;

  // descriptors, then the forward pass leaving the state entering every token chunk
  gdp_descriptors d;
  char *p = ws + L.desc;
  d.chunk_indices = (int32_t *)p; p += align256((size_t)L.nt_cap * 8);
  d.chunk_indices_dp = (int32_t *)p; p += align256((size_t)L.ntdp_cap * 8);
  d.chunk_offsets = (int32_t *)p; p += align256((size_t)(N + 1) * 4);
  d.chunk_offsets_dp = (int32_t *)p;
  d.nt_cap = L.nt_cap; d.ntdp_cap = L.ntdp_cap;
  gdp_tensor cu = *cu_seqlens;
  if ((rc = gdp_build_descriptors(&cu, n, T, &d, stream)) != GDP_OK) return rc;
  gdp_tensor none{};
  hipError_t e;
  const int idt = dt == GDP_BF16 ? gdp::IN_BF16 : gdp::IN_F32;
  const int64_t csr = L.nt_cap > 0 ? L.nt_cap : 1;
  if (!chunked) {  // the forward pass leaving the state entering every token chunk
    gdp_tensor tcs{ws + L.cs, GDP_F32, 4, {csr, Hv, K, V}, {Hv * K * V, K * V, V, 1}};
    gdp_tensor to{ws + L.o, dt, 3, {T, Hv, V}, {Hv * V, V, 1}};
    if ((rc = prefill_impl(q, k, v, g_log, beta, n, cu_seqlens, scale, initial_state, 0, use_qk_l2norm, &none, &none,
                           1, &to, &none, &tcs, &d, ws + L.fwd, workspace_bytes - L.fwd, stream, false, true)) != GDP_OK)
      return rc;
  }
  if (!chunked) {  // the per-token kernel accumulates dq, dk, dg_log and dbeta with atomics
    for (const gdp_tensor *t : {dq, dk, dg_log, dbeta}) {
      int64_t cnt = 1;
      for (int i = 0; i < t->ndim; ++i) cnt *= t->shape[i];
      if ((e = gdp::launch_fill((int32_t *)t->data, cnt, 0, (hipStream_t)stream)) != hipSuccess)
        return fail(GDP_EHIP, "zero fill launch: %s", hipGetErrorString(e));
    }
  }
  if (chunked) {
    // the chunked kernels store every entry inside the sequences once; only the
    // rows outside them are zeroed here
    if ((rc = zero_rows_outside(dq, cu_seqlens, T, N, 1, Hqk, K, stream)) != GDP_OK ||
        (rc = zero_rows_outside(dk, cu_seqlens, T, N, n, Hk, K, stream)) != GDP_OK ||
        (rc = zero_rows_outside(dg_log, cu_seqlens, T, N, 1, Hv, 1, stream)) != GDP_OK ||
        (rc = zero_rows_outside(dbeta, cu_seqlens, T, N, n, Hv, 1, stream)) != GDP_OK)
      return rc;
    gdp::BwdChunkArgs c;
    std::memset(&c, 0, sizeof c);
    c.q = q->data; c.q_st = q->stride[0]; c.q_sh = q->stride[1];
    c.k = k->data; c.k_st = k->stride[0]; c.k_sh = k->stride[1];
    c.v = v->data; c.v_st = v->stride[0]; c.v_sh = v->stride[1];
    c.g = (const float *)g_log->data; c.g_st = g_log->stride[0]; c.g_sh = g_log->stride[1];
    c.beta = (const float *)beta->data; c.b_st = beta->stride[0]; c.b_sh = beta->stride[1];
    c.cu = cu_seqlens->data; c.cu_is64 = cu_seqlens->dtype == GDP_I64;
    c.T = T; c.N = (int)N; c.n = n; c.Hqk = (int)Hqk; c.Hv = (int)Hv; c.Hk = (int)Hk;
    c.scale = (scale == 0.0f) ? (float)(1.0 / std::sqrt((double)K)) : scale;
    c.l2norm = use_qk_l2norm ? 1 : 0;
    c.chunk_indices_dp = d.chunk_indices_dp;
    c.chunk_offsets_dp = d.chunk_offsets_dp;
    c.ntdp_rows = L.ntdp_cap;
    c.bundle = ws + L.xb;
    c.s0 = present(initial_state) ? (const float *)initial_state->data : nullptr;
    c.states = ws + L.xs;
    c.dstates = (float *)(ws + L.xd);
    c.dout = d_o->data; c.do_st = d_o->stride[0]; c.do_sh = d_o->stride[1];
    c.dfinal = present(d_final_state) ? (const float *)d_final_state->data : nullptr;
    c.ds0 = present(d_initial_state) ? (float *)d_initial_state->data : nullptr;
    c.dq = (float *)dq->data; c.dq_st = dq->stride[0]; c.dq_sh = dq->stride[1];
    c.dk = (float *)dk->data; c.dk_st = dk->stride[0]; c.dk_sh = dk->stride[1];
    c.dv = (float *)dv->data; c.dv_st = dv->stride[0]; c.dv_sh = dv->stride[1];
    c.dg = (float *)dg_log->data; c.dg_st = dg_log->stride[0]; c.dg_sh = dg_log->stride[1];
    c.dbeta = (float *)dbeta->data; c.db_st = dbeta->stride[0]; c.db_sh = dbeta->stride[1];
    if ((e = gdp::launch_bwd_chunked(c, (int)K, (int)V, (hipStream_t)stream)) != hipSuccess)
      return fail(GDP_EHIP, "chunked backward launch: %s", hipGetErrorString(e));
    return bwd_finish(q, k, dq, dk, dv, cu_seqlens, T, N, n, Hqk, Hk, Hv, K, V, idt, 0, stream);
  }
  // the rows' L2-norm factors (or a single 1 read with zero strides)
  float *rq = (float *)(ws + L.rn), *rk = (float *)(ws + L.rn + align256((size_t)T * Hqk * 4));
  float *one = (float *)(ws + L.fwd - 256);
  if (use_qk_l2norm) {
    gdp::NormGradArgs ra;
    ra.x = q->data; ra.x_st = q->stride[0]; ra.x_sh = q->stride[1];
    ra.g = rq; ra.g_st = Hqk; ra.g_sh = 1; ra.rows = T * Hqk; ra.heads = (int)Hqk;
    if ((e = gdp::launch_row_norm(ra, idt, (int)K, (hipStream_t)stream)) != hipSuccess)
      return fail(GDP_EHIP, "row norm launch: %s", hipGetErrorString(e));
    ra.x = k->data; ra.x_st = k->stride[0]; ra.x_sh = k->stride[1];
    ra.g = rk; ra.g_st = Hk; ra.rows = T * n * Hk; ra.heads = (int)Hk;
    if ((e = gdp::launch_row_norm(ra, idt, (int)K, (hipStream_t)stream)) != hipSuccess)
      return fail(GDP_EHIP, "row norm launch: %s", hipGetErrorString(e));
  } else if ((e = gdp::launch_fill((int32_t *)one, 1, 0x3f800000, (hipStream_t)stream)) != hipSuccess) {
    return fail(GDP_EHIP, "fill launch: %s", hipGetErrorString(e));
  }
  gdp::BwdArgs a;
  std::memset(&a, 0, sizeof a);
  if (use_qk_l2norm) {
    a.rq = rq; a.rq_st = Hqk; a.rq_sh = 1;
    a.rk = rk; a.rk_st = Hk; a.rk_sh = 1;
  } else {
    a.rq = one; a.rk = one;  // zero strides
  }
  a.q = q->data; a.q_st = q->stride[0]; a.q_sh = q->stride[1];
  a.k = k->data; a.k_st = k->stride[0]; a.k_sh = k->stride[1];
  a.v = v->data; a.v_st = v->stride[0]; a.v_sh = v->stride[1];
  a.g = (const float *)g_log->data; a.g_st = g_log->stride[0]; a.g_sh = g_log->stride[1];
  a.beta = (const float *)beta->data; a.b_st = beta->stride[0]; a.b_sh = beta->stride[1];
  a.cu = cu_seqlens->data; a.cu_is64 = cu_seqlens->dtype == GDP_I64;
  a.T = T; a.N = (int)N; a.n = n; a.Hqk = (int)Hqk; a.Hv = (int)Hv; a.Hk = (int)Hk;
  a.scale = (scale == 0.0f) ? (float)(1.0 / std::sqrt((double)K)) : scale;
  a.chunk_states = (const float *)(ws + L.cs);
  a.cs_rows = csr;
  a.chunk_offsets = d.chunk_offsets;
  a.dout = d_o->data; a.do_st = d_o->stride[0]; a.do_sh = d_o->stride[1];
  a.dfinal = present(d_final_state) ? (const float *)d_final_state->data : nullptr;
  a.dq = (float *)dq->data; a.dq_st = dq->stride[0]; a.dq_sh = dq->stride[1];
  a.dk = (float *)dk->data; a.dk_st = dk->stride[0]; a.dk_sh = dk->stride[1];
  a.dv = (float *)dv->data; a.dv_st = dv->stride[0]; a.dv_sh = dv->stride[1];
  a.dg = (float *)dg_log->data; a.dg_st = dg_log->stride[0]; a.dg_sh = dg_log->stride[1];
  a.dbeta = (float *)dbeta->data; a.db_st = dbeta->stride[0]; a.db_sh = dbeta->stride[1];
  a.ds0 = present(d_initial_state) ? (float *)d_initial_state->data : nullptr;
  if ((e = gdp::launch_backward(a, idt, (int)K, (int)V, (hipStream_t)stream)) != hipSuccess)
    return fail(GDP_EHIP, "backward launch: %s", hipGetErrorString(e));
  return bwd_finish(q, k, dq, dk, dv, cu_seqlens, T, N, n, Hqk, Hk, Hv, K, V, idt, use_qk_l2norm, stream);
}

int gdp_recurrent_decode(const gdp_tensor *q, const gdp_tensor *k, const gdp_tensor *v, const gdp_tensor *g_log,
                         const gdp_tensor *beta, int32_t n, float scale, int32_t use_qk_l2norm,
                         const gdp_tensor *state_cache, const gdp_tensor *state_indices, const gdp_tensor *o,
                         void *stream) {
  g_last_error.clear();
  if (!present(q) || !present(k) || !present(v) || !present(g_log) || !present(beta) || !present(o))
    return fail(GDP_EINVAL, "q, k, v, g_log, beta and o are required");
  if (!present(state_cache) || !present(state_indices))
    return fail(GDP_EINVAL, "state_cache and state_indices are required");
  if (n < 1) return fail(GDP_EINVAL, "num_householder must be >= 1, got %d", n);
  if (q->ndim != 3 || k->ndim != 3 || v->ndim != 3)
    return fail(GDP_EINVAL, "q must be [N, Hqk, K], k [N*n, Hk, K] and v [N*n, Hv, V]");
  const int64_t N = q->shape[0], Hqk = q->shape[1], K = q->shape[2];
  const int64_t Hv = v->shape[1], V = v->shape[2], Hk = k->shape[1];
  if (Hqk < 1 || Hv < 1 || K < 1 || V < 1) return fail(GDP_EINVAL, "head counts and dims must be positive");
  if (Hv % Hqk != 0) return fail(GDP_EINVAL, "Hv (%lld) must be a multiple of Hqk (%lld)", (long long)Hv, (long long)Hqk);
  if (Hk != Hqk && Hk != Hv) return fail(GDP_EINVAL, "k must have Hqk or Hv heads, got %lld", (long long)Hk);
  if (N > INT32_MAX || Hv > 65535) return fail(GDP_EINVAL, "too many sequences or heads");
  const int32_t dt = q->dtype;
  if (dt != GDP_F32 && dt != GDP_BF16) return fail(GDP_EUNSUPPORTED, "q must be float32 or bfloat16");
  if (k->dtype != dt || v->dtype != dt || o->dtype != dt)
    return fail(GDP_EUNSUPPORTED, "q, k, v and o must share one dtype");
  if (g_log->dtype != GDP_F32 || beta->dtype != GDP_F32 || state_cache->dtype != GDP_F32)
    return fail(GDP_EUNSUPPORTED, "g_log, beta and state_cache must be float32");
  if (state_indices->dtype != GDP_I32 && state_indices->dtype != GDP_I64)
    return fail(GDP_EINVAL, "state_indices must be int32 or int64");
  int rc;
  const int64_t sq[3] = {N, Hqk, K}, sk[3] = {N * n, Hk, K}, sv[3] = {N * n, Hv, V};
  const int64_t sg[2] = {N, Hv}, sb[2] = {N * n, Hv}, so[3] = {N, Hv, V}, si[1] = {N};
  const int64_t sc[4] = {-1, Hv, K, V};
  if ((rc = check_shape(q, "q", 3, sq)) || (rc = check_shape(k, "k", 3, sk)) || (rc = check_shape(v, "v", 3, sv)) ||
      (rc = check_shape(g_log, "g_log", 2, sg)) || (rc = check_shape(beta, "beta", 2, sb)) ||
      (rc = check_shape(o, "o", 3, so)) || (rc = check_shape(state_indices, "state_indices", 1, si)) ||
      (rc = check_shape(state_cache, "state_cache", 4, sc)))
    return rc;
  for (const gdp_tensor *t : {q, k, v, g_log, beta, o})
    if (!nonneg_strides(t)) return fail(GDP_EINVAL, "negative strides are not supported");
  if (!contiguous(state_cache)) return fail(GDP_EINVAL, "state_cache must be contiguous");
  if (!gdp::decode_supported((int)K, (int)V))
    return fail(GDP_EUNSUPPORTED, "head dims K=%lld V=%lld are not served", (long long)K, (long long)V);
  // the state cache is read and written; o is written: neither may overlap an input or the other
  Range ins[] = {range_of(q, "q"), range_of(k, "k"), range_of(v, "v"), range_of(g_log, "g_log"),
                 range_of(beta, "beta"), range_of(state_indices, "state_indices")};
  Range outs[] = {range_of(o, "o"), range_of(state_cache, "state_cache")};
  for (const Range &ro : outs)
    for (const Range &ri : ins)
      if (overlap(ro, ri)) return fail(GDP_EALIAS, "%s overlaps input %s", ro.name, ri.name);
  if (overlap(outs[0], outs[1])) return fail(GDP_EALIAS, "o overlaps state_cache");

  gdp::DecodeArgs a;
  std::memset(&a, 0, sizeof a);
  a.q = q->data; a.q_st = q->stride[0]; a.q_sh = q->stride[1];
  a.k = k->data; a.k_st = k->stride[0]; a.k_sh = k->stride[1];
  a.v = v->data; a.v_st = v->stride[0]; a.v_sh = v->stride[1];
  a.g = (const float *)g_log->data; a.g_st = g_log->stride[0]; a.g_sh = g_log->stride[1];
  a.beta = (const float *)beta->data; a.b_st = beta->stride[0]; a.b_sh = beta->stride[1];
  a.N = (int)N; a.n = n; a.Hqk = (int)Hqk; a.Hv = (int)Hv; a.Hk = (int)Hk;
  a.scale = (scale == 0.0f) ? (float)(1.0 / std::sqrt((double)K)) : scale;
  a.l2norm = use_qk_l2norm ? 1 : 0;
  a.cache = (float *)state_cache->data;
  a.num_slots = state_cache->shape[0];
  a.slots = state_indices->data;
  a.slots_is64 = state_indices->dtype == GDP_I64;
  a.o = o->data; a.o_st = o->stride[0]; a.o_sh = o->stride[1];
  hipError_t e;
  if (debug_validate()) {
    gdp::ValidateArgs va;
    std::memset(&va, 0, sizeof va);
    va.slots = a.slots; va.slots_is64 = a.slots_is64; va.nslots_given = N; va.num_slots = a.num_slots;
    if ((e = gdp::launch_validate(va, (hipStream_t)stream)) != hipSuccess)
      return fail(GDP_EHIP, "validation launch: %s", hipGetErrorString(e));
  }
  e = gdp::launch_decode(a, dt == GDP_BF16 ? gdp::IN_BF16 : gdp::IN_F32, (int)K, (int)V, (hipStream_t)stream);
  if (e != hipSuccess) return fail(GDP_EHIP, "decode launch: %s", hipGetErrorString(e));
  return GDP_OK;
}

}  // extern "C"
