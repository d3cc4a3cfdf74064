/*
 * gdp_oracle.c -- plain fp64 CPU oracle for the Gated DeltaProduct (GDP)
 * prefill forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library path may include, link,
 * load or call this file.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code, header, table or
 * helper with the HIP implementation.
 *
 * What it computes (FlashInfer docs, "flashinfer.gdp_prefill.
 * chunk_gated_delta_product", the recurrence display at the top of the page):
 * for every sequence and every state head, token by token,
 *     S <- alpha_t * S                                   (decay first)
 *     for j = 0..n-1, sub-token row r = t*n + j:
 *         e_r = beta_r * (v_r - S^T k_r)                 (v_new)
 *         S   <- S + k_r e_r^T
 *     o_t = scale * S^T q_t                              (after the last update)
 * S is stored K-major, S[kk][vv], as the Megatron Core page's initial_state
 * shape [N, H, K, V] says; the FlashInfer formula is the same recurrence on the
 * transposed (V-major) state.  alpha_t = exp(g_log_t) because the Megatron
 * page's g argument holds log decays.  With n = 1 this is the gated delta
 * rule written out on the blog page's "GDN: fixed state instead of a per-token
 * cache" section (Sbar = lambda S, vhat = Sbar^T k, e = beta (v - vhat),
 * S = Sbar + k e^T, r = q^T S).
 *
 * Readings of points the pages leave open (each also listed in the design
 * notes):
 *   - scale == 0 means K^-1/2 (FlashInfer: "when None or 0.0").
 *   - use_qk_l2norm divides every q row and every k sub-token row, per qk
 *     head, by sqrt(sum x^2 + 1e-6).
 *   - state head h reads qk head h / (Hv / Hqk) (contiguous groups).
 *   - chunk_states row chunk_offsets[i] + c is the state entering token
 *     chunk c of sequence i, i.e. after its first 64*c tokens (Megatron
 *     page, return_chunk_states); the final state is not a row.
 *   - the state cache is an output sink: slot state_indices[i] >= 0 receives
 *     the final state of sequence i; -1 writes nothing.
 *   - a zero-length sequence has no chunks and its final state is its
 *     initial state.
 *
 * Chains (sequence, state head) are independent, so they are spread over a
 * pthread pool, longest first.  Inside a chain the loop is the plain
 * recurrence above with no blocking or reordering.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GDPO_CHUNK 64

typedef struct {
  int64_t T, N;
  int n, Hqk, Hv, K, V;
  const double *q, *k, *v, *g_log, *beta;
  const int64_t *cu;
  double scale;
  const double *s0;
  int l2norm;
  double *o, *final_state, *chunk_states;
  const int64_t *chunk_offsets;
  double *cache;
  const int64_t *slots;
  double *vnew;
  int64_t *order; /* chain ids, longest sequence first */
  int64_t nchains;
  int64_t next;
  pthread_mutex_t mu;
} gdpo_problem;

/* x <- x / sqrt(sum x^2 + 1e-6) */
static void l2_normalise(double *x, int d) {
  double ss = 0.0;
  for (int i = 0; i < d; ++i) ss += x[i] * x[i];
  double r = 1.0 / sqrt(ss + 1e-6);
  for (int i = 0; i < d; ++i) x[i] *= r;
}

static void run_chain(const gdpo_problem *p, int64_t seq, int h, double *S,
                      double *kap, double *e, double *qv) {
  const int K = p->K, V = p->V, n = p->n, Hv = p->Hv, Hqk = p->Hqk;
  const int hq = h / (Hv / Hqk);
  const int64_t t0 = p->cu[seq], t1 = p->cu[seq + 1];
  const size_t KV = (size_t)K * V;

  /* 1. starting state */
  if (p->s0)
    memcpy(S, p->s0 + ((size_t)seq * Hv + h) * KV, KV * sizeof(double));
  else
    memset(S, 0, KV * sizeof(double));

  for (int64_t t = t0; t < t1; ++t) {
    const int64_t rel = t - t0;
    /* 2.1 the state entering token chunk rel/64 */
    if (p->chunk_states && rel % GDPO_CHUNK == 0) {
      int64_t row = p->chunk_offsets[seq] + rel / GDPO_CHUNK;
      memcpy(p->chunk_states + ((size_t)row * Hv + h) * KV, S, KV * sizeof(double));
    }
    /* 2.2 decay once per real token, before its updates */
    const double alpha = exp(p->g_log[(size_t)t * Hv + h]);
    for (size_t x = 0; x < KV; ++x) S[x] *= alpha;

    /* 2.3 the n beta-gated Householder updates on rows t*n .. t*n+n-1 */
    for (int j = 0; j < n; ++j) {
      const int64_t r = t * n + j;
      memcpy(kap, p->k + ((size_t)r * Hqk + hq) * K, K * sizeof(double));
      if (p->l2norm) l2_normalise(kap, K);
      const double b = p->beta[(size_t)r * Hv + h];
      const double *vr = p->v + ((size_t)r * Hv + h) * V;
      for (int c = 0; c < V; ++c) e[c] = 0.0;
      for (int a = 0; a < K; ++a) {
        const double ka = kap[a];
        const double *Sa = S + (size_t)a * V;
        for (int c = 0; c < V; ++c) e[c] += Sa[c] * ka; /* (S^T k)[c] */
      }
      for (int c = 0; c < V; ++c) e[c] = b * (vr[c] - e[c]);
      if (p->vnew) memcpy(p->vnew + ((size_t)r * Hv + h) * V, e, V * sizeof(double));
      for (int a = 0; a < K; ++a) {
        const double ka = kap[a];
        double *Sa = S + (size_t)a * V;
        for (int c = 0; c < V; ++c) Sa[c] += ka * e[c]; /* S += k e^T */
      }
    }

    /* 2.4 readout after the last update */
    memcpy(qv, p->q + ((size_t)t * Hqk + hq) * K, K * sizeof(double));
    if (p->l2norm) l2_normalise(qv, K);
    double *ot = p->o + ((size_t)t * Hv + h) * V;
    for (int c = 0; c < V; ++c) e[c] = 0.0;
    for (int a = 0; a < K; ++a) {
      const double qa = qv[a];
      const double *Sa = S + (size_t)a * V;
      for (int c = 0; c < V; ++c) e[c] += Sa[c] * qa;
    }
    for (int c = 0; c < V; ++c) ot[c] = p->scale * e[c];
  }

  /* 3. final state and cache slot */
  if (p->final_state)
    memcpy(p->final_state + ((size_t)seq * Hv + h) * KV, S, KV * sizeof(double));
  if (p->cache && p->slots && p->slots[seq] >= 0)
    memcpy(p->cache + ((size_t)p->slots[seq] * Hv + h) * KV, S, KV * sizeof(double));
}

static void *worker(void *arg) {
  gdpo_problem *p = (gdpo_problem *)arg;
  const size_t KV = (size_t)p->K * p->V;
  double *S = (double *)malloc(KV * sizeof(double));
  double *kap = (double *)malloc((size_t)p->K * sizeof(double));
  double *qv = (double *)malloc((size_t)p->K * sizeof(double));
  double *e = (double *)malloc((size_t)p->V * sizeof(double));
  if (!S || !kap || !qv || !e) {
    free(S); free(kap); free(qv); free(e);
    return (void *)1;
  }
  for (;;) {
    pthread_mutex_lock(&p->mu);
    int64_t idx = p->next++;
    pthread_mutex_unlock(&p->mu);
    if (idx >= p->nchains) break;
    int64_t chain = p->order[idx];
    run_chain(p, chain / p->Hv, (int)(chain % p->Hv), S, kap, e, qv);
  }
  free(S); free(kap); free(qv); free(e);
  return NULL;
}

static const gdpo_problem *g_sort_problem;
static int by_length_desc(const void *a, const void *b) {
  const gdpo_problem *p = g_sort_problem;
  int64_t ca = *(const int64_t *)a, cb = *(const int64_t *)b;
  int64_t la = p->cu[ca / p->Hv + 1] - p->cu[ca / p->Hv];
  int64_t lb = p->cu[cb / p->Hv + 1] - p->cu[cb / p->Hv];
  if (la != lb) return la > lb ? -1 : 1;
  return ca < cb ? -1 : (ca > cb ? 1 : 0);
}

/*
 * Full forward pass.  All float arrays are contiguous fp64 in the layouts
 *   q [T, Hqk, K]   k [T*n, Hqk, K]   v [T*n, Hv, V]   g_log [T, Hv]
 *   beta [T*n, Hv]  cu_seqlens [N+1]  initial_state [N, Hv, K, V] (or NULL)
 *   o [T, Hv, V]    final_state [N, Hv, K, V] (or NULL)
 *   chunk_states [NT, Hv, K, V] with chunk_offsets [N+1] (both or neither)
 *   state_cache [num_slots, Hv, K, V] with state_indices [N] (both or neither)
 *   vnew [T*n, Hv, V] (or NULL): every e_r, for stage-level checks.
 * Returns 0, or -1 for invalid sizes, -2 when a thread could not start.
 */
int gdpo_prefill(int64_t T, int64_t N, int n, int Hqk, int Hv, int K, int V,
                 const double *q, const double *k, const double *v,
                 const double *g_log, const double *beta,
                 const int64_t *cu_seqlens, double scale,
                 const double *initial_state, int use_qk_l2norm, double *o,
                 double *final_state, double *chunk_states,
                 const int64_t *chunk_offsets, double *state_cache,
                 const int64_t *state_indices, int64_t num_slots, double *vnew,
                 int nthreads) {
  if (T < 0 || N < 0 || n < 1 || Hqk < 1 || Hv < 1 || K < 1 || V < 1) return -1;
  if (Hv % Hqk != 0) return -1;
  if (cu_seqlens[0] != 0 || cu_seqlens[N] != T) return -1;
  for (int64_t i = 0; i < N; ++i)
    if (cu_seqlens[i + 1] < cu_seqlens[i]) return -1;
  if ((chunk_states == NULL) != (chunk_offsets == NULL)) return -1;
  if ((state_cache == NULL) != (state_indices == NULL)) return -1;
  if (state_indices)
    for (int64_t i = 0; i < N; ++i)
      if (state_indices[i] < -1 || state_indices[i] >= num_slots) return -1;

  gdpo_problem p;
  memset(&p, 0, sizeof p);
  p.T = T; p.N = N; p.n = n; p.Hqk = Hqk; p.Hv = Hv; p.K = K; p.V = V;
  p.q = q; p.k = k; p.v = v; p.g_log = g_log; p.beta = beta;
  p.cu = cu_seqlens;
  p.scale = (scale == 0.0) ? 1.0 / sqrt((double)K) : scale;
  p.s0 = initial_state;
  p.l2norm = use_qk_l2norm;
  p.o = o; p.final_state = final_state;
  p.chunk_states = chunk_states; p.chunk_offsets = chunk_offsets;
  p.cache = state_cache; p.slots = state_indices;
  p.vnew = vnew;
  p.nchains = N * Hv;
  p.order = (int64_t *)malloc((size_t)(p.nchains > 0 ? p.nchains : 1) * sizeof(int64_t));
  if (!p.order) return -2;
  for (int64_t c = 0; c < p.nchains; ++c) p.order[c] = c;
  g_sort_problem = &p;
  qsort(p.order, (size_t)p.nchains, sizeof(int64_t), by_length_desc);
  pthread_mutex_init(&p.mu, NULL);

  if (nthreads < 1) nthreads = 1;
  if (nthreads > p.nchains) nthreads = (int)(p.nchains > 0 ? p.nchains : 1);
  int rc = 0;
  if (nthreads == 1) {
    if (worker(&p) != NULL) rc = -2;
  } else {
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    int started = 0;
    if (!th) rc = -2;
    for (int i = 0; th && i < nthreads; ++i) {
      if (pthread_create(&th[i], NULL, worker, &p) != 0) { rc = -2; break; }
      ++started;
    }
    for (int i = 0; i < started; ++i) {
      void *ret = NULL;
      pthread_join(th[i], &ret);
      if (ret != NULL) rc = -2;
    }
    free(th);
  }
  pthread_mutex_destroy(&p.mu);
  free(p.order);
  return rc;
}

/*
 * Chunk descriptors for both chunkings (Megatron Core page, the
 * chunk_indices / chunk_indices_dp / chunk_offsets arguments and the
 * two-chunkings paragraph): sequence i has ceil(L_i/64) token chunks and
 * ceil(n*L_i/64) expanded chunks.  Rows (i, c) are written sequence-major with
 * c ascending; rows past the real count up to the given capacity hold
 * (-1, -1).  Offsets are exclusive prefix sums of length N+1.
 * Returns 0, or -1 if a capacity is too small or cu_seqlens is not monotone.
 */
int gdpo_descriptors(const int64_t *cu_seqlens, int64_t N, int n,
                     int64_t nt_cap, int64_t ntdp_cap, int32_t *chunk_indices,
                     int32_t *chunk_indices_dp, int32_t *chunk_offsets,
                     int32_t *chunk_offsets_dp) {
  if (N < 0 || n < 1) return -1;
  int64_t nt = 0, ntdp = 0;
  for (int64_t i = 0; i < N; ++i) {
    int64_t L = cu_seqlens[i + 1] - cu_seqlens[i];
    if (L < 0) return -1;
    int64_t ct = (L + GDPO_CHUNK - 1) / GDPO_CHUNK;
    int64_t cd = (L * n + GDPO_CHUNK - 1) / GDPO_CHUNK;
    chunk_offsets[i] = (int32_t)nt;
    chunk_offsets_dp[i] = (int32_t)ntdp;
    if (nt + ct > nt_cap || ntdp + cd > ntdp_cap) return -1;
    for (int64_t c = 0; c < ct; ++c) {
      chunk_indices[2 * (nt + c)] = (int32_t)i;
      chunk_indices[2 * (nt + c) + 1] = (int32_t)c;
    }
    for (int64_t c = 0; c < cd; ++c) {
      chunk_indices_dp[2 * (ntdp + c)] = (int32_t)i;
      chunk_indices_dp[2 * (ntdp + c) + 1] = (int32_t)c;
    }
    nt += ct;
    ntdp += cd;
  }
  chunk_offsets[N] = (int32_t)nt;
  chunk_offsets_dp[N] = (int32_t)ntdp;
  for (int64_t r = nt; r < nt_cap; ++r) chunk_indices[2 * r] = chunk_indices[2 * r + 1] = -1;
  for (int64_t r = ntdp; r < ntdp_cap; ++r) chunk_indices_dp[2 * r] = chunk_indices_dp[2 * r + 1] = -1;
  return 0;
}
