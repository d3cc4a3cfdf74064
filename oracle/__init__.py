"""fp64 CPU oracle for chunked Gated DeltaProduct prefill.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The library path never imports this
package, and this package imports nothing from the library.

The arithmetic lives in ``gdp_oracle.c`` (a plain token-by-token recurrence,
FlashInfer docs "flashinfer.gdp_prefill.chunk_gated_delta_product", the
recurrence display); this module only marshals numpy arrays into it.  The
single-token decode step is that same recurrence on one-token sequences whose
states come from, and go back to, the state cache.

Every function here is pinned by ``tests/test_oracle_pins.py`` against
brute-force Householder products, closed forms and invariants.
"""
import ctypes
import math
import os

import numpy as np

from . import build as _build

_LIB = None


def _lib():
    """The oracle library: GDP_ORACLE_LIBRARY names another build of it (the
    sanitized one of the CPU sanitizer run); otherwise the in-tree build."""
    global _LIB
    if _LIB is None:
        path = os.environ.get("GDP_ORACLE_LIBRARY")
        if not path:
            path = _build.LIB
            if not os.path.exists(path):
                _build.compile_oracle()
        _LIB = load(path)
    return _LIB


def load(path):
    """Load an oracle shared library (the real one or a test-built variant)."""
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    i64p = ctypes.POINTER(ctypes.c_int64)
    i32p = ctypes.POINTER(ctypes.c_int32)
    lib.gdpo_prefill.restype = ctypes.c_int
    lib.gdpo_prefill.argtypes = [
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_int, ctypes.c_int,
        dp, dp, dp, dp, dp, i64p, ctypes.c_double, dp, ctypes.c_int, dp, dp, dp,
        i64p, dp, i64p, ctypes.c_int64, dp, ctypes.c_int]
    lib.gdpo_descriptors.restype = ctypes.c_int
    lib.gdpo_descriptors.argtypes = [i64p, ctypes.c_int64, ctypes.c_int, ctypes.c_int64,
                                     ctypes.c_int64, i32p, i32p, i32p, i32p]
    return lib


def _f64(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a, ctype=ctypes.c_double):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def default_threads():
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def descriptor_capacity(T, N, n):
    """Upper bounds on the token-stream and expanded-stream chunk counts
    that depend only on (T, N, n): sum ceil(L/64) <= floor((T + 63 N)/64)."""
    return (T + 63 * N) // 64, (n * T + 63 * N) // 64


def descriptors(cu_seqlens, n, nt_cap=None, ntdp_cap=None, lib=None):
    """Chunk descriptors of both chunkings (Megatron Core page, the
    chunk_indices / chunk_indices_dp / chunk_offsets arguments)."""
    lib = lib or _lib()
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    N = cu.shape[0] - 1
    T = int(cu[-1])
    cap_t, cap_d = descriptor_capacity(T, N, n)
    nt_cap = cap_t if nt_cap is None else nt_cap
    ntdp_cap = cap_d if ntdp_cap is None else ntdp_cap
    ci = np.zeros((max(nt_cap, 1), 2), np.int32)
    cid = np.zeros((max(ntdp_cap, 1), 2), np.int32)
    off = np.zeros(N + 1, np.int32)
    offd = np.zeros(N + 1, np.int32)
    rc = lib.gdpo_descriptors(_ptr(cu, ctypes.c_int64), N, n, nt_cap, ntdp_cap,
                              _ptr(ci, ctypes.c_int32), _ptr(cid, ctypes.c_int32),
                              _ptr(off, ctypes.c_int32), _ptr(offd, ctypes.c_int32))
    if rc != 0:
        raise ValueError("gdpo_descriptors rejected its arguments")
    return {"chunk_indices": ci[:nt_cap], "chunk_indices_dp": cid[:ntdp_cap],
            "chunk_offsets": off, "chunk_offsets_dp": offd}


def prefill(q, k, v, g_log, beta, num_householder, cu_seqlens, scale=None,
            initial_state=None, use_qk_l2norm=False, return_chunk_states=False,
            state_cache=None, state_indices=None, dump_vnew=False, threads=None,
            lib=None):
    """Run the fp64 token loop.

    Shapes (leading batch dim of 1 not accepted here):
      q [T, Hqk, K], k [T*n, Hqk, K], v [T*n, Hv, V], g_log [T, Hv] (log decays),
      beta [T*n, Hv], cu_seqlens [N+1], initial_state [N, Hv, K, V] or None,
      state_cache [S, Hv, K, V] (copied, then written at state_indices) or None.
    Returns a dict with o, final_state and, on request, chunk_states,
    chunk_offsets, state_cache and vnew (every e_r).
    """
    lib = lib or _lib()
    n = int(num_householder)
    q = _f64(q); k = _f64(k); v = _f64(v); g = _f64(g_log); b = _f64(beta)
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    T, Hqk, K = q.shape
    V = v.shape[2]
    Hv = v.shape[1]
    N = cu.shape[0] - 1
    if k.shape != (T * n, Hqk, K) or v.shape != (T * n, Hv, V):
        raise ValueError("k/v shapes do not match q and num_householder")
    if g.shape != (T, Hv) or b.shape != (T * n, Hv):
        raise ValueError("g_log/beta shapes")
    s0 = None if initial_state is None else _f64(initial_state)
    if s0 is not None and s0.shape != (N, Hv, K, V):
        raise ValueError("initial_state shape")
    o = np.zeros((T, Hv, V), np.float64)
    fin = np.zeros((N, Hv, K, V), np.float64)
    cs = offs = None
    if return_chunk_states:
        d = descriptors(cu, n, lib=lib)
        offs = d["chunk_offsets"].astype(np.int64)
        cs = np.zeros((int(offs[-1]), Hv, K, V), np.float64)
    cache = slots = None
    nslots = 0
    if state_cache is not None:
        cache = _f64(state_cache).copy()
        slots = np.ascontiguousarray(np.asarray(state_indices, dtype=np.int64))
        nslots = cache.shape[0]
    vn = np.zeros((T * n, Hv, V), np.float64) if dump_vnew else None
    sc = 0.0 if scale is None else float(scale)
    rc = lib.gdpo_prefill(T, N, n, Hqk, Hv, K, V, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                          _ptr(b), _ptr(cu, ctypes.c_int64), sc, _ptr(s0),
                          int(bool(use_qk_l2norm)), _ptr(o), _ptr(fin), _ptr(cs),
                          _ptr(offs, ctypes.c_int64), _ptr(cache),
                          _ptr(slots, ctypes.c_int64), nslots, _ptr(vn),
                          int(threads or default_threads()))
    if rc != 0:
        raise ValueError(f"gdpo_prefill failed with code {rc}")
    out = {"o": o, "final_state": fin,
           "scale": (1.0 / math.sqrt(K)) if sc == 0.0 else sc}
    if return_chunk_states:
        out["chunk_states"] = cs
        out["chunk_offsets"] = offs
    if cache is not None:
        out["state_cache"] = cache
    if vn is not None:
        out["vnew"] = vn
    return out


def decode(q, k, v, g_log, beta, num_householder, state_cache, state_indices, scale=None,
           use_qk_l2norm=False, threads=None, lib=None):
    """One recurrent step per sequence on the state cache, in place.

    The recurrent decode step of the blog page's GDN section (Sbar = lambda S,
    vhat = Sbar^T k, e = beta (v - vhat), S = Sbar + k e^T, r = q^T S), with the
    n Householder rows of the FlashInfer recurrence display, reading the state
    of sequence i from state_cache[state_indices[i]] and writing it back there
    (Megatron Core page, state / state_indices).  It is the prefill token loop
    run on one-token sequences whose initial states are the cache rows.
    A negative index marks a padding entry: its output row is zero and the
    cache is not touched.  Two entries may not name the same slot.

    Shapes: q [N, Hqk, K], k [N*n, Hqk, K], v [N*n, Hv, V], g_log [N, Hv],
    beta [N*n, Hv], state_cache [S, Hv, K, V], state_indices [N].
    Returns {"o": [N, Hv, V], "state_cache": the updated copy}.
    """
    n = int(num_householder)
    q = _f64(q); k = _f64(k); v = _f64(v); g = _f64(g_log); b = _f64(beta)
    cache = _f64(state_cache).copy()
    slots = np.asarray(state_indices, dtype=np.int64)
    N, Hqk, K = q.shape
    Hv, V = v.shape[1], v.shape[2]
    if k.shape != (N * n, Hqk, K) or v.shape != (N * n, Hv, V) or g.shape != (N, Hv) or b.shape != (N * n, Hv):
        raise ValueError("decode: shapes do not match q and num_householder")
    if slots.shape != (N,) or cache.shape[1:] != (Hv, K, V):
        raise ValueError("decode: state_indices / state_cache shapes")
    sel = np.nonzero((slots >= 0) & (slots < cache.shape[0]))[0]
    if len(set(slots[sel].tolist())) != len(sel):
        raise ValueError("decode: two entries name the same cache slot")
    o = np.zeros((N, Hv, V), np.float64)
    if sel.size:
        rows = (sel[:, None] * n + np.arange(n)[None, :]).reshape(-1)
        res = prefill(q[sel], k[rows], v[rows], g[sel], b[rows], n, np.arange(sel.size + 1), scale=scale,
                      initial_state=cache[slots[sel]], use_qk_l2norm=use_qk_l2norm, threads=threads, lib=lib)
        o[sel] = res["o"]
        cache[slots[sel]] = res["final_state"]
    return {"o": o, "state_cache": cache}


def prefill_flashinfer(q, k, v, g=None, beta=None, num_householder=1, scale=None, initial_state=None,
                       output_final_state=False, cu_seqlens=None, use_qk_l2norm_in_kernel=False,
                       threads=None, lib=None):
    """The prefill in the FlashInfer convention (FlashInfer docs,
    "flashinfer.gdp_prefill.chunk_gated_delta_product": recurrence display and
    parameter list), restated for the token loop above:
      - g is the decay alpha itself; the loop multiplies S by exp(g_log), so
        g_log = ln(alpha); g None means alpha = 1 (g_log = 0);
      - beta None means all ones;
      - k may carry one head per q head or one per v (state) head; with
        Hk = Hv != Hq the loop, which reads q and k through one head index, gets
        q with each head repeated for the Hv / Hq state heads that read it;
      - states are V-major [N, H, V, K] (entry [v][k] = S[k][v] of the loop).
    Shapes: q [T, Hq, d], k [T*n, Hk, d], v [T*n, Hv, d], g [T, Hv],
    beta [T*n, Hv], initial_state [N, Hv, d, d].  Returns {"o", "final_state"}
    with final_state V-major (None unless output_final_state)."""
    n = int(num_householder)
    q = _f64(q); k = _f64(k); v = _f64(v)
    T, Hq, d = q.shape
    Hk, Hv = k.shape[1], v.shape[1]
    if Hk not in (Hq, Hv) or Hv % Hq != 0:
        raise ValueError("k must have Hq or Hv heads, and Hv must be a multiple of Hq")
    if Hk == Hv and Hq != Hv:
        q = np.repeat(q, Hv // Hq, axis=1)
    g_log = np.zeros((T, Hv)) if g is None else np.log(_f64(g))
    b = np.ones((T * n, Hv)) if beta is None else _f64(beta)
    s0 = None if initial_state is None else np.ascontiguousarray(np.swapaxes(_f64(initial_state), 2, 3))
    res = prefill(q, k, v, g_log, b, n, cu_seqlens, scale=scale, initial_state=s0,
                  use_qk_l2norm=use_qk_l2norm_in_kernel, threads=threads, lib=lib)
    fin = np.ascontiguousarray(np.swapaxes(res["final_state"], 2, 3)) if output_final_state else None
    return {"o": res["o"], "final_state": fin}
