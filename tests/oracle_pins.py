"""Pins for the fp64 oracle: checks against things other than the oracle itself.

Each pin takes an oracle shared library handle (the real one, or a build of
the oracle source with a planted mistake) and raises AssertionError when the
oracle disagrees with what the pages and the mathematics fix:

  * brute force on tiny inputs: the composition of the token's n Householder
    maps written as explicit matrix products (FlashInfer docs,
    "flashinfer.gdp_prefill.chunk_gated_delta_product", recurrence display);
  * closed forms: one token with n = 2 from a zero state; beta = 0 (pure
    decay); alpha = 1, beta = 0 (a plain GEMM readout);
  * invariants: n = 1 equals the gated delta rule of the blog page's GDN
    section; n copies equal n = 1 on the expanded stream with the decay
    interleaved as [g, 0, ..., 0] (Megatron Core page, stage 1); orthonormal
    keys with beta = 1 are recalled exactly; beta = 2 with unit keys is an
    orthogonal reflection; splitting a sequence and resuming from the final
    state matches the unsplit run (blog page, "GDN: pass the state, not the
    KV"); packed sequences equal separate runs; grouped q/k heads equal
    repeat-interleaved heads; chunk_states row c equals the final state of
    the run cut after 64*c tokens (Megatron Core page, return_chunk_states);
    cache slots receive final states and -1 writes nothing (Megatron Core
    page, state / state_indices); the in-kernel L2 norm is invariant to
    positive row scaling; scale None/0 means K^-1/2 (FlashInfer page, scale);
  * the single-token decode step on the state cache: brute force per entry
    (padding entries untouched), and T decode steps equal a T-token prefill.
"""
import numpy as np

import oracle

RNG_SEED = 12345


def _unit_rows(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def make_problem(rng, lens, n, Hqk, Hv, K, V, init=True, unit_qk=True):
    lens = list(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T = int(cu[-1])
    N = len(lens)
    q = rng.standard_normal((T, Hqk, K))
    k = rng.standard_normal((T * n, Hqk, K))
    if unit_qk:
        q = _unit_rows(q)
        k = _unit_rows(k)
    v = rng.standard_normal((T * n, Hv, V))
    g = -np.log1p(np.exp(rng.standard_normal((T, Hv))))  # -softplus, alpha in (0,1)
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T * n, Hv))))
    s0 = 0.3 * rng.standard_normal((N, Hv, K, V)) if init else None
    return dict(q=q, k=k, v=v, g_log=g, beta=beta, num_householder=n, cu_seqlens=cu,
                initial_state=s0)


def brute_force(q, k, v, g_log, beta, num_householder, cu_seqlens, scale=None,
                initial_state=None, use_qk_l2norm=False):
    """Per token: S_t = H_{n-1}..H_0 (alpha_t S_{t-1}) + sum_j H_{n-1}..H_{j+1} beta_j k_j v_j^T,
    with H_j = I - beta_j k_j k_j^T, then o_t = scale * S_t^T q_t.  Explicit matrices."""
    n = num_householder
    T, Hqk, K = q.shape
    Hv, V = v.shape[1], v.shape[2]
    N = len(cu_seqlens) - 1
    sc = 1.0 / np.sqrt(K) if not scale else scale
    o = np.zeros((T, Hv, V))
    fin = np.zeros((N, Hv, K, V))
    grp = Hv // Hqk
    for i in range(N):
        for h in range(Hv):
            hq = h // grp
            S = np.zeros((K, V)) if initial_state is None else initial_state[i, h].copy()
            for t in range(cu_seqlens[i], cu_seqlens[i + 1]):
                ks = [k[t * n + j, hq].copy() for j in range(n)]
                qt = q[t, hq].copy()
                if use_qk_l2norm:
                    ks = [x / np.sqrt(x @ x + 1e-6) for x in ks]
                    qt = qt / np.sqrt(qt @ qt + 1e-6)
                bs = [beta[t * n + j, h] for j in range(n)]
                Hs = [np.eye(K) - bs[j] * np.outer(ks[j], ks[j]) for j in range(n)]
                M = np.eye(K)
                for j in range(n):
                    M = Hs[j] @ M
                Snew = M @ (np.exp(g_log[t, h]) * S)
                for j in range(n):
                    P = np.eye(K)
                    for jj in range(j + 1, n):
                        P = Hs[jj] @ P
                    Snew = Snew + P @ (bs[j] * np.outer(ks[j], v[t * n + j, h]))
                S = Snew
                o[t, h] = sc * (S.T @ qt)
            fin[i, h] = S
    return o, fin


def gated_delta_rule_p1(q, k, v, g_log, beta, S0, scale):
    """The blog page's single-token GDN recurrence (one sequence, one head):
    Sbar = lambda S; vhat = Sbar^T k; e = beta (v - vhat); S = Sbar + k e^T; r = q^T S."""
    S = S0.copy()
    out = []
    for t in range(q.shape[0]):
        Sbar = np.exp(g_log[t]) * S
        vhat = Sbar.T @ k[t]
        e = beta[t] * (v[t] - vhat)
        S = Sbar + np.outer(k[t], e)
        out.append(scale * (q[t] @ S))
    return np.array(out), S


def _close(a, b, tol=1e-11, what=""):
    a = np.asarray(a); b = np.asarray(b)
    err = np.max(np.abs(a - b)) / max(1.0, np.sqrt(np.mean(b * b))) if a.size else 0.0
    assert err <= tol, f"{what}: err {err:.3e} > {tol:.1e}"


def _run(lib, prob, **kw):
    args = dict(prob)
    args.update(kw)
    return oracle.prefill(lib=lib, threads=2, **args)


# ---------------------------------------------------------------- pins

def pin_brute_force(lib):
    rng = np.random.default_rng(RNG_SEED)
    cases = [((3,), 1, 1, 1, 4, 3), ((2, 4, 1), 2, 1, 2, 5, 3), ((4, 3), 3, 2, 2, 3, 5),
             ((1, 4), 2, 2, 4, 4, 2)]
    for lens, n, Hqk, Hv, K, V in cases:
        for l2 in (False, True):
            prob = make_problem(rng, lens, n, Hqk, Hv, K, V, unit_qk=not l2)
            ref_o, ref_s = brute_force(use_qk_l2norm=l2, scale=0.7, **prob)
            out = _run(lib, prob, scale=0.7, use_qk_l2norm=l2)
            _close(out["o"], ref_o, what=f"o {lens} n={n} l2={l2}")
            _close(out["final_state"], ref_s, what=f"S {lens} n={n} l2={l2}")


def pin_one_token_closed_form(lib):
    """One token, zero state, n = 2: S = beta0 (I - beta1 k1 k1^T) k0 v0^T + beta1 k1 v1^T."""
    rng = np.random.default_rng(RNG_SEED + 1)
    K, V = 4, 3
    k = _unit_rows(rng.standard_normal((2, 1, K)))
    v = rng.standard_normal((2, 1, V))
    q = rng.standard_normal((1, 1, K))
    beta = np.array([[0.3], [0.8]])
    g = np.array([[-0.4]])
    k0, k1 = k[0, 0], k[1, 0]
    S = beta[0, 0] * (np.eye(K) - beta[1, 0] * np.outer(k1, k1)) @ np.outer(k0, v[0, 0]) \
        + beta[1, 0] * np.outer(k1, v[1, 0])
    o = 0.5 * S.T @ q[0, 0]
    out = oracle.prefill(q, k, v, g, beta, 2, [0, 1], scale=0.5, lib=lib, threads=1)
    _close(out["final_state"][0, 0], S, what="one-token state")
    _close(out["o"][0, 0], o, what="one-token output")


def pin_n1_is_gated_delta_rule(lib):
    rng = np.random.default_rng(RNG_SEED + 2)
    prob = make_problem(rng, (9,), 1, 1, 1, 6, 4)
    out = _run(lib, prob, scale=0.9)
    ref_o, ref_s = gated_delta_rule_p1(prob["q"][:, 0], prob["k"][:, 0], prob["v"][:, 0],
                                       prob["g_log"][:, 0], prob["beta"][:, 0],
                                       prob["initial_state"][0, 0], 0.9)
    _close(out["o"][:, 0], ref_o, what="n=1 output")
    _close(out["final_state"][0, 0], ref_s, what="n=1 state")


def pin_expansion_equivalence(lib):
    """n copies == n=1 on the expanded stream with decays [g_t, 0, .., 0], read at t*n+n-1."""
    rng = np.random.default_rng(RNG_SEED + 3)
    for n in (2, 3):
        prob = make_problem(rng, (5, 3), n, 1, 2, 4, 4)
        out = _run(lib, prob, scale=0.6)
        T = prob["q"].shape[0]
        gx = np.zeros((T * n, 2))
        gx[::n] = prob["g_log"]
        qx = np.repeat(prob["q"], n, axis=0)
        ex = dict(prob, q=qx, g_log=gx, num_householder=1, cu_seqlens=prob["cu_seqlens"] * n)
        outx = _run(lib, ex, scale=0.6)
        _close(out["o"], outx["o"][n - 1::n], what=f"expanded outputs n={n}")
        _close(out["final_state"], outx["final_state"], what=f"expanded state n={n}")


def pin_beta_zero_pure_decay(lib):
    rng = np.random.default_rng(RNG_SEED + 4)
    prob = make_problem(rng, (6,), 2, 1, 1, 3, 5)
    prob["beta"] = np.zeros_like(prob["beta"])
    out = _run(lib, prob, scale=1.3)
    G = np.cumsum(prob["g_log"][:, 0])
    S0 = prob["initial_state"][0, 0]
    ref_o = 1.3 * np.exp(G)[:, None] * (prob["q"][:, 0] @ S0)
    _close(out["o"][:, 0], ref_o, what="beta=0 outputs")
    _close(out["final_state"][0, 0], np.exp(G[-1]) * S0, what="beta=0 state")


def pin_identity_gate_plain_gemm(lib):
    rng = np.random.default_rng(RNG_SEED + 5)
    prob = make_problem(rng, (5,), 1, 1, 1, 4, 6, unit_qk=False)
    prob["beta"] = np.zeros_like(prob["beta"])
    prob["g_log"] = np.zeros_like(prob["g_log"])
    out = _run(lib, prob, scale=0.25)
    ref = 0.25 * prob["q"][:, 0] @ prob["initial_state"][0, 0]
    _close(out["o"][:, 0], ref, what="alpha=1 beta=0 GEMM")


def pin_orthonormal_recall(lib):
    """alpha = 1, beta = 1, orthonormal keys: S^T k_j = v_j for every key written."""
    rng = np.random.default_rng(RNG_SEED + 6)
    K, V, n = 6, 3, 2
    Qm, _ = np.linalg.qr(rng.standard_normal((K, K)))
    keys = Qm.T[:6]  # 6 orthonormal rows
    T = 3
    k = keys.reshape(T * n, 1, K)
    v = rng.standard_normal((T * n, 1, V))
    q = rng.standard_normal((T, 1, K))
    out = oracle.prefill(q, k, v, np.zeros((T, 1)), np.ones((T * n, 1)), n, [0, T],
                         initial_state=rng.standard_normal((1, 1, K, V)), lib=lib, threads=1)
    S = out["final_state"][0, 0]
    _close(keys @ S, v[:, 0], tol=1e-12, what="orthonormal recall")


def pin_reflection(lib):
    """alpha = 1, beta = 2, unit key, v = 0: S <- (I - 2kk^T) S, orthogonal; twice restores."""
    rng = np.random.default_rng(RNG_SEED + 7)
    K, V = 5, 4
    kk = _unit_rows(rng.standard_normal(K))
    S0 = rng.standard_normal((1, 1, K, V))
    k = np.stack([kk, kk]).reshape(2, 1, K)
    z = np.zeros((2, 1, V))
    one = oracle.prefill(np.ones((1, 1, K)), k[:1], z[:1], np.zeros((1, 1)), np.full((1, 1), 2.0),
                         1, [0, 1], initial_state=S0, lib=lib, threads=1)
    S1 = one["final_state"][0, 0]
    _close(np.linalg.norm(S1), np.linalg.norm(S0), tol=1e-12, what="reflection norm")
    two = oracle.prefill(np.ones((1, 1, K)), k, z, np.zeros((1, 1)), np.full((2, 1), 2.0),
                         2, [0, 1], initial_state=S0, lib=lib, threads=1)
    _close(two["final_state"], S0, tol=1e-12, what="double reflection")


def pin_split_resume(lib):
    rng = np.random.default_rng(RNG_SEED + 8)
    n, L, L1 = 2, 150, 70
    prob = make_problem(rng, (L,), n, 2, 4, 5, 3)
    full = _run(lib, prob, scale=0.5)
    a = dict(prob, q=prob["q"][:L1], k=prob["k"][:L1 * n], v=prob["v"][:L1 * n],
             g_log=prob["g_log"][:L1], beta=prob["beta"][:L1 * n], cu_seqlens=[0, L1])
    ra = _run(lib, a, scale=0.5)
    b = dict(prob, q=prob["q"][L1:], k=prob["k"][L1 * n:], v=prob["v"][L1 * n:],
             g_log=prob["g_log"][L1:], beta=prob["beta"][L1 * n:], cu_seqlens=[0, L - L1],
             initial_state=ra["final_state"])
    rb = _run(lib, b, scale=0.5)
    _close(np.concatenate([ra["o"], rb["o"]]), full["o"], what="split outputs")
    _close(rb["final_state"], full["final_state"], what="split state")


def pin_varlen_independence(lib):
    rng = np.random.default_rng(RNG_SEED + 9)
    n = 3
    lens = (7, 0, 12, 1)
    prob = make_problem(rng, lens, n, 1, 2, 4, 4)
    packed = _run(lib, prob, scale=0.4)
    cu = prob["cu_seqlens"]
    for i in range(len(lens)):
        t0, t1 = cu[i], cu[i + 1]
        one = dict(prob, q=prob["q"][t0:t1], k=prob["k"][t0 * n:t1 * n], v=prob["v"][t0 * n:t1 * n],
                   g_log=prob["g_log"][t0:t1], beta=prob["beta"][t0 * n:t1 * n],
                   cu_seqlens=[0, t1 - t0], initial_state=prob["initial_state"][i:i + 1])
        r = _run(lib, one, scale=0.4)
        _close(packed["o"][t0:t1], r["o"], what=f"varlen seq {i} outputs")
        _close(packed["final_state"][i], r["final_state"][0], what=f"varlen seq {i} state")
    # a zero-length sequence leaves its initial state untouched
    _close(packed["final_state"][1], prob["initial_state"][1], tol=0.0, what="empty sequence")


def pin_gqa_repeat_interleave(lib):
    rng = np.random.default_rng(RNG_SEED + 10)
    prob = make_problem(rng, (5, 4), 2, 2, 6, 4, 3)
    grouped = _run(lib, prob, scale=0.8)
    rep = dict(prob, q=np.repeat(prob["q"], 3, axis=1), k=np.repeat(prob["k"], 3, axis=1))
    full = _run(lib, rep, scale=0.8)
    _close(grouped["o"], full["o"], tol=0.0, what="GQA outputs")
    _close(grouped["final_state"], full["final_state"], tol=0.0, what="GQA states")


def pin_linearity(lib):
    """For fixed k, beta, g the map (S0, V) -> (S, o) is linear; S does not depend on scale."""
    rng = np.random.default_rng(RNG_SEED + 11)
    p1 = make_problem(rng, (8,), 2, 1, 1, 4, 3)
    p2 = dict(p1, v=rng.standard_normal(p1["v"].shape),
              initial_state=rng.standard_normal(p1["initial_state"].shape))
    r1 = _run(lib, p1, scale=0.5)
    r2 = _run(lib, p2, scale=0.5)
    p3 = dict(p1, v=2.0 * p1["v"] - 3.0 * p2["v"],
              initial_state=2.0 * p1["initial_state"] - 3.0 * p2["initial_state"])
    r3 = _run(lib, p3, scale=0.5)
    _close(r3["o"], 2 * r1["o"] - 3 * r2["o"], what="linear outputs")
    _close(r3["final_state"], 2 * r1["final_state"] - 3 * r2["final_state"], what="linear states")
    r4 = _run(lib, p1, scale=1.7)
    _close(r4["final_state"], r1["final_state"], tol=0.0, what="state independent of scale")
    _close(r4["o"], r1["o"] * (1.7 / 0.5), what="output linear in scale")


def pin_default_scale(lib):
    rng = np.random.default_rng(RNG_SEED + 12)
    prob = make_problem(rng, (4,), 1, 1, 1, 9, 2)
    a = _run(lib, prob, scale=None)
    b = _run(lib, prob, scale=0.0)
    c = _run(lib, prob, scale=1.0 / 3.0)
    _close(a["o"], c["o"], what="scale None == K^-1/2")
    _close(b["o"], c["o"], what="scale 0.0 == K^-1/2")


def pin_chunk_states(lib):
    rng = np.random.default_rng(RNG_SEED + 13)
    n = 2
    lens = (130, 64, 1, 65)
    prob = make_problem(rng, lens, n, 1, 2, 3, 4)
    out = _run(lib, prob, scale=0.5, return_chunk_states=True)
    cu = prob["cu_seqlens"]
    offs = out["chunk_offsets"]
    cs = out["chunk_states"]
    assert cs.shape[0] == sum((L + 63) // 64 for L in lens)
    for i, L in enumerate(lens):
        nchunks = (L + 63) // 64
        assert offs[i + 1] - offs[i] == nchunks
        for c in range(nchunks):
            t0 = cu[i]
            cut = 64 * c
            sub = dict(prob, q=prob["q"][t0:t0 + cut], k=prob["k"][t0 * n:(t0 + cut) * n],
                       v=prob["v"][t0 * n:(t0 + cut) * n], g_log=prob["g_log"][t0:t0 + cut],
                       beta=prob["beta"][t0 * n:(t0 + cut) * n], cu_seqlens=[0, cut],
                       initial_state=prob["initial_state"][i:i + 1])
            r = _run(lib, sub, scale=0.5)
            _close(cs[offs[i] + c], r["final_state"][0], what=f"chunk state seq {i} c {c}")


def pin_state_cache(lib):
    rng = np.random.default_rng(RNG_SEED + 14)
    prob = make_problem(rng, (5, 3, 0, 4), 2, 1, 2, 3, 3)
    cache0 = rng.standard_normal((6, 2, 3, 3))
    slots = np.array([4, -1, 0, 2])
    out = _run(lib, prob, scale=0.5, state_cache=cache0, state_indices=slots)
    cache = out["state_cache"]
    for i, s in enumerate(slots):
        if s >= 0:
            _close(cache[s], out["final_state"][i], tol=0.0, what=f"slot {s}")
    for s in (1, 3, 5):
        assert np.array_equal(cache[s], cache0[s]), f"slot {s} must stay untouched"


def pin_l2norm_scale_invariance(lib):
    rng = np.random.default_rng(RNG_SEED + 15)
    prob = make_problem(rng, (6, 5), 2, 1, 2, 8, 3, unit_qk=False)
    a = _run(lib, prob, scale=0.5, use_qk_l2norm=True)
    sq = rng.uniform(0.5, 4.0, size=prob["q"].shape[:2] + (1,))
    sk = rng.uniform(0.5, 4.0, size=prob["k"].shape[:2] + (1,))
    b = _run(lib, dict(prob, q=prob["q"] * sq, k=prob["k"] * sk), scale=0.5, use_qk_l2norm=True)
    _close(b["o"], a["o"], tol=1e-6, what="l2norm invariance")
    # pre-normalised rows: in-kernel normalisation changes nothing beyond the epsilon
    un = dict(prob, q=_unit_rows(prob["q"]), k=_unit_rows(prob["k"]))
    c = _run(lib, un, scale=0.5, use_qk_l2norm=True)
    d = _run(lib, un, scale=0.5, use_qk_l2norm=False)
    _close(c["o"], d["o"], tol=1e-5, what="l2norm on unit rows")
    _close(c["o"], a["o"], tol=1e-5, what="l2norm equals host normalisation")


def pin_decay_before_update(lib):
    """Decay once per token before its updates (FlashInfer page): with one
    token, zero state and beta = 1, unit key: S = k v^T regardless of alpha."""
    K, V = 3, 2
    k = np.array([[[0.6, 0.8, 0.0]]])
    v = np.array([[[2.0, -1.0]]])
    out = oracle.prefill(np.array([[[1.0, 0.0, 0.0]]]), k, v, np.array([[-3.0]]),
                         np.ones((1, 1)), 1, [0, 1], lib=lib, threads=1)
    _close(out["final_state"][0, 0], np.outer(k[0, 0], v[0, 0]), tol=1e-15, what="decay order")


ALL_PINS = [
    pin_brute_force, pin_one_token_closed_form, pin_n1_is_gated_delta_rule,
    pin_expansion_equivalence, pin_beta_zero_pure_decay, pin_identity_gate_plain_gemm,
    pin_orthonormal_recall, pin_reflection, pin_split_resume, pin_varlen_independence,
    pin_gqa_repeat_interleave, pin_linearity, pin_default_scale, pin_chunk_states,
    pin_state_cache, pin_l2norm_scale_invariance, pin_decay_before_update,
]


def _decode_problem(rng, N, n, Hqk, Hv, K, V, S):
    q = _unit_rows(rng.standard_normal((N, Hqk, K)))
    k = _unit_rows(rng.standard_normal((N * n, Hqk, K)))
    v = rng.standard_normal((N * n, Hv, V))
    g = -np.log1p(np.exp(rng.standard_normal((N, Hv))))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((N * n, Hv))))
    cache = 0.3 * rng.standard_normal((S, Hv, K, V))
    return q, k, v, g, beta, cache


def pin_decode_brute_force(lib):
    """Each entry's step is the explicit Householder product applied to its cache row;
    padding entries (-1) leave o zero and the cache untouched."""
    rng = np.random.default_rng(RNG_SEED + 40)
    N, n, Hqk, Hv, K, V, S = 5, 3, 1, 2, 4, 3, 7
    q, k, v, g, beta, cache = _decode_problem(rng, N, n, Hqk, Hv, K, V, S)
    slots = np.array([4, -1, 0, 6, -1])
    res = oracle.decode(q, k, v, g, beta, n, cache, slots, lib=lib)
    want_cache = cache.copy()
    for i in range(N):
        if slots[i] < 0:
            _close(res["o"][i], np.zeros((Hv, V)), what="padding output")
            continue
        rows = np.arange(i * n, (i + 1) * n)
        bo, bfin = brute_force(q[i:i + 1], k[rows], v[rows], g[i:i + 1], beta[rows], n, np.array([0, 1]),
                               initial_state=cache[slots[i]][None])
        _close(res["o"][i], bo[0], what=f"decode o[{i}]")
        want_cache[slots[i]] = bfin[0]
    _close(res["state_cache"], want_cache, what="decode cache")


def pin_decode_steps_equal_prefill(lib):
    """T decode steps of N sequences, each on its own slot, equal the prefill of the
    T-token sequences started from those slots."""
    rng = np.random.default_rng(RNG_SEED + 41)
    N, T, n, Hqk, Hv, K, V, S = 3, 5, 2, 1, 2, 4, 3, 4
    prob = make_problem(rng, [T] * N, n, Hqk, Hv, K, V, init=False)
    cache = 0.3 * rng.standard_normal((S, Hv, K, V))
    slots = np.array([2, 0, 3])
    ref = oracle.prefill(prob["q"], prob["k"], prob["v"], prob["g_log"], prob["beta"], n, prob["cu_seqlens"],
                         initial_state=cache[slots], lib=lib)
    cur = cache.copy()
    for t in range(T):
        tok = np.arange(N) * T + t  # token t of every sequence
        rows = (tok[:, None] * n + np.arange(n)[None, :]).reshape(-1)
        step = oracle.decode(prob["q"][tok], prob["k"][rows], prob["v"][rows], prob["g_log"][tok],
                             prob["beta"][rows], n, cur, slots, lib=lib)
        _close(step["o"], ref["o"][tok], what=f"decode step {t}")
        cur = step["state_cache"]
    _close(cur[slots], ref["final_state"], what="decode final states")
    untouched = [s for s in range(S) if s not in slots]
    _close(cur[untouched], cache[untouched], what="untouched slots")

ALL_PINS += [pin_decode_brute_force, pin_decode_steps_equal_prefill]


def flashinfer_literal(q, k, v, alpha, beta, n, cu, scale=None, init=None, l2norm=False):
    """The FlashInfer recurrence display taken literally, per (sequence, head), on a
    V-major state S [V, K]: S *= alpha_t; for each j, v_new = beta (v - S k),
    S += v_new (x) k; o_t = scale S q_t.  k has Hq or Hv heads; alpha/beta None
    mean ones."""
    T, Hq, d = q.shape
    Hk, Hv = k.shape[1], v.shape[1]
    sc = 1.0 / np.sqrt(d) if not scale else scale
    o = np.zeros((T, Hv, d))
    fin = np.zeros((len(cu) - 1, Hv, d, d))
    for i in range(len(cu) - 1):
        for h in range(Hv):
            hq, hk = h // (Hv // Hq), h // (Hv // Hk)
            S = np.zeros((d, d)) if init is None else init[i, h].copy()
            for t in range(cu[i], cu[i + 1]):
                S = (1.0 if alpha is None else alpha[t, h]) * S
                for j in range(n):
                    kv = k[t * n + j, hk].copy()
                    if l2norm:
                        kv = kv / np.sqrt(kv @ kv + 1e-6)
                    b = 1.0 if beta is None else beta[t * n + j, h]
                    vnew = b * (v[t * n + j, h] - S @ kv)
                    S = S + np.outer(vnew, kv)
                qt = q[t, hq].copy()
                if l2norm:
                    qt = qt / np.sqrt(qt @ qt + 1e-6)
                o[t, h] = sc * (S @ qt)
            fin[i, h] = S
    return o, fin


def pin_flashinfer_literal(lib):
    """The FlashInfer-convention front end (linear alpha, V-major states, None
    gates, k with one head per state head) against the page's recurrence display
    written out literally."""
    rng = np.random.default_rng(23)
    cu = [0, 3, 5]
    for (Hq, Hk, Hv, n, with_gates, l2) in [(1, 2, 2, 2, True, False), (2, 2, 4, 3, False, True),
                                            (2, 4, 4, 1, True, True)]:
        T, d = cu[-1], 4
        q = rng.standard_normal((T, Hq, d)); k = rng.standard_normal((T * n, Hk, d))
        if not l2:
            k /= np.linalg.norm(k, axis=-1, keepdims=True)
        v = rng.standard_normal((T * n, Hv, d))
        alpha = rng.uniform(0.3, 1.0, (T, Hv)) if with_gates else None
        beta = rng.uniform(0.1, 0.9, (T * n, Hv)) if with_gates else None
        init = rng.standard_normal((2, Hv, d, d)) * 0.3 if with_gates else None
        ro, rf = flashinfer_literal(q, k, v, alpha, beta, n, cu, scale=0.7, init=init, l2norm=l2)
        res = oracle.prefill_flashinfer(q, k, v, alpha, beta, n, scale=0.7, initial_state=init,
                                        output_final_state=True, cu_seqlens=np.array(cu), use_qk_l2norm_in_kernel=l2,
                                        lib=lib)
        _close(res["o"], ro, what=f"o Hq={Hq} Hk={Hk} Hv={Hv}")
        _close(res["final_state"], rf, what=f"S Hq={Hq} Hk={Hk} Hv={Hv}")


ALL_PINS += [pin_flashinfer_literal]


# ---------------------------------------------------------------- backward oracle

def pin_backward_forward_matches_c_oracle(lib):
    """The autograd token loop's forward equals the C oracle (GQA, l2norm, n=3)."""
    from oracle import backward as ob
    import torch
    rng = np.random.default_rng(31)
    for l2 in (False, True):
        prob = make_problem(rng, (3, 1, 4), 3, 1, 2, 5, 3, unit_qk=not l2)
        o, fin = ob.forward_torch(*[torch.tensor(prob[x]) for x in ("q", "k", "v", "g_log", "beta")], 3,
                                  prob["cu_seqlens"], scale=0.7,
                                  initial_state=torch.tensor(prob["initial_state"]), use_qk_l2norm=l2)
        out = _run(lib, prob, scale=0.7, use_qk_l2norm=l2)
        _close(o.numpy(), out["o"], what=f"o l2={l2}")
        _close(fin.numpy(), out["final_state"], what=f"S l2={l2}")


def pin_backward_finite_differences(lib):
    """Every gradient of the backward oracle against central differences of the
    C oracle's forward on a tiny problem (k with one head per state head)."""
    from oracle import backward as ob
    rng = np.random.default_rng(37)
    lens, n, Hq, Hk, Hv, K, V = (2, 3), 2, 1, 2, 2, 3, 2
    T, N = sum(lens), len(lens)
    cu = np.concatenate([[0], np.cumsum(lens)])
    q = rng.standard_normal((T, Hq, K)); k = rng.standard_normal((T * n, Hk, K))
    v = rng.standard_normal((T * n, Hv, V)); g = -rng.uniform(0.05, 0.7, (T, Hv))
    b = rng.uniform(0.2, 0.9, (T * n, Hv)); s0 = 0.5 * rng.standard_normal((N, Hv, K, V))
    do = rng.standard_normal((T, Hv, V)); dfin = rng.standard_normal((N, Hv, K, V))
    for l2 in (False, True):
        grads = ob.backward(q, k, v, g, b, n, cu, do, dfin, scale=0.6, initial_state=s0, use_qk_l2norm=l2)

        def loss(q_, k_, v_, g_, b_, s0_):
            # the C oracle reads q and k through one head index: give it q per k head
            out = oracle.prefill(np.repeat(q_, Hk // Hq, axis=1), k_, v_, g_, b_, n, cu, scale=0.6,
                                 initial_state=s0_, use_qk_l2norm=l2, lib=lib)
            return float(np.sum(out["o"] * do) + np.sum(out["final_state"] * dfin))

        base = [q, k, v, g, b, s0]
        for idx, name in enumerate(["dq", "dk", "dv", "dg_log", "dbeta", "dinitial_state"]):
            x = base[idx]
            num = np.zeros_like(x)
            h = 1e-6
            for pos in np.ndindex(*x.shape):
                xp = x.copy(); xp[pos] += h
                xm = x.copy(); xm[pos] -= h
                args_p = list(base); args_p[idx] = xp
                args_m = list(base); args_m[idx] = xm
                num[pos] = (loss(*args_p) - loss(*args_m)) / (2 * h)
            _close(grads[name], num, tol=1e-6, what=f"{name} l2={l2}")


ALL_PINS += [pin_backward_forward_matches_c_oracle, pin_backward_finite_differences]
