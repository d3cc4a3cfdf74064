"""HIP path vs the fp64 oracle, element by element, through the C ABI (needs a gfx950 GPU)."""
import numpy as np
import pytest
import torch

import oracle
from gated_deltaproduct_recurrence_amd import workloads
from tests.parity import TOL, ErrAcc, oracle_run, rel_err, to_device, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gdp():
    from gated_deltaproduct_recurrence_amd import binding
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return binding


# bf16 inputs have three kernel paths: the fused single kernel, the WY + scan
# pair, and the segmented path (fused kernel on segments of long sequences,
# K == V only).  Tests over bf16 inputs run each path forced through
# GDP_PREFILL_PATH.
PATHS = ["fused", "split", "segmented"]
# the fused kernel has two output forms for n = 2: per expanded chunk (the
# default) and per token chunk (the form every other n uses); "fused_tc" runs
# the second on the same inputs
FUSED_FORMS = PATHS + ["fused_tc"]


def set_path(monkeypatch, p):
    monkeypatch.setenv("GDP_PREFILL_PATH", "fused" if p == "fused_tc" else p)
    if p == "fused_tc":
        monkeypatch.setenv("GDP_FUSED_OUTPUTS", "token_chunk")
    else:
        monkeypatch.delenv("GDP_FUSED_OUTPUTS", raising=False)


@pytest.fixture(params=FUSED_FORMS)
def path(request, monkeypatch):
    set_path(monkeypatch, request.param)
    return request.param


def run_gpu(gdp, inp):
    args = dict(inp)
    res = gdp.chunk_prefill(**args)
    torch.cuda.synchronize()
    return res


def check_all(inp, res, ref, tol, what=""):
    o, fs = res[0], res[1]
    e = rel_err(to_np(o), ref["o"])
    assert e <= tol, f"{what} o err {e:.3e}"
    if fs is not None:
        e = rel_err(to_np(fs), ref["final_state"])
        assert e <= tol, f"{what} final_state err {e:.3e}"
    return e


# ---------------------------------------------------------------- descriptors

@pytest.mark.parametrize("lens,n", [([37, 64, 200, 511], 2), ([0, 1, 0, 64, 65, 3000, 0], 3),
                                    ([5] * 3000, 1), ([1] * 1500 + [700] * 20 + [0] * 10, 5)])
def test_descriptors_bitexact(gdp, lens, n):
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T = int(cu[-1])
    for dtype in (torch.int32, torch.int64):
        got = gdp.gdp_build_descriptors(torch.tensor(cu, dtype=dtype, device="cuda"), n, T)
        torch.cuda.synchronize()
        ref = oracle.descriptors(cu, n)
        for key in ("chunk_indices", "chunk_indices_dp", "chunk_offsets", "chunk_offsets_dp"):
            assert np.array_equal(got[key].cpu().numpy(), ref[key]), key


def test_descriptors_larger_capacity_padding(gdp):
    cu = np.array([0, 37, 101, 301, 812])
    got = gdp.gdp_build_descriptors(torch.tensor(cu, dtype=torch.int32, device="cuda"), 2, 812,
                                    nt_cap=40, ntdp_cap=50)
    ref = oracle.descriptors(cu, 2, nt_cap=40, ntdp_cap=50)
    assert np.array_equal(got["chunk_indices"].cpu().numpy(), ref["chunk_indices"])
    assert np.array_equal(got["chunk_indices_dp"].cpu().numpy(), ref["chunk_indices_dp"])


# ---------------------------------------------------------------- the five workloads

def test_workload0_fp32_full_parity(gdp):
    w = workloads.workload(0)
    inp = workloads.generate(w, "cpu")
    ref = oracle_run(inp)
    res = run_gpu(gdp, to_device(inp))
    check_all(inp, res, ref, TOL[w.dtype], what=w.name)


@pytest.mark.parametrize("wid", [1, 2])
def test_workload_full_parity(gdp, wid, path):
    w = workloads.workload(wid)
    inp = workloads.generate(w, "cpu")
    inp["output_final_state"] = True  # workload 2 is timed without it; parity checks it too
    ref = oracle_run(inp)
    res = run_gpu(gdp, to_device(inp))
    check_all(inp, res, ref, TOL[w.dtype], what=w.name)


def _serving_mix_run(gdp, inp, w, desc, cache0, sentinel):
    """One low-level call on the serving mix into a sentinel-filled chunk-state
    buffer and a fresh copy of the cache; returns (o, chunk_states, cache)."""
    T, N, n = w.T, w.N, w.n
    nt_cap, _ = gdp.gdp_descriptor_capacity(T, N, n)
    cs = torch.full((nt_cap, w.Hv, w.K, w.V), sentinel, dtype=torch.float32, device="cuda")
    cache = cache0.clone()
    o = torch.empty((T, w.Hv, w.V), dtype=w.dtype, device="cuda")
    ws = torch.empty(gdp.gdp_workspace_bytes(T, N, n, w.Hqk, w.Hv, w.K, w.V), dtype=torch.uint8, device="cuda")
    gdp.gdp_chunk_prefill(inp["q"], inp["k"], inp["v"], inp["g_log"], inp["beta"], n, inp["cu_seqlens"], 0.0, None,
                          False, False, cache, inp["state_indices"], True, o, None, cs, desc, ws)
    torch.cuda.synchronize()
    return o, cs, cache


def test_workload_serving_mix_every_head(gdp, monkeypatch):
    """Random-length mix (64 sequences + 4 zero-length padding sequences, n=3,
    H=32) with cache slots and chunk states, on every kernel path.  Every state
    head's o, chunk-state rows and written cache slots are compared with the
    oracle, which runs four heads at a time (the error's max and rms are taken
    over the whole tensor); the untouched slots and the padding chunk-state rows
    are bit-exact, and the descriptors' offsets equal the oracle's."""
    w = workloads.workload(3)
    cpu_inp = workloads.generate(w, "cpu")
    inp = to_device(cpu_inp)
    T, N, n = w.T, w.N, w.n
    desc = gdp.gdp_build_descriptors(inp["cu_seqlens"], n, T)
    sentinel = 12345.0
    cache0 = inp["state_cache"].clone()
    runs = {}
    for p in PATHS:
        monkeypatch.setenv("GDP_PREFILL_PATH", p)
        runs[p] = _serving_mix_run(gdp, inp, w, desc, cache0, sentinel)
        print(f"serving mix: {p} path ran", flush=True)
    offs = desc["chunk_offsets"].cpu().numpy()
    NT = int(offs[-1])
    slots = inp["state_indices"].cpu().numpy()
    written = [int(s) for s in slots if s >= 0]
    untouched = sorted(set(range(cache0.shape[0])) - set(written))
    for p, (o, cs, cache) in runs.items():
        assert torch.all(cs[NT:] == sentinel), f"{p}: padding chunk-state rows were written"
        assert torch.equal(cache[untouched], cache0[untouched]), f"{p}: untouched cache slots changed"
    acc = {(p, what): ErrAcc() for p in PATHS for what in ("o", "chunk_states", "cache")}
    for h0 in range(0, w.Hv, 4):
        heads = list(range(h0, h0 + 4))
        ref = oracle_run(cpu_inp, heads=heads)
        assert np.array_equal(offs, ref["chunk_offsets"])
        for p, (o, cs, cache) in runs.items():
            acc[p, "o"].add(to_np(o[:, heads]), ref["o"])
            acc[p, "chunk_states"].add(to_np(cs[:NT, heads]), ref["chunk_states"])
            acc[p, "cache"].add(to_np(cache[written][:, heads]), ref["state_cache"][written])
        del ref
        print(f"serving mix: heads {h0}..{h0 + 3} compared", flush=True)
    for (p, what), a in acc.items():
        assert a.err() <= TOL[w.dtype], f"{p}: {what} err {a.err():.3e}"


def test_workload_serving_mix_graph_replay(gdp):
    """The serving mix at its full size (T, N) as a captured graph: descriptor
    build plus prefill (cache slots, chunk states), captured once and replayed
    for three seeded length sets of the same T and N.  Every replay's o, chunk
    states and cache equal an eager call on the same lengths bit for bit."""
    w = workloads.workload(3)
    inp = workloads.generate(w, "cuda")
    T, N, n = w.T, w.N, w.n
    nt_cap, ntdp_cap = gdp.gdp_descriptor_capacity(T, N, n)
    cu = inp["cu_seqlens"].clone()
    desc = {"chunk_indices": torch.empty((nt_cap, 2), dtype=torch.int32, device="cuda"),
            "chunk_indices_dp": torch.empty((ntdp_cap, 2), dtype=torch.int32, device="cuda"),
            "chunk_offsets": torch.empty(N + 1, dtype=torch.int32, device="cuda"),
            "chunk_offsets_dp": torch.empty(N + 1, dtype=torch.int32, device="cuda")}
    o = torch.empty((T, w.Hv, w.V), dtype=w.dtype, device="cuda")
    cs = torch.zeros((nt_cap, w.Hv, w.K, w.V), dtype=torch.float32, device="cuda")
    cache = inp["state_cache"]
    ws = torch.empty(gdp.gdp_workspace_bytes(T, N, n, w.Hqk, w.Hv, w.K, w.V), dtype=torch.uint8, device="cuda")

    def call():
        gdp.gdp_build_descriptors(cu, n, T, out=desc)
        gdp.gdp_chunk_prefill(inp["q"], inp["k"], inp["v"], inp["g_log"], inp["beta"], n, cu, 0.0, None, False,
                              False, cache, inp["state_indices"], True, o, None, cs, desc, ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    lens0 = list(w.lens)
    rng = np.random.default_rng(33)
    lens1 = [lens0[i] for i in rng.permutation(len(lens0))]
    lens2 = list(lens1)
    for i in range(0, len(lens2) - 1, 2):  # move tokens between neighbours, T unchanged
        m = int(rng.integers(0, lens2[i] + 1))
        lens2[i] -= m
        lens2[i + 1] += m
    for lens in (lens0, lens1, lens2):
        assert sum(lens) == T
        full = lens + [0] * w.pad_sequences
        cu.copy_(torch.tensor([0] + [int(x) for x in np.cumsum(full)], dtype=torch.int32, device="cuda"))
        cs.zero_()
        graph.replay()
        torch.cuda.synchronize()
        ro, rcs, rcache = o.clone(), cs.clone(), cache.clone()
        cs.zero_()
        call()
        torch.cuda.synchronize()
        assert torch.equal(ro, o), "replayed o differs from eager"
        assert torch.equal(rcs, cs), "replayed chunk states differ from eager"
        assert torch.equal(rcache, cache), "replayed cache differs from eager"
        assert torch.isfinite(o.float()).all()


def test_workload_long_context_every_chain(gdp):
    """Full-size long-context run (8 x 65536 tokens, n=2, Hqk=16 / Hv=32) in the
    benchmark's launch configuration.  The oracle runs one sequence and eight q/k
    heads (sixteen state heads) at a time; every output and every chain's final
    state is compared, with the error's max and rms over the whole tensor."""
    w = workloads.workload(4)
    inp = workloads.generate(w, "cuda")
    o, fs = gdp.chunk_prefill(**inp)
    torch.cuda.synchronize()
    cu = inp["cu_seqlens"].cpu().numpy()
    n, grp, half = w.n, w.Hv // w.Hqk, w.Hqk // 2
    acc_o, acc_s = ErrAcc(), ErrAcc()
    for seq in range(w.N):
        t0, t1 = int(cu[seq]), int(cu[seq + 1])
        for g0 in (0, half):
            qk = slice(g0, g0 + half)
            heads = slice(grp * g0, grp * (g0 + half))
            sub = dict(q=inp["q"][t0:t1, qk], k=inp["k"][t0 * n:t1 * n, qk], v=inp["v"][t0 * n:t1 * n, heads],
                       g_log=inp["g_log"][t0:t1, heads], beta=inp["beta"][t0 * n:t1 * n, heads], num_householder=n,
                       cu_seqlens=torch.tensor([0, t1 - t0]), scale=None,
                       initial_state=inp["initial_state"][seq:seq + 1, heads], use_qk_l2norm=True)
            ref = oracle_run(sub)
            acc_o.add(to_np(o[t0:t1, heads]), ref["o"])
            acc_s.add(to_np(fs[seq:seq + 1, heads]), ref["final_state"])
            del ref, sub
        print(f"long context: sequence {seq} compared (o err so far {acc_o.err():.3e})", flush=True)
    assert acc_o.err() <= TOL[w.dtype], f"o err {acc_o.err():.3e}"
    assert acc_s.err() <= TOL[w.dtype], f"final_state err {acc_s.err():.3e}"


# ---------------------------------------------------------------- strong decays and non-finite inputs

STRONG = [
    # lens, n, Hqk, Hv, K, V, dtype, l2norm
    ([700, 300, 77], 2, 2, 4, 128, 128, torch.bfloat16, True),
    ([400, 129], 3, 1, 2, 128, 128, torch.bfloat16, False),
    ([130, 70], 2, 1, 2, 64, 64, torch.float32, False),
]
STRONG_PATHS = [(i, p) for i, c in enumerate(STRONG) for p in (FUSED_FORMS if c[6] == torch.bfloat16 else ["auto"])]


def strong_decay_inputs(ci):
    """g_log = -softplus(N(0,1) + 2) (alpha about 0.12) with 2% of the (token,
    head) entries at -40: the allowed range of the gate (alpha in (0, 1]) taken
    to where a 64-token chunk's decay sum underflows exp2."""
    lens, n, Hqk, Hv, K, V, dt, l2 = STRONG[ci]
    w = workloads.custom(lens, n, Hqk, Hv, K, V, dtype=dt, l2norm_in_kernel=l2, g_shift=-2.0, init_std=0.2,
                         seed=90 + ci)
    inp = workloads.generate(w, "cpu")
    hit = torch.rand(inp["g_log"].shape, generator=torch.Generator().manual_seed(190 + ci)) < 0.02
    inp["g_log"][hit] = -40.0
    inp["return_chunk_states"] = True
    return w, inp


def min_chunk_decay_sum_base2(g_log, cu):
    """Smallest base-2 decay sum over the 64-token chunks of every sequence and head."""
    g = g_log.double().numpy() * np.log2(np.e)
    best = 0.0
    for i in range(len(cu) - 1):
        for c0 in range(int(cu[i]), int(cu[i + 1]), 64):
            best = min(best, float(g[c0:min(c0 + 64, int(cu[i + 1]))].sum(0).min()))
    return best


@pytest.mark.parametrize("ci,kpath", STRONG_PATHS, ids=[f"strong{i}-{p}" for i, p in STRONG_PATHS])
def test_strong_decay_parity(gdp, ci, kpath, monkeypatch):
    """Strong decays against the oracle on every path: the chunks whose decay sum
    falls below 2^-100 take the per-entry decay branch of the output scores, and
    the state's lazy decay scale is renormalised, in every chunk."""
    set_path(monkeypatch, kpath)
    w, inp = strong_decay_inputs(ci)
    assert min_chunk_decay_sum_base2(inp["g_log"], inp["cu_seqlens"].numpy()) < -100.0
    ref = oracle_run(inp)
    o, fs, cs, offs = gdp.chunk_prefill(**to_device(inp))
    torch.cuda.synchronize()
    tol = TOL[w.dtype]
    e = rel_err(to_np(o), ref["o"])
    assert e <= tol, f"o err {e:.3e}"
    e = rel_err(to_np(fs), ref["final_state"])
    assert e <= tol, f"final state err {e:.3e}"
    NT = int(offs[-1].item())
    e = rel_err(to_np(cs[:NT]), ref["chunk_states"])
    assert e <= tol, f"chunk states err {e:.3e}"


def test_non_finite_input_stays_in_its_chain(gdp, path):
    """A NaN in one v row of one chain (sequence, state head) and an infinite beta
    in another reach only those chains, from the 64-token chunk of the bad token
    on (inside a chunk the masked products multiply it by zero, which gives NaN):
    every other chain's outputs and final state, and those chains' outputs before
    that chunk, are bit-equal to the clean run."""
    w = workloads.workload(1)
    clean = to_device(workloads.generate(w, "cpu"))
    n = w.n
    cu = clean["cu_seqlens"].cpu().numpy()
    bad = dict(clean)
    bad["v"] = clean["v"].clone()
    bad["beta"] = clean["beta"].clone()
    # chain (sequence 3, head 1): NaN in v at token 300 of the sequence, sub-row 1
    t_a = int(cu[3]) + 300
    bad["v"][t_a * n + 1, 1, 5] = float("nan")
    # chain (sequence 2, head 2): infinite beta at token 70 of the sequence, sub-row 0
    t_b = int(cu[2]) + 70
    bad["beta"][t_b * n, 2] = float("inf")
    o0, s0 = gdp.chunk_prefill(**clean)
    o1, s1 = gdp.chunk_prefill(**bad)
    torch.cuda.synchronize()
    for (seq, h, t) in ((3, 1, t_a), (2, 2, t_b)):
        c0 = int(cu[seq]) + (t - int(cu[seq])) // 64 * 64
        assert torch.equal(o1[int(cu[seq]):c0, h], o0[int(cu[seq]):c0, h]), "outputs before the bad chunk changed"
        assert not torch.isfinite(o1[t, h].float()).all(), "the bad token's output is finite"
        assert not torch.isfinite(s1[seq, h]).all(), "the chain's final state is finite"
        o1[int(cu[seq]):int(cu[seq + 1]), h] = o0[int(cu[seq]):int(cu[seq + 1]), h]
        s1[seq, h] = s0[seq, h]
    assert torch.equal(o1, o0), "a non-finite input reached another chain's outputs"
    assert torch.equal(s1, s0), "a non-finite input reached another chain's final state"


# ---------------------------------------------------------------- ragged tails, dims, dtypes, edge cases

CASES = [
    # lens, n, Hqk, Hv, K, V, dtype, l2norm
    ([1], 1, 1, 1, 64, 64, torch.float32, False),
    ([63, 64, 65], 1, 2, 2, 64, 64, torch.float32, True),
    ([130, 7], 3, 1, 2, 64, 128, torch.float32, False),
    ([200, 1, 96], 2, 2, 4, 128, 128, torch.bfloat16, True),
    ([21, 22, 23, 43], 3, 2, 2, 128, 64, torch.bfloat16, False),
    ([150], 4, 1, 1, 64, 128, torch.bfloat16, False),
    ([33, 0, 97], 5, 1, 3, 64, 64, torch.bfloat16, True),
    ([300], 2, 1, 2, 128, 128, torch.bfloat16, False),
]


CASE_PATHS = [(i, p) for i, c in enumerate(CASES)
              for p in (FUSED_FORMS if c[6] == torch.bfloat16 else ["auto"]) if p != "segmented" or c[4] == c[5]]


@pytest.mark.parametrize("ci,kpath", CASE_PATHS, ids=[f"case{i}-{p}" for i, p in CASE_PATHS])
def test_ragged_parity(gdp, ci, kpath, monkeypatch):
    set_path(monkeypatch, kpath)
    lens, n, Hqk, Hv, K, V, dtype, l2 = CASES[ci]
    w = workloads.custom(lens, n, Hqk, Hv, K, V, dtype=dtype, l2norm_in_kernel=l2, init_std=0.2)
    inp = workloads.generate(w, "cpu")
    inp["return_chunk_states"] = True
    ref = oracle_run(inp)
    o, fs, cs, offs = gdp.chunk_prefill(**to_device(inp))
    torch.cuda.synchronize()
    tol = TOL[dtype]
    assert rel_err(to_np(o), ref["o"]) <= tol
    assert rel_err(to_np(fs), ref["final_state"]) <= tol
    NT = int(offs[-1].item())
    assert NT == ref["chunk_states"].shape[0]
    assert rel_err(to_np(cs[:NT]), ref["chunk_states"]) <= tol


def test_all_sequences_empty(gdp, path):
    w = workloads.custom([0, 0, 0], 2, 1, 2, 64, 64, dtype=torch.bfloat16, init_std=0.3)
    inp = to_device(workloads.generate(w, "cpu"))
    o, fs = gdp.chunk_prefill(**inp)
    torch.cuda.synchronize()
    assert o.shape[0] == 0
    assert torch.equal(fs, inp["initial_state"])


def test_strided_q_and_o(gdp, path):
    w = workloads.custom([100, 29], 2, 2, 2, 128, 128, dtype=torch.bfloat16)
    inp = to_device(workloads.generate(w, "cpu"))
    ref_o, ref_s = gdp.chunk_prefill(**inp)
    big = torch.zeros((inp["q"].shape[0], 2, 3 * 128), dtype=torch.bfloat16, device="cuda")
    big[:, :, 128:256] = inp["q"]
    obig = torch.zeros((inp["q"].shape[0], 2, 2 * 128 + 64), dtype=torch.bfloat16, device="cuda")
    args = dict(inp, q=big[:, :, 128:256], out=obig[:, :, 64:192])
    o, s = gdp.chunk_prefill(**args)
    torch.cuda.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(s, ref_s)
    assert torch.all(obig[:, :, :64] == 0) and torch.all(obig[:, :, 192:] == 0)


def test_determinism_and_caller_descriptors(gdp, path):
    w = workloads.workload(1)
    inp = to_device(workloads.generate(w, "cpu"))
    a = gdp.chunk_prefill(**inp)
    b = gdp.chunk_prefill(**inp)
    desc = gdp.gdp_build_descriptors(inp["cu_seqlens"], w.n, w.T, nt_cap=64, ntdp_cap=100)
    c = gdp.chunk_prefill(**inp, descriptors=desc)
    torch.cuda.synchronize()
    for x, y in ((a, b), (a, c)):
        assert torch.equal(x[0], y[0]) and torch.equal(x[1], y[1])


def test_split_and_resume_on_gpu(gdp, path):
    w = workloads.custom([333], 2, 1, 2, 128, 128, dtype=torch.bfloat16)
    inp = to_device(workloads.generate(w, "cpu"))
    full_o, full_s = gdp.chunk_prefill(**inp)
    L1, n = 190, 2
    a = dict(inp, q=inp["q"][:L1], k=inp["k"][:L1 * n], v=inp["v"][:L1 * n], g_log=inp["g_log"][:L1],
             beta=inp["beta"][:L1 * n], cu_seqlens=torch.tensor([0, L1], dtype=torch.int32, device="cuda"))
    oa, sa = gdp.chunk_prefill(**a)
    b = dict(inp, q=inp["q"][L1:], k=inp["k"][L1 * n:], v=inp["v"][L1 * n:], g_log=inp["g_log"][L1:],
             beta=inp["beta"][L1 * n:], cu_seqlens=torch.tensor([0, 333 - L1], dtype=torch.int32, device="cuda"),
             initial_state=sa)
    ob, sb = gdp.chunk_prefill(**b)
    torch.cuda.synchronize()
    e = rel_err(to_np(torch.cat([oa, ob])), to_np(full_o))
    assert e <= 1.5e-2
    assert rel_err(to_np(sb), to_np(full_s)) <= 1.5e-2


def test_graph_capture_replay(gdp, path):
    """Descriptors at capacity keep the grid fixed for (T, N): a captured call
    replays correctly with new cu_seqlens contents of the same T and N."""
    w = workloads.custom([100, 60, 40], 2, 2, 2, 128, 128, dtype=torch.bfloat16)
    inp = to_device(workloads.generate(w, "cpu"))
    T, N = w.T, w.N
    ws = torch.empty(gdp.gdp_workspace_bytes(T, N, 2, 2, 2, 128, 128, torch.bfloat16), dtype=torch.uint8,
                     device="cuda")
    o = torch.empty((T, 2, 128), dtype=torch.bfloat16, device="cuda")
    fs = torch.empty((N, 2, 128, 128), dtype=torch.float32, device="cuda")
    cu = inp["cu_seqlens"].clone()

    def call():
        gdp.gdp_chunk_prefill(inp["q"], inp["k"], inp["v"], inp["g_log"], inp["beta"], 2, cu, 0.0,
                              inp["initial_state"], True, False, None, None, False, o, fs, None, None, ws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for lens in ([100, 60, 40], [1, 198, 1], [0, 0, 200], [67, 66, 67]):
        cu.copy_(torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32, device="cuda"))
        g.replay()
        torch.cuda.synchronize()
        go, gs = o.clone(), fs.clone()
        call()
        torch.cuda.synchronize()
        assert torch.equal(go, o) and torch.equal(gs, fs), f"replay differs from eager for {lens}"


@pytest.mark.parametrize("d", [128, 64])
def test_segmented_long_sequence(gdp, monkeypatch, d):
    """A sequence long enough for several segments, with GQA, chunk states and a
    cache slot: the automatic choice is the segmented path (4 chains, a dozen
    segments for the longer sequence, so the combine steps through many maps);
    every output, the final state, the chunk-state rows and the cache slot match
    the oracle, and the fused path on the same inputs."""
    monkeypatch.delenv("GDP_PREFILL_PATH", raising=False)
    w = workloads.custom([3000, 1500], 2, 1, 2, d, d, dtype=torch.bfloat16, l2norm_in_kernel=True, init_std=0.2,
                         seed=31, state_cache_slots=3)
    inp = workloads.generate(w, "cpu")
    inp["state_indices"] = torch.tensor([2, 0], dtype=torch.int32)
    inp["return_chunk_states"] = True
    ref = oracle_run(inp)
    dev = to_device(inp)
    cache0 = dev["state_cache"].clone()
    o, fs, cs, offs = gdp.chunk_prefill(**dev)
    torch.cuda.synchronize()
    tol = TOL[torch.bfloat16]
    assert rel_err(to_np(o), ref["o"]) <= tol
    assert rel_err(to_np(fs), ref["final_state"]) <= tol
    NT = int(offs[-1].item())
    assert rel_err(to_np(cs[:NT]), ref["chunk_states"]) <= tol
    assert rel_err(to_np(dev["state_cache"][[2, 0]]), ref["state_cache"][[2, 0]]) <= tol
    assert torch.equal(dev["state_cache"][1], cache0[1])
    monkeypatch.setenv("GDP_PREFILL_PATH", "fused")
    dev2 = to_device(inp)
    o2, fs2, _, _ = gdp.chunk_prefill(**dev2)
    torch.cuda.synchronize()
    assert rel_err(to_np(o), to_np(o2)) <= tol and rel_err(to_np(fs), to_np(fs2)) <= tol


def test_fused_and_split_agree(gdp, monkeypatch):
    """Every bf16 path and fused output form on the varlen workload: each within
    tolerance of the oracle, and of the split pair."""
    w = workloads.workload(1)
    inp = workloads.generate(w, "cpu")
    ref = oracle_run(inp)
    dev = to_device(inp)
    out = {}
    for p in FUSED_FORMS:
        set_path(monkeypatch, p)
        out[p] = run_gpu(gdp, dev)
        check_all(inp, out[p], ref, TOL[w.dtype], what=p)
    for p in ("fused", "fused_tc", "segmented"):
        assert rel_err(to_np(out[p][0]), to_np(out["split"][0])) <= TOL[w.dtype], p
        assert rel_err(to_np(out[p][1]), to_np(out["split"][1])) <= TOL[w.dtype], p


@pytest.mark.parametrize("N,Hqk,Hv", [(40, 4, 8), (90, 1, 3)], ids=["grouped-heads", "odd-grid"])
def test_longest_first_order_every_chain(gdp, N, Hqk, Hv, monkeypatch):
    """More chains than CUs with mixed lengths: the fused kernel runs its chains
    longest sequence first.  Every head of every sequence (outputs, final states,
    cache slots) matches the oracle, so the order visits each chain exactly once,
    for a grid of whole q/k head groups (N*Hv = 320) and one that does not split
    into 8 XCD lists (N*Hv = 270)."""
    monkeypatch.delenv("GDP_PREFILL_PATH", raising=False)
    gen = torch.Generator().manual_seed(N)
    lens = torch.randint(0, 200, (N,), generator=gen).tolist()
    w = workloads.custom(lens, 2, Hqk, Hv, 64, 64, dtype=torch.bfloat16, init_std=0.2, seed=41,
                         state_cache_slots=N + 3)
    inp = workloads.generate(w, "cpu")
    ref = oracle_run(inp)
    dev = to_device(inp)
    cache0 = dev["state_cache"].clone()
    o, fs = gdp.chunk_prefill(**dev)
    torch.cuda.synchronize()
    tol = TOL[torch.bfloat16]
    check_all(inp, (o, fs), ref, tol, what="ordered")
    slots = inp["state_indices"].numpy()
    assert rel_err(to_np(dev["state_cache"][slots]), ref["state_cache"][slots]) <= tol
    untouched = sorted(set(range(N + 3)) - set(slots.tolist()))
    assert torch.equal(dev["state_cache"][untouched], cache0[untouched])


@pytest.mark.parametrize("N", [1500, 5000], ids=["N1500-ordered", "N5000-unordered"])
@pytest.mark.parametrize("kpath", ["fused", "split"])
def test_many_short_sequences(gdp, N, kpath, monkeypatch):
    """Thousands of sequences of 0..6 tokens: the descriptor scan over several
    1024-sequence passes, the longest-first work order (up to 4096 sequences;
    beyond that the grid runs in sequence order), zero-length sequences, and
    chunk states, against the oracle."""
    monkeypatch.setenv("GDP_PREFILL_PATH", kpath)
    lens = np.random.default_rng(N).integers(0, 7, size=N).tolist()
    w = workloads.custom(lens, 2, 1, 2, 64, 64, dtype=torch.bfloat16, init_std=0.2, seed=N)
    inp = workloads.generate(w, "cpu")
    inp["return_chunk_states"] = True
    ref = oracle_run(inp)
    o, fs, cs, offs = gdp.chunk_prefill(**to_device(inp))
    torch.cuda.synchronize()
    tol = TOL[torch.bfloat16]
    assert rel_err(to_np(o), ref["o"]) <= tol
    assert rel_err(to_np(fs), ref["final_state"]) <= tol
    NT = int(offs[-1].item())
    assert NT == ref["chunk_states"].shape[0] == sum(1 for L in lens if L > 0)
    assert rel_err(to_np(cs[:NT]), ref["chunk_states"]) <= tol
