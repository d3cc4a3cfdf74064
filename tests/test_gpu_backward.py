"""Gradients of the prefill (gdp_chunk_prefill_backward) against the fp64
autograd oracle, element by element, through the C ABI (needs a gfx950 GPU)."""
import numpy as np
import pytest
import torch

from gated_deltaproduct_recurrence_amd import workloads
from oracle import backward as obwd
from tests.parity import TOL, oracle_run, rel_err, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gdp():
    from gated_deltaproduct_recurrence_amd import binding
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return binding


CASES = [
    # lens, n, Hqk, Hk, Hv, K, V, dtype, l2norm, init, dfinal
    ([37, 64, 130], 2, 2, 2, 4, 128, 128, torch.bfloat16, False, True, True),
    ([70, 1, 0, 9], 3, 1, 1, 2, 64, 64, torch.float32, True, True, False),
    ([100, 29], 1, 1, 2, 2, 64, 128, torch.bfloat16, True, False, True),
    ([65, 63], 3, 2, 2, 2, 128, 64, torch.bfloat16, False, False, False),
    ([45, 80], 2, 2, 4, 4, 128, 128, torch.bfloat16, True, True, False),
    ([30, 41], 4, 1, 2, 2, 128, 128, torch.bfloat16, True, True, True),
    ([19, 0, 26], 5, 1, 1, 2, 64, 64, torch.bfloat16, False, True, False),
]


def run_case(gdp, ci, seed=0):
    lens, n, Hqk, Hk, Hv, K, V, dt, l2, init, dfin = CASES[ci]
    w = workloads.custom(lens, n, Hqk, Hv, K, V, dtype=dt, l2norm_in_kernel=l2, init_std=0.2 if init else 0.0,
                         seed=100 + ci)
    inp = workloads.generate(w, "cpu")
    gen = torch.Generator().manual_seed(200 + ci)
    T, N = w.T, w.N
    if Hk != Hqk:  # one k head per state head
        k = torch.randn(T * n, Hk, K, generator=gen)
        inp["k"] = (k if l2 else k / k.norm(dim=-1, keepdim=True)).to(dt)
    d_o = torch.randn(T, Hv, V, generator=gen).to(dt)
    d_fin = torch.randn(N, Hv, K, V, generator=gen) if dfin else None
    ref = obwd.backward(to_np(inp["q"]), to_np(inp["k"]), to_np(inp["v"]), to_np(inp["g_log"]), to_np(inp["beta"]),
                        n, inp["cu_seqlens"].numpy(), to_np(d_o), None if d_fin is None else d_fin.numpy(),
                        initial_state=to_np(inp["initial_state"]), use_qk_l2norm=l2)
    dev = lambda x: None if x is None else x.cuda()
    res = gdp.chunk_prefill_backward(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["g_log"]),
                                     dev(inp["beta"]), n, dev(inp["cu_seqlens"]), dev(d_o), dev(d_fin),
                                     initial_state=dev(inp["initial_state"]), use_qk_l2norm=l2)
    torch.cuda.synchronize()
    return res, ref, TOL[dt]


@pytest.mark.parametrize("kpath", ["chunked", "recurrent-fused", "recurrent-split"])
@pytest.mark.parametrize("ci", range(len(CASES)))
def test_backward_parity(gdp, ci, kpath, monkeypatch):
    """Every case on the chunked path (the default for bfloat16 inputs; float32
    inputs always take the recurrent one) and on the recurrent path with either
    forward rerun."""
    if kpath == "recurrent-fused" and CASES[ci][7] == torch.float32:
        pytest.skip("float32 inputs run the split forward only")
    if kpath.startswith("recurrent"):
        monkeypatch.setenv("GDP_BACKWARD_PATH", "recurrent")
        monkeypatch.setenv("GDP_PREFILL_PATH", kpath.split("-")[1])
    res, ref, tol = run_case(gdp, ci)
    names = ["dq", "dk", "dv", "dg_log", "dbeta"] + (["d_initial_state"] if res["d_initial_state"] is not None else [])
    for name in names:
        key = "dinitial_state" if name == "d_initial_state" else name
        e = rel_err(to_np(res[name]), ref[key])
        assert e <= tol, f"case {ci} {kpath}: {name} err {e:.3e}"


def test_backward_strong_decays(gdp):
    """Decays down to g_log = -40 on some tokens (the chunk's cumulative decay
    underflows): the chunked path's decay ratios and factors stay finite and the
    gradients match the oracle."""
    lens, n, Hqk, Hv, K, V = [150, 70], 2, 2, 4, 128, 128
    w = workloads.custom(lens, n, Hqk, Hv, K, V, dtype=torch.bfloat16, l2norm_in_kernel=True, init_std=0.2,
                         seed=91)
    inp = workloads.generate(w, "cpu")
    gen = torch.Generator().manual_seed(92)
    g = -torch.nn.functional.softplus(torch.randn(w.T, Hv, generator=gen) + 2.0)
    g[torch.rand(w.T, Hv, generator=gen) < 0.05] = -40.0
    inp["g_log"] = g
    d_o = torch.randn(w.T, Hv, V, generator=gen).to(torch.bfloat16)
    ref = obwd.backward(to_np(inp["q"]), to_np(inp["k"]), to_np(inp["v"]), to_np(g), to_np(inp["beta"]), n,
                        inp["cu_seqlens"].numpy(), to_np(d_o), None, initial_state=to_np(inp["initial_state"]),
                        use_qk_l2norm=True)
    dev = lambda x: None if x is None else x.cuda()
    res = gdp.chunk_prefill_backward(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(g), dev(inp["beta"]), n,
                                     dev(inp["cu_seqlens"]), dev(d_o), None, initial_state=dev(inp["initial_state"]),
                                     use_qk_l2norm=True)
    torch.cuda.synchronize()
    for name in ("dq", "dk", "dv", "dg_log", "dbeta", "d_initial_state"):
        key = "dinitial_state" if name == "d_initial_state" else name
        x = to_np(res[name])
        assert np.isfinite(x).all(), name
        e = rel_err(x, ref[key])
        assert e <= TOL[torch.bfloat16], f"{name} err {e:.3e}"


def test_backward_zero_length_and_padding_rows(gdp):
    """A zero-length sequence contributes nothing, and its initial-state gradient
    is d_final_state passed straight through."""
    res, ref, tol = run_case(gdp, 1)
    lens = CASES[1][0]
    assert lens[2] == 0
    assert rel_err(to_np(res["d_initial_state"][2]), ref["dinitial_state"][2]) <= tol


def test_backward_long_context_sampled(gdp):
    """Full-size long-context gradients (8 x 65536 tokens, n=2, Hqk=16 / Hv=32,
    in-kernel norm), as the benchmark runs them.  A token's gradients depend only
    on the inputs from that token on and on the state entering it, so the oracle
    checks the last M tokens of sampled (sequence, q/k head) groups: the fp64
    forward oracle gives the state entering the suffix from the prefix, and the
    autograd oracle differentiates the suffix alone.  The two state heads of the
    group are both in the sample, so dq and dk (summed over them) compare too."""
    w = workloads.workload(4)
    inp = workloads.generate(w, "cuda")
    gen = torch.Generator(device="cuda").manual_seed(404)
    d_o = torch.randn(w.T, w.Hv, w.V, generator=gen, device="cuda").to(w.dtype)
    res = gdp.chunk_prefill_backward(inp["q"], inp["k"], inp["v"], inp["g_log"], inp["beta"], w.n,
                                     inp["cu_seqlens"], d_o, None, initial_state=inp["initial_state"],
                                     use_qk_l2norm=True)
    torch.cuda.synchronize()
    for name in ("dq", "dk", "dv", "dg_log", "dbeta"):
        assert torch.isfinite(res[name]).all(), name
    cu = inp["cu_seqlens"].cpu().numpy()
    n, M = w.n, 160
    for seq, hq in ((7, 5), (2, 12)):
        t0, t1 = int(cu[seq]), int(cu[seq + 1])
        ts = t1 - M
        heads = [2 * hq, 2 * hq + 1]
        prefix = dict(q=inp["q"][t0:ts, hq:hq + 1], k=inp["k"][t0 * n:ts * n, hq:hq + 1],
                      v=inp["v"][t0 * n:ts * n, heads], g_log=inp["g_log"][t0:ts, heads],
                      beta=inp["beta"][t0 * n:ts * n, heads], num_householder=n,
                      cu_seqlens=torch.tensor([0, ts - t0]), scale=None,
                      initial_state=inp["initial_state"][seq:seq + 1, heads], use_qk_l2norm=True)
        s_mid = oracle_run(prefix, threads=2)["final_state"]
        ref = obwd.backward(to_np(inp["q"][ts:t1, hq:hq + 1]), to_np(inp["k"][ts * n:t1 * n, hq:hq + 1]),
                            to_np(inp["v"][ts * n:t1 * n, heads]), to_np(inp["g_log"][ts:t1, heads]),
                            to_np(inp["beta"][ts * n:t1 * n, heads]), n, np.array([0, M]),
                            to_np(d_o[ts:t1, heads]), None, initial_state=s_mid, use_qk_l2norm=True)
        got = {"dq": res["dq"][ts:t1, hq:hq + 1], "dk": res["dk"][ts * n:t1 * n, hq:hq + 1],
               "dv": res["dv"][ts * n:t1 * n, heads], "dg_log": res["dg_log"][ts:t1, heads],
               "dbeta": res["dbeta"][ts * n:t1 * n, heads]}
        for name, x in got.items():
            e = rel_err(to_np(x), ref[name])
            assert e <= TOL[w.dtype], f"seq {seq} q/k head {hq}: {name} err {e:.3e}"


def test_backward_strided_d_o_and_dv(gdp):
    """d_o and dv may have strided rows (views into wider buffers): same
    gradients as the contiguous call, checked against the oracle."""
    lens, n, Hqk, Hk, Hv, K, V, dt, l2, init, dfin = CASES[0]
    w = workloads.custom(lens, n, Hqk, Hv, K, V, dtype=dt, l2norm_in_kernel=l2, init_std=0.2, seed=100)
    inp = workloads.generate(w, "cpu")
    gen = torch.Generator().manual_seed(200)
    T, N = w.T, w.N
    d_o_wide = torch.randn(T, Hv + 3, V, generator=gen).to(dt)
    d_o = d_o_wide[:, 1:1 + Hv]  # row stride (Hv + 3) V
    ref = obwd.backward(to_np(inp["q"]), to_np(inp["k"]), to_np(inp["v"]), to_np(inp["g_log"]), to_np(inp["beta"]),
                        n, inp["cu_seqlens"].numpy(), to_np(d_o.contiguous()), None,
                        initial_state=to_np(inp["initial_state"]), use_qk_l2norm=l2)
    dev = lambda x: None if x is None else x.cuda()
    f32 = dict(dtype=torch.float32, device="cuda")
    dq, dk = torch.empty((T, Hqk, K), **f32), torch.empty((T * n, Hk, K), **f32)
    dv_wide = torch.full((T * n, Hv + 2, V), float("nan"), **f32)
    dv = dv_wide[:, 2:]
    dg, db = torch.empty((T, Hv), **f32), torch.empty((T * n, Hv), **f32)
    ds0 = torch.empty((N, Hv, K, V), **f32)
    ws = torch.empty(gdp.gdp_backward_workspace_bytes(T, N, n, Hqk, Hv, K, V, dt), dtype=torch.uint8, device="cuda")
    gdp.gdp_chunk_prefill_backward(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["g_log"]), dev(inp["beta"]), n,
                                   dev(inp["cu_seqlens"]), 0.0, dev(inp["initial_state"]), l2, dev(d_o_wide)[:, 1:1 + Hv],
                                   None, dq, dk, dv, dg, db, ds0, ws)
    torch.cuda.synchronize()
    tol = TOL[dt]
    for name, x in (("dq", dq), ("dk", dk), ("dv", dv), ("dg_log", dg), ("dbeta", db), ("dinitial_state", ds0)):
        e = rel_err(to_np(x), ref[name])
        assert e <= tol, f"{name} err {e:.3e}"
    assert torch.isnan(dv_wide[:, :2]).all(), "dv wrote outside its view"


def test_backward_graph_capture_replay(gdp):
    """The backward call (forward rerun, fills, backward and norm kernels) is
    captured in a HIP graph and replayed three times, with eager work between
    the replays: every replay matches the eager call (float atomics may reorder
    the last bits) and the oracle."""
    lens, n, Hqk, Hk, Hv, K, V, dt, l2, init, dfin = CASES[0]
    w = workloads.custom(lens, n, Hqk, Hv, K, V, dtype=dt, l2norm_in_kernel=l2, init_std=0.2, seed=100)
    inp = {k: (x.cuda() if isinstance(x, torch.Tensor) else x) for k, x in workloads.generate(w, "cpu").items()}
    gen = torch.Generator().manual_seed(200)
    T, N = w.T, w.N
    d_o = torch.randn(T, Hv, V, generator=gen).to(dt).cuda()
    f32 = dict(dtype=torch.float32, device="cuda")
    outs = {"dq": torch.empty((T, Hqk, K), **f32), "dk": torch.empty((T * n, Hk, K), **f32),
            "dv": torch.empty((T * n, Hv, V), **f32), "dg_log": torch.empty((T, Hv), **f32),
            "dbeta": torch.empty((T * n, Hv), **f32), "dinitial_state": torch.empty((N, Hv, K, V), **f32)}
    ws = torch.empty(gdp.gdp_backward_workspace_bytes(T, N, n, Hqk, Hv, K, V, dt), dtype=torch.uint8, device="cuda")

    def call():
        gdp.gdp_chunk_prefill_backward(inp["q"], inp["k"], inp["v"], inp["g_log"], inp["beta"], n, inp["cu_seqlens"],
                                       0.0, inp["initial_state"], l2, d_o, None, outs["dq"], outs["dk"], outs["dv"],
                                       outs["dg_log"], outs["dbeta"], outs["dinitial_state"], ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = {k: x.clone() for k, x in outs.items()}
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    ref = obwd.backward(to_np(inp["q"]), to_np(inp["k"]), to_np(inp["v"]), to_np(inp["g_log"]), to_np(inp["beta"]), n,
                        inp["cu_seqlens"].cpu().numpy(), to_np(d_o), None, initial_state=to_np(inp["initial_state"]),
                        use_qk_l2norm=l2)
    for rep in range(3):
        for x in outs.values():
            x.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for name, x in outs.items():
            assert rel_err(to_np(x), to_np(eager[name])) <= 1e-5, f"replay {rep}: {name} differs from eager"
            assert rel_err(to_np(x), ref[name]) <= TOL[dt], f"replay {rep}: {name} vs oracle"
        call()  # eager work between the replays
        torch.cuda.synchronize()


def _backward_into(gdp, inp, n, d_o, cu, fill=float("nan")):
    """Low-level backward call into caller buffers pre-filled with `fill`."""
    T, Hqk, K = inp["q"].shape
    Hk, Hv, V = inp["k"].shape[1], inp["v"].shape[1], inp["v"].shape[2]
    N = cu.shape[0] - 1
    f32 = dict(dtype=torch.float32, device="cuda")
    outs = {"dq": torch.full((T, Hqk, K), fill, **f32), "dk": torch.full((T * n, Hk, K), fill, **f32),
            "dv": torch.full((T * n, Hv, V), fill, **f32), "dg_log": torch.full((T, Hv), fill, **f32),
            "dbeta": torch.full((T * n, Hv), fill, **f32), "dinitial_state": torch.full((N, Hv, K, V), fill, **f32)}
    ws = torch.empty(gdp.gdp_backward_workspace_bytes(T, N, n, Hqk, Hv, K, V, inp["q"].dtype), dtype=torch.uint8,
                     device="cuda")
    gdp.gdp_chunk_prefill_backward(inp["q"], inp["k"], inp["v"], inp["g_log"], inp["beta"], n, cu, 0.0,
                                   inp["initial_state"], inp["use_qk_l2norm"], d_o, None, outs["dq"], outs["dk"],
                                   outs["dv"], outs["dg_log"], outs["dbeta"], outs["dinitial_state"], ws)
    torch.cuda.synchronize()
    return outs


@pytest.mark.parametrize("cu_list", [[0, 50, 100], [7, 50, 100]], ids=["tail-padding", "head-and-tail-padding"])
def test_backward_rows_outside_the_sequences_are_zero(gdp, cu_list):
    """cu_seqlens covering only part of T (a fixed padded T under graph capture):
    every gradient, dv included, is 0 on the sub-rows no sequence covers (the
    buffers start as NaN), and the covered rows match the oracle run on them."""
    n, T = 2, 120
    w = workloads.custom([T // 2, T // 2], n, 1, 2, 128, 128, dtype=torch.bfloat16, init_std=0.2, seed=77)
    inp = {k: (x.cuda() if isinstance(x, torch.Tensor) else x) for k, x in workloads.generate(w, "cpu").items()}
    d_o = torch.randn(T, 2, 128, generator=torch.Generator().manual_seed(78)).to(torch.bfloat16).cuda()
    cu = torch.tensor(cu_list, dtype=torch.int32, device="cuda")
    outs = _backward_into(gdp, inp, n, d_o, cu)
    lo, hi = cu_list[0], cu_list[-1]
    for name, per in (("dq", 1), ("dk", n), ("dv", n), ("dg_log", 1), ("dbeta", n)):
        x = outs[name]
        assert torch.all(x[:lo * per] == 0) and torch.all(x[hi * per:] == 0), f"{name} padding rows not zero"
    sub = np.array(cu_list) - lo
    ref = obwd.backward(to_np(inp["q"][lo:hi]), to_np(inp["k"][lo * n:hi * n]), to_np(inp["v"][lo * n:hi * n]),
                        to_np(inp["g_log"][lo:hi]), to_np(inp["beta"][lo * n:hi * n]), n, sub, to_np(d_o[lo:hi]), None,
                        initial_state=to_np(inp["initial_state"]), use_qk_l2norm=False)
    for name, per in (("dq", 1), ("dk", n), ("dv", n), ("dg_log", 1), ("dbeta", n)):
        e = rel_err(to_np(outs[name][lo * per:hi * per]), ref[name])
        assert e <= TOL[torch.bfloat16], f"{name} err {e:.3e}"
    assert rel_err(to_np(outs["dinitial_state"]), ref["dinitial_state"]) <= TOL[torch.bfloat16]


def test_backward_non_monotone_cu_seqlens_stays_in_bounds(gdp):
    """cu_seqlens = [0, T, 0, T] (not monotone) makes the descriptors place the
    last sequence's chunk-state rows past the buffer; the backward reads a zero
    state there instead of reading out of bounds, and the call completes with
    finite gradients."""
    n, T = 2, 640
    w = workloads.custom([T], n, 1, 2, 64, 64, dtype=torch.bfloat16, init_std=0.2, seed=79)
    inp = workloads.generate(w, "cpu")
    inp["initial_state"] = torch.cat([inp["initial_state"]] * 3)
    inp = {k: (x.cuda() if isinstance(x, torch.Tensor) else x) for k, x in inp.items()}
    d_o = torch.randn(T, 2, 64, generator=torch.Generator().manual_seed(80)).to(torch.bfloat16).cuda()
    cu = torch.tensor([0, T, 0, T], dtype=torch.int32, device="cuda")
    assert gdp.gdp_descriptor_capacity(T, 3, n)[0] < 20  # the last sequence's rows 10..19 lie past it
    outs = _backward_into(gdp, inp, n, d_o, cu, fill=0.0)
    for name, x in outs.items():
        assert torch.isfinite(x).all(), name
