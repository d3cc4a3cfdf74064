"""gdp_chunk_prefill_noalloc (no workspace argument, static per-GPU scratch)
against gdp_chunk_prefill with a workspace, through the C ABI (needs a gfx950
GPU)."""
import pytest
import torch

from gated_deltaproduct_recurrence_amd import workloads
from tests.parity import TOL, oracle_run, rel_err, to_device, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gdp():
    from gated_deltaproduct_recurrence_amd import binding
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return binding


def _both(gdp, inp, w):
    """The same prefill through both entry points into separate outputs."""
    T, N, n = w.T, w.N, w.n
    nt_cap, _ = gdp.gdp_descriptor_capacity(T, N, n)
    res = []
    for noalloc in (False, True):
        o = torch.full((T, w.Hv, w.V), float("nan"), dtype=w.dtype, device="cuda")
        fs = torch.full((N, w.Hv, w.K, w.V), float("nan"), dtype=torch.float32, device="cuda")
        cs = torch.full((max(nt_cap, 1), w.Hv, w.K, w.V), float("nan"), dtype=torch.float32, device="cuda")
        args = (inp["q"], inp["k"], inp["v"], inp["g_log"], inp["beta"], n, inp["cu_seqlens"], inp["scale"] or 0.0,
                inp["initial_state"], True, inp["use_qk_l2norm"], None, None, True, o, fs, cs, None)
        if noalloc:
            gdp.gdp_chunk_prefill_noalloc(*args)
        else:
            ws = torch.empty(gdp.gdp_workspace_bytes(T, N, n, w.Hqk, w.Hv, w.K, w.V, w.dtype), dtype=torch.uint8,
                             device="cuda")
            gdp.gdp_chunk_prefill(*args, ws)
        torch.cuda.synchronize()
        res.append((o, fs, cs))
    return res


@pytest.mark.parametrize("kpath", ["fused", "split", "segmented"])
def test_noalloc_matches_the_workspace_entry(gdp, kpath, monkeypatch):
    """Two calls in a row through the entry point without a workspace, the
    second with a smaller input (so the scratch array still holds the first
    call's descriptors, order and WY matrices): each equals the workspace entry
    point's result on the same inputs bit for bit, and is within the oracle's
    tolerance."""
    monkeypatch.setenv("GDP_PREFILL_PATH", kpath)
    big = workloads.custom([700, 300, 77, 512], 2, 2, 4, 128, 128, dtype=torch.bfloat16, l2norm_in_kernel=True,
                           init_std=0.2, seed=501)
    small = workloads.custom([300, 45], 3, 1, 2, 128, 128, dtype=torch.bfloat16, init_std=0.2, seed=502)
    for w in (big, small):
        cpu = workloads.generate(w, "cpu")
        inp = to_device(cpu)
        (o0, f0, c0), (o1, f1, c1) = _both(gdp, inp, w)
        assert torch.equal(o0, o1), f"{kpath}: o differs"
        assert torch.equal(f0, f1), f"{kpath}: final state differs"
        nt = sum((L + 63) // 64 for L in w.lens)
        assert torch.equal(c0[:nt], c1[:nt]), f"{kpath}: chunk states differ"
        ref = oracle_run(dict(cpu, return_chunk_states=True))
        tol = TOL[w.dtype]
        assert rel_err(to_np(o1), ref["o"]) <= tol
        assert rel_err(to_np(f1), ref["final_state"]) <= tol
        assert rel_err(to_np(c1[:nt]), ref["chunk_states"]) <= tol


def test_noalloc_float32_inputs(gdp, monkeypatch):
    """float32 inputs (the split path), twice, the second call smaller."""
    monkeypatch.delenv("GDP_PREFILL_PATH", raising=False)
    for w in (workloads.workload(0), workloads.custom([90, 33], 2, 1, 2, 64, 64, dtype=torch.float32, seed=503)):
        cpu = workloads.generate(w, "cpu")
        (o0, f0, _), (o1, f1, _) = _both(gdp, to_device(cpu), w)
        assert torch.equal(o0, o1) and torch.equal(f0, f1)
        ref = oracle_run(cpu)
        assert rel_err(to_np(o1), ref["o"]) <= TOL[torch.float32]
