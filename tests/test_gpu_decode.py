"""The single-token decode step on the state cache: HIP path vs the fp64
oracle through the C ABI (needs a gfx950 GPU)."""
import numpy as np
import pytest
import torch

import oracle
from gated_deltaproduct_recurrence_amd import workloads
from tests.parity import TOL, rel_err, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gdp():
    from gated_deltaproduct_recurrence_amd import binding
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return binding


def oracle_decode(inp):
    return oracle.decode(to_np(inp["q"]), to_np(inp["k"]), to_np(inp["v"]), to_np(inp["g_log"]),
                         to_np(inp["beta"]), inp["num_householder"], to_np(inp["state_cache"]),
                         inp["state_indices"].cpu().numpy(), use_qk_l2norm=inp["use_qk_l2norm"])


def run_decode(gdp, inp):
    dev = {k: (v.to("cuda") if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    o = gdp.recurrent_decode(**dev)
    torch.cuda.synchronize()
    return o, dev["state_cache"]


CASES = [
    # N, n, Hqk, Hv, K, V, slots, pad, dtype, l2norm
    (1, 1, 1, 1, 64, 64, 3, 0, torch.float32, False),
    (7, 2, 2, 4, 128, 128, 16, 2, torch.bfloat16, True),
    (5, 3, 1, 2, 64, 128, 9, 1, torch.bfloat16, False),
    (4, 1, 2, 2, 128, 64, 4, 0, torch.float32, True),
    (33, 2, 4, 8, 128, 128, 64, 5, torch.bfloat16, False),
    (3, 4, 1, 1, 64, 64, 5, 3, torch.bfloat16, True),
]


@pytest.mark.parametrize("case", CASES, ids=[f"case{i}" for i in range(len(CASES))])
def test_decode_parity(gdp, case):
    N, n, Hqk, Hv, K, V, slots, pad, dtype, l2 = case
    inp = workloads.decode_batch(N, n, Hqk, Hv, K, V, slots, pad=pad, dtype=dtype, l2norm_in_kernel=l2, seed=N)
    ref = oracle_decode(inp)
    cache0 = inp["state_cache"].clone()
    o, cache = run_decode(gdp, inp)
    tol = TOL[dtype]
    idx = inp["state_indices"].numpy()
    live = idx >= 0
    assert rel_err(to_np(o)[live], ref["o"][live]) <= tol
    assert torch.all(o[torch.from_numpy(~live).cuda()] == 0), "padding rows must be zero"
    written = sorted(int(s) for s in idx[live])
    assert rel_err(to_np(cache[written]), ref["state_cache"][written]) <= tol
    untouched = sorted(set(range(slots)) - set(written))
    assert torch.equal(cache[untouched].cpu(), cache0[untouched]), "untouched slots changed"


def test_decode_int64_indices_and_out_of_range(gdp):
    inp = workloads.decode_batch(6, 2, 1, 2, 128, 128, 8, dtype=torch.bfloat16, seed=3)
    idx = inp["state_indices"].to(torch.int64)
    idx[2] = 8          # past the cache: treated like padding
    inp["state_indices"] = idx
    ref = oracle_decode(inp)
    cache0 = inp["state_cache"].clone()
    o, cache = run_decode(gdp, inp)
    live = np.array([i != 2 for i in range(6)])
    assert rel_err(to_np(o)[live], ref["o"][live]) <= TOL[torch.bfloat16]
    assert torch.all(o[2] == 0)
    untouched = sorted(set(range(8)) - set(int(s) for s in idx[live].tolist()))
    assert torch.equal(cache[untouched].cpu(), cache0[untouched])


def test_decode_steps_equal_prefill(gdp):
    """T decode steps of N sequences from their cache slots reproduce the GPU
    prefill (and the oracle prefill) of the T-token sequences started there."""
    N, T, n, Hqk, Hv, K, V = 3, 70, 2, 1, 2, 128, 128
    w = workloads.custom([T] * N, n, Hqk, Hv, K, V, dtype=torch.bfloat16, l2norm_in_kernel=True, init_std=0.0,
                         seed=21)
    pre = workloads.generate(w, "cpu")
    cache = 0.3 * torch.randn((5, Hv, K, V), generator=torch.Generator().manual_seed(5))
    slots = torch.tensor([4, 0, 2], dtype=torch.int32)
    ref = oracle.prefill(to_np(pre["q"]), to_np(pre["k"]), to_np(pre["v"]), to_np(pre["g_log"]),
                         to_np(pre["beta"]), n, pre["cu_seqlens"].numpy(), initial_state=to_np(cache[slots]),
                         use_qk_l2norm=True)
    dev = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in pre.items()}
    dev["initial_state"] = cache[slots].cuda()
    o_pre, s_pre = gdp.chunk_prefill(**dev)
    c = cache.cuda()
    sl = slots.cuda()
    outs = []
    for t in range(T):
        tok = torch.arange(N) * T + t
        rows = (tok[:, None] * n + torch.arange(n)[None, :]).reshape(-1)
        outs.append(gdp.recurrent_decode(dev["q"][tok.cuda()], dev["k"][rows.cuda()], dev["v"][rows.cuda()],
                                         dev["g_log"][tok.cuda()], dev["beta"][rows.cuda()], n, c, sl,
                                         use_qk_l2norm=True))
    torch.cuda.synchronize()
    o_dec = torch.stack(outs, 1).reshape(N * T, Hv, V)
    tol = TOL[torch.bfloat16]
    assert rel_err(to_np(o_dec), ref["o"]) <= tol
    assert rel_err(to_np(c[sl.long()]), ref["final_state"]) <= tol
    assert rel_err(to_np(o_dec), to_np(o_pre)) <= tol
    assert rel_err(to_np(c[sl.long()]), to_np(s_pre)) <= tol


def test_decode_serving_batch_sampled(gdp):
    """The benchmark's decode batch (256 entries, n=2, Hqk=16 / Hv=32, K=V=128,
    bf16, in-kernel L2 norm, 1024 cache slots, 8 padding entries): sampled
    entries against the oracle, the whole cache against untouched slots."""
    N, n, Hqk, Hv, K, V, S = 256, 2, 16, 32, 128, 128, 1024
    inp = workloads.decode_batch(N, n, Hqk, Hv, K, V, S, pad=8, dtype=torch.bfloat16, l2norm_in_kernel=True,
                                 g_shift=3.0, seed=2024, device="cuda")
    cache0 = inp["state_cache"].clone()
    o = gdp.recurrent_decode(**inp)
    torch.cuda.synchronize()
    idx = inp["state_indices"].cpu().numpy()
    rng = np.random.default_rng(0)
    picks = rng.choice(np.nonzero(idx >= 0)[0], 6, replace=False)
    for i in picks:
        rows = [i * n + j for j in range(n)]
        ref = oracle.decode(to_np(inp["q"][i:i + 1]), to_np(inp["k"][rows]), to_np(inp["v"][rows]),
                            to_np(inp["g_log"][i:i + 1]), to_np(inp["beta"][rows]), n,
                            to_np(cache0[idx[i]:idx[i] + 1]), np.array([0]), use_qk_l2norm=True)
        assert rel_err(to_np(o[i]), ref["o"][0]) <= TOL[torch.bfloat16], f"entry {i}"
        assert rel_err(to_np(inp["state_cache"][idx[i]]), ref["state_cache"][0]) <= TOL[torch.bfloat16]
    untouched = sorted(set(range(S)) - set(int(s) for s in idx if s >= 0))
    assert torch.equal(inp["state_cache"][untouched], cache0[untouched])
    assert torch.all(o[torch.from_numpy(idx < 0).cuda()] == 0)
