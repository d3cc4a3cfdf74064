"""The FlashInfer-convention entry point (gdp_chunk_gated_delta_product) against
the oracle's FlashInfer front end, element by element, through the C ABI
(needs a gfx950 GPU)."""
import pytest
import torch

import oracle
from gated_deltaproduct_recurrence_amd import workloads
from tests.parity import rel_err, to_np

pytestmark = pytest.mark.gpu

TOL = 1.5e-2  # bf16 inputs


@pytest.fixture(scope="module")
def gdp():
    from gated_deltaproduct_recurrence_amd import binding
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return binding


def run_both(gdp, inp, output_final_state=True, state_dtype=torch.float32, scale=None):
    ref = oracle.prefill_flashinfer(
        to_np(inp["q"]), to_np(inp["k"]), to_np(inp["v"]), to_np(inp["g"]), to_np(inp["beta"]),
        inp["num_householder"], scale=scale, initial_state=to_np(inp["initial_state"]),
        output_final_state=output_final_state, cu_seqlens=inp["cu_seqlens"].numpy(),
        use_qk_l2norm_in_kernel=inp["use_qk_l2norm_in_kernel"])
    dev = {key: (val.cuda() if isinstance(val, torch.Tensor) else val) for key, val in inp.items()}
    T, Hv, d = dev["q"].shape[0], dev["v"].shape[1], dev["q"].shape[2]
    N = dev["cu_seqlens"].shape[0] - 1
    out = torch.full((T, Hv, d), float("nan"), dtype=dev["q"].dtype, device="cuda")
    fs = torch.full((N, Hv, d, d), float("nan"), dtype=state_dtype, device="cuda") if output_final_state else None
    res = gdp.chunk_gated_delta_product(scale=scale, output_final_state=output_final_state, output=out,
                                        output_state=fs, **dev)
    torch.cuda.synchronize()
    if output_final_state:
        o, f = res
        assert o.data_ptr() == out.data_ptr() and f.data_ptr() == fs.data_ptr(), "preallocated buffers not used"
    else:
        o, f = res, None
        assert o.data_ptr() == out.data_ptr()
    return o, f, ref


CASES = [
    # lens, n, Hq, Hk, Hv, d, g dtype, beta dtype, init (std, dtype), l2norm
    ([37, 64, 200, 511], 2, 2, 2, 4, 128, torch.float32, torch.float32, (0.1, torch.float32), False),
    ([150, 3, 97], 3, 2, 4, 4, 128, torch.bfloat16, torch.bfloat16, (0.1, torch.bfloat16), True),
    ([130, 65], 1, 1, 2, 2, 64, torch.float16, None, (0.0, None), False),
    ([33, 0, 200], 2, 1, 1, 2, 64, None, torch.float32, (0.2, torch.float32), True),
]
# float16 q/k/v (restated as bfloat16 operands; beta in q's dtype)
HALF_CASES = [
    ([37, 64, 200, 511], 2, 2, 2, 4, 128, torch.float16, torch.float16, (0.1, torch.float32), True),
    ([150, 3, 97], 3, 2, 4, 4, 64, torch.float32, None, (0.0, None), False),
]
PATHS = ["fused", "split", "segmented"]


@pytest.mark.parametrize("kpath", PATHS)
@pytest.mark.parametrize("ci", range(len(CASES)))
def test_flashinfer_parity(gdp, ci, kpath, monkeypatch):
    lens, n, Hq, Hk, Hv, d, gdt, bdt, (istd, sdt), l2 = CASES[ci]
    monkeypatch.setenv("GDP_PREFILL_PATH", kpath)
    inp = workloads.flashinfer_batch(lens, n, Hq, Hk, Hv, d, g_dtype=gdt, beta_dtype=bdt, init_std=istd,
                                     state_dtype=sdt or torch.float32, l2norm_in_kernel=l2, g_shift=1.0, seed=ci)
    o, f, ref = run_both(gdp, inp, state_dtype=sdt or torch.float32)
    e1, e2 = rel_err(to_np(o), ref["o"]), rel_err(to_np(f), ref["final_state"])
    assert e1 <= TOL and e2 <= TOL, f"case {ci} {kpath}: o {e1:.3e} final state {e2:.3e}"


@pytest.mark.parametrize("ci", range(len(HALF_CASES)))
def test_flashinfer_float16_inputs(gdp, ci):
    lens, n, Hq, Hk, Hv, d, gdt, bdt, (istd, sdt), l2 = HALF_CASES[ci]
    inp = workloads.flashinfer_batch(lens, n, Hq, Hk, Hv, d, dtype=torch.float16, g_dtype=gdt, beta_dtype=bdt,
                                     init_std=istd, state_dtype=sdt or torch.float32, l2norm_in_kernel=l2,
                                     g_shift=1.0, seed=50 + ci)
    o, f, ref = run_both(gdp, inp, state_dtype=sdt or torch.float32)
    assert o.dtype == torch.float16
    e1, e2 = rel_err(to_np(o), ref["o"]), rel_err(to_np(f), ref["final_state"])
    assert e1 <= TOL and e2 <= TOL, f"half case {ci}: o {e1:.3e} final state {e2:.3e}"


def test_flashinfer_no_final_state_and_scale(gdp):
    inp = workloads.flashinfer_batch([100, 28], 2, 2, 2, 4, 128, init_std=0.1, seed=5)
    o, f, ref = run_both(gdp, inp, output_final_state=False, scale=0.5)
    assert f is None
    assert rel_err(to_np(o), ref["o"]) <= TOL


def test_flashinfer_matches_megatron_entry(gdp):
    """The same problem through both entry points: log decays and K-major states
    on one side, linear decays and V-major states on the other."""
    inp = workloads.flashinfer_batch([300, 77], 2, 2, 2, 4, 128, init_std=0.1, seed=9)
    dev = {key: (val.cuda() if isinstance(val, torch.Tensor) else val) for key, val in inp.items()}
    o1, f1 = gdp.chunk_gated_delta_product(output_final_state=True, **dev)
    o2, f2 = gdp.chunk_prefill(dev["q"], dev["k"], dev["v"], torch.log(dev["g"]), dev["beta"], 2, dev["cu_seqlens"],
                               initial_state=dev["initial_state"].transpose(2, 3).contiguous(), output_final_state=True)
    torch.cuda.synchronize()
    assert rel_err(to_np(o1), to_np(o2)) <= 1e-2
    assert rel_err(to_np(f1), to_np(f2.transpose(2, 3))) <= 1e-2
