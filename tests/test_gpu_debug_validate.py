"""The opt-in device checks of the data-dependent arguments (GDP_DEBUG_VALIDATE=1):
each kind of bad cu_seqlens / state_indices sets its bit of the debug word, valid
calls set none, and nothing is checked without the variable (needs a gfx950 GPU).

Every bad value used here stays in bounds in the kernels: sequence ranges are
clamped to [0, T] and cache slots outside [0, slots) are skipped."""
import pytest
import torch

from gated_deltaproduct_recurrence_amd import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gdp():
    from gated_deltaproduct_recurrence_amd import binding
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return binding


def prefill_inputs(T=64, Hqk=1, Hv=2, K=64, V=64, seed=0):
    g = torch.Generator().manual_seed(seed)
    q = torch.nn.functional.normalize(torch.randn(T, Hqk, K, generator=g), dim=-1)
    k = torch.nn.functional.normalize(torch.randn(T, Hqk, K, generator=g), dim=-1)
    v = torch.randn(T, Hv, V, generator=g)
    g_log = -torch.nn.functional.softplus(torch.randn(T, Hv, generator=g))
    beta = torch.sigmoid(torch.randn(T, Hv, generator=g))
    cast = dict(q=q.to(torch.bfloat16), k=k.to(torch.bfloat16), v=v.to(torch.bfloat16), g_log=g_log, beta=beta)
    return {name: x.cuda() for name, x in cast.items()}


def run_prefill(gdp, inp, cu, slots=None, nslots=4):
    cu_t = torch.tensor(cu, dtype=torch.int32, device="cuda")
    Hv, K, V = inp["v"].shape[1], inp["q"].shape[2], inp["v"].shape[2]
    cache = torch.zeros(nslots, Hv, K, V, dtype=torch.float32, device="cuda") if slots is not None else None
    idx = torch.tensor(slots, dtype=torch.int32, device="cuda") if slots is not None else None
    gdp.chunk_prefill(inp["q"], inp["k"], inp["v"], inp["g_log"], inp["beta"], 1, cu_t,
                      state_cache=cache, state_indices=idx)
    return gdp.gdp_debug_status(clear=True)


@pytest.fixture
def validating(monkeypatch, gdp):
    monkeypatch.setenv("GDP_DEBUG_VALIDATE", "1")
    gdp.gdp_debug_status(clear=True)
    yield
    gdp.gdp_debug_status(clear=True)


def test_valid_calls_record_nothing(gdp, validating):
    inp = prefill_inputs()
    assert run_prefill(gdp, inp, [0, 40, 64]) == 0
    assert run_prefill(gdp, inp, [0, 40, 64], slots=[1, 3]) == 0
    assert run_prefill(gdp, inp, [0, 0, 64, 64], slots=[-1, 0, -1]) == 0  # -1: no write, repeated -1 is fine


def test_bad_cu_seqlens(gdp, validating):
    inp = prefill_inputs()
    assert run_prefill(gdp, inp, [0, 40, 30, 64]) == gdp.GDP_DBG_CU  # decreases
    assert run_prefill(gdp, inp, [0, 40, 70]) == gdp.GDP_DBG_CU      # past T
    assert run_prefill(gdp, inp, [-1, 40, 64]) == gdp.GDP_DBG_CU     # below 0


def test_bad_state_indices(gdp, validating):
    inp = prefill_inputs()
    assert run_prefill(gdp, inp, [0, 40, 64], slots=[2, 2]) == gdp.GDP_DBG_DUP
    assert run_prefill(gdp, inp, [0, 40, 64], slots=[4, 0]) == gdp.GDP_DBG_SLOT   # past the 4 slots
    assert run_prefill(gdp, inp, [0, 40, 64], slots=[-2, 0]) == gdp.GDP_DBG_SLOT  # below -1
    both = run_prefill(gdp, inp, [0, 40, 30, 64], slots=[1, 9, 1])
    assert both == gdp.GDP_DBG_CU | gdp.GDP_DBG_SLOT | gdp.GDP_DBG_DUP


def test_decode_duplicate_and_out_of_range_slots(gdp, validating):
    inp = workloads.decode_batch(6, 2, 1, 2, 128, 128, 8, dtype=torch.bfloat16, seed=3)
    dev = {k: (v.to("cuda") if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    gdp.recurrent_decode(**dev)
    assert gdp.gdp_debug_status(clear=True) == 0
    idx = dev["state_indices"].to(torch.int64).clone()
    idx[1] = idx[0] if idx[0] >= 0 else 0
    idx[0] = idx[1]
    idx[4] = 8  # past the cache
    dev["state_indices"] = idx
    gdp.recurrent_decode(**dev)
    assert gdp.gdp_debug_status(clear=True) == gdp.GDP_DBG_DUP | gdp.GDP_DBG_SLOT


def test_no_check_without_the_variable(gdp, monkeypatch):
    monkeypatch.delenv("GDP_DEBUG_VALIDATE", raising=False)
    gdp.gdp_debug_status(clear=True)
    inp = prefill_inputs()
    assert run_prefill(gdp, inp, [0, 40, 30, 64], slots=[1, 1, 9]) == 0
