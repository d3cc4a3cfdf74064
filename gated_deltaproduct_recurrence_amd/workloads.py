"""Seeded synthetic inputs for chunked GDP prefill and the decode step.

Input generation only -- this module holds none of the method's arithmetic.
It serves both the GPU path's tests and benchmark and the oracle-side checks
(the same tensors go to both).  The distributions are the ones stated for the
five workloads: q, k ~ N(0,1) (unit-normalised rows when the in-kernel L2 norm
is off), v ~ N(0,1), g_log = -softplus(N(0,1) - shift) (so alpha = exp(g_log)
lies in (0,1)), beta = sigmoid(N(0,1)), initial states ~ N(0, sigma^2).

Generation order is fixed: lengths and slot indices, q, k, v, g, beta,
initial state, cache sentinel; seed = 1000 + workload id.  Large workloads are
drawn on the device with torch's device generator.
"""
from dataclasses import dataclass, field

import torch

CHUNK = 64


@dataclass
class Workload:
    name: str
    lens: list
    n: int
    Hqk: int
    Hv: int
    K: int
    V: int
    dtype: torch.dtype
    l2norm_in_kernel: bool
    g_shift: float = 0.0
    init_std: float = 0.0          # 0 -> no initial state
    output_final_state: bool = True
    scale: float = None
    state_cache_slots: int = 0     # 0 -> no state cache
    pad_sequences: int = 0         # zero-length sequences appended (slot -1)
    return_chunk_states: bool = False
    seed: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def T(self):
        return int(sum(self.lens))

    @property
    def N(self):
        return len(self.lens) + self.pad_sequences


def _lens_c3(gen):
    return (torch.randint(1, 4097, (64,), generator=gen, device=gen.device)).cpu().tolist()


def workload(wid, device="cpu"):
    """Workload `wid` (0..4) with its lengths drawn (for the random-length mix)."""
    if wid == 0:
        return Workload("single sequence L=128, n=2, H=2, K=V=64, fp32", [128], 2, 2, 2, 64, 64,
                        torch.float32, False, scale=1.0 / 8.0, seed=1000)
    if wid == 1:
        return Workload("varlen lengths {37,64,200,511}, n=2, H=4, K=V=128, bf16", [37, 64, 200, 511], 2, 4, 4,
                        128, 128, torch.bfloat16, False, init_std=0.1, seed=1001)
    if wid == 2:
        return Workload("single sequence L=32768, n=1, H=16, K=V=128, bf16, in-kernel L2 norm", [32768], 1, 16, 16,
                        128, 128, torch.bfloat16, True, g_shift=2.0, output_final_state=False, seed=1002)
    if wid == 3:
        gen = torch.Generator(device="cpu").manual_seed(1003)
        lens = _lens_c3(gen)
        return Workload("serving mix: 64 sequences L~U[1,4096] + 4 padding, n=3, H=32, K=V=128, bf16, "
                        "state cache + chunk states", lens, 3, 32, 32, 128, 128, torch.bfloat16, False,
                        output_final_state=False, state_cache_slots=128, pad_sequences=4,
                        return_chunk_states=True, seed=1003)
    if wid == 4:
        return Workload("long-context prefill: 8 x 65536 tokens, n=2, Hqk=16 / Hv=32, K=V=128, bf16, "
                        "in-kernel L2 norm", [65536] * 8, 2, 16, 32, 128, 128, torch.bfloat16, True, g_shift=3.0,
                        init_std=0.1, seed=1004)
    raise ValueError(wid)


def custom(lens, n, Hqk, Hv, K, V, dtype=torch.bfloat16, l2norm_in_kernel=False, g_shift=0.0, init_std=0.1,
           seed=7, **kw):
    return Workload("custom", list(lens), n, Hqk, Hv, K, V, dtype, l2norm_in_kernel, g_shift=g_shift,
                    init_std=init_std, seed=seed, **kw)


def _unit_rows(x):
    return x / x.norm(dim=-1, keepdim=True)


def generate(w: Workload, device="cpu"):
    """Draw the inputs of workload `w` on `device`.  Returns a dict of tensors
    and flags ready for the library's chunk_prefill front end."""
    dev = torch.device(device)
    gen = torch.Generator(device=dev).manual_seed(w.seed)
    lens = list(w.lens) + [0] * w.pad_sequences
    cu = torch.tensor([0] + list(torch.tensor(lens).cumsum(0).tolist()), dtype=torch.int32, device=dev)
    N = len(lens)
    slots = None
    if w.state_cache_slots:
        perm = torch.randperm(w.state_cache_slots, generator=torch.Generator().manual_seed(w.seed))
        slots = torch.cat([perm[:N - w.pad_sequences], torch.full((w.pad_sequences,), -1)]).to(torch.int32).to(dev)
    T, n = w.T, w.n

    def randn(*shape):
        return torch.randn(*shape, generator=gen, device=dev, dtype=torch.float32)

    q = randn(T, w.Hqk, w.K)
    k = randn(T * n, w.Hqk, w.K)
    if not w.l2norm_in_kernel:
        q = _unit_rows(q)
        k = _unit_rows(k)
    q = q.to(w.dtype)
    k = k.to(w.dtype)
    v = randn(T * n, w.Hv, w.V).to(w.dtype)
    g = -torch.nn.functional.softplus(randn(T, w.Hv) - w.g_shift)
    beta = torch.sigmoid(randn(T * n, w.Hv))
    s0 = (w.init_std * randn(N, w.Hv, w.K, w.V)) if w.init_std > 0 else None
    cache = randn(w.state_cache_slots, w.Hv, w.K, w.V) if w.state_cache_slots else None
    return dict(q=q, k=k, v=v, g_log=g, beta=beta, num_householder=n, cu_seqlens=cu, scale=w.scale,
                initial_state=s0, output_final_state=w.output_final_state, use_qk_l2norm=w.l2norm_in_kernel,
                state_cache=cache, state_indices=slots, return_chunk_states=w.return_chunk_states)


def decode_batch(N, n, Hqk, Hv, K, V, slots, pad=0, dtype=torch.bfloat16, l2norm_in_kernel=False, g_shift=0.0,
                 cache_std=0.3, seed=11, device="cpu"):
    """Inputs of one decode step for N entries: one token (n sub-rows) each, a
    state cache of `slots` rows ~ N(0, cache_std^2), and state indices that are a
    seeded permutation of the slots with `pad` entries set to -1 at seeded
    positions.  Distributions as for the prefill workloads."""
    dev = torch.device(device)
    gen = torch.Generator(device=dev).manual_seed(seed)
    cpu_gen = torch.Generator().manual_seed(seed)
    idx = torch.randperm(slots, generator=cpu_gen)[:N].to(torch.int32)
    if pad:
        idx[torch.randperm(N, generator=cpu_gen)[:pad]] = -1
    idx = idx.to(dev)

    def randn(*shape):
        return torch.randn(*shape, generator=gen, device=dev, dtype=torch.float32)

    q = randn(N, Hqk, K)
    k = randn(N * n, Hqk, K)
    if not l2norm_in_kernel:
        q = _unit_rows(q)
        k = _unit_rows(k)
    v = randn(N * n, Hv, V)
    g = -torch.nn.functional.softplus(randn(N, Hv) - g_shift)
    beta = torch.sigmoid(randn(N * n, Hv))
    cache = cache_std * randn(slots, Hv, K, V)
    return dict(q=q.to(dtype), k=k.to(dtype), v=v.to(dtype), g_log=g, beta=beta, num_householder=n,
                state_cache=cache, state_indices=idx, use_qk_l2norm=l2norm_in_kernel)


def flashinfer_batch(lens, n, Hq, Hk, Hv, d, dtype=torch.bfloat16, l2norm_in_kernel=False, g_shift=0.0,
                     g_dtype=torch.float32, beta_dtype=torch.float32, init_std=0.0, state_dtype=torch.float32,
                     seed=17, device="cpu"):
    """Inputs in the FlashInfer convention: q [T, Hq, d], k [T*n, Hk, d],
    v [T*n, Hv, d], g = alpha = exp(-softplus(N(0,1) - shift)) in (0, 1)
    (g_dtype None: absent), beta = sigmoid(N(0,1)) (beta_dtype None: absent),
    V-major initial states ~ N(0, init_std^2) (init_std 0: absent).  Same
    distributions as the prefill workloads."""
    dev = torch.device(device)
    gen = torch.Generator(device=dev).manual_seed(seed)
    cu = torch.tensor([0] + list(torch.tensor(list(lens)).cumsum(0).tolist()), dtype=torch.int32, device=dev)
    T, N = int(sum(lens)), len(lens)

    def randn(*shape):
        return torch.randn(*shape, generator=gen, device=dev, dtype=torch.float32)

    q = randn(T, Hq, d)
    k = randn(T * n, Hk, d)
    if not l2norm_in_kernel:
        q = _unit_rows(q)
        k = _unit_rows(k)
    v = randn(T * n, Hv, d)
    alpha = torch.exp(-torch.nn.functional.softplus(randn(T, Hv) - g_shift))
    beta = torch.sigmoid(randn(T * n, Hv))
    s0 = init_std * randn(N, Hv, d, d) if init_std > 0 else None
    return dict(q=q.to(dtype), k=k.to(dtype), v=v.to(dtype), g=None if g_dtype is None else alpha.to(g_dtype),
                beta=None if beta_dtype is None else beta.to(beta_dtype), num_householder=n, cu_seqlens=cu,
                initial_state=None if s0 is None else s0.to(state_dtype), use_qk_l2norm_in_kernel=l2norm_in_kernel)
