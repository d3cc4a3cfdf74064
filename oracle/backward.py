"""fp64 CPU oracle for the gradients of the GDP prefill (test infrastructure only).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers; the library path never imports it.

The pages give no backward formulas.  The blog page "Attention Cache and
Sequence Parallelism" only notes, in its section on why training differs, that
activations are kept for backward or recomputed by checkpointing, and, in the
section "GDN: pass the state, not the KV", that the backward dependencies run
in the opposite direction.
So the gradients here are those of the forward recurrence itself, written as
a plain fp64 token loop in PyTorch CPU ops (FlashInfer docs,
"flashinfer.gdp_prefill.chunk_gated_delta_product", the recurrence display, in
the K-major orientation the library uses) and differentiated by
torch.autograd.  The loop restates the recurrence step by step:

    S <- exp(g_log_t) S;  for j: e = beta (v - S^T k), S <- S + k e^T;
    o_t = scale S^T q_t

with the optional per-row L2 normalisation x / sqrt(sum x^2 + 1e-6) of q and k.
Pinned by central finite differences and against the C oracle's forward
(tests/oracle_pins.py).
"""
import math

import numpy as np
import torch


def _t(x):
    return torch.as_tensor(np.asarray(x, dtype=np.float64), dtype=torch.float64)


def forward_torch(q, k, v, g_log, beta, n, cu_seqlens, scale=None, initial_state=None, use_qk_l2norm=False):
    """The forward token loop on fp64 tensors (autograd-capable).  Shapes as for
    oracle.prefill, with k [T*n, Hk, K] (Hk = Hqk or Hv).  Returns (o, final_state)."""
    T, Hq, K = q.shape
    Hk, Hv, V = k.shape[1], v.shape[1], v.shape[2]
    sc = 1.0 / math.sqrt(K) if not scale else float(scale)
    gq, gk = Hv // Hq, Hv // Hk
    if use_qk_l2norm:
        q = q / torch.sqrt((q * q).sum(-1, keepdim=True) + 1e-6)
        k = k / torch.sqrt((k * k).sum(-1, keepdim=True) + 1e-6)
    qh = q[:, torch.arange(Hv) // gq]   # [T, Hv, K]: the q head each state head reads
    kh = k[:, torch.arange(Hv) // gk]   # [T*n, Hv, K]
    outs, finals = [], []
    cu = [int(x) for x in cu_seqlens]
    for i in range(len(cu) - 1):
        S = torch.zeros(Hv, K, V, dtype=torch.float64) if initial_state is None else initial_state[i]
        for t in range(cu[i], cu[i + 1]):
            S = torch.exp(g_log[t])[:, None, None] * S
            for j in range(n):
                r = t * n + j
                kr = kh[r]                                               # [Hv, K]
                e = beta[r][:, None] * (v[r] - torch.einsum("hkv,hk->hv", S, kr))
                S = S + kr[:, :, None] * e[:, None, :]
            outs.append(sc * torch.einsum("hkv,hk->hv", S, qh[t]))
        finals.append(S)
    o = torch.stack(outs) if outs else torch.zeros(0, Hv, V, dtype=torch.float64)
    return o, torch.stack(finals) if finals else torch.zeros(0, Hv, K, V, dtype=torch.float64)


def backward(q, k, v, g_log, beta, num_householder, cu_seqlens, do, dfinal_state=None, scale=None,
             initial_state=None, use_qk_l2norm=False):
    """Gradients of <o, do> + <final_state, dfinal_state> with respect to every
    input.  Returns a dict of numpy fp64 arrays: dq, dk, dv, dg_log, dbeta and
    dinitial_state (None without an initial state)."""
    args = [_t(x).requires_grad_(True) for x in (q, k, v, g_log, beta)]
    s0 = None if initial_state is None else _t(initial_state).requires_grad_(True)
    o, fin = forward_torch(*args, int(num_householder), cu_seqlens, scale=scale, initial_state=s0,
                           use_qk_l2norm=use_qk_l2norm)
    loss = (o * _t(do)).sum()
    if dfinal_state is not None:
        loss = loss + (fin * _t(dfinal_state)).sum()
    inputs = args + ([s0] if s0 is not None else [])
    grads = torch.autograd.grad(loss, inputs, allow_unused=True)
    names = ["dq", "dk", "dv", "dg_log", "dbeta"]
    out = {}
    for name, x, gr in zip(names, args, grads):
        out[name] = (gr if gr is not None else torch.zeros_like(x)).detach().numpy()
    out["dinitial_state"] = grads[5].detach().numpy() if s0 is not None else None
    return out
