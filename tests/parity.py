"""Helpers shared by the GPU parity tests: run the HIP path and the oracle on
the same inputs and compare with  err = max|x - ref| / max(1, rms(ref))."""
import numpy as np
import torch

import oracle

TOL = {torch.float32: 1e-4, torch.bfloat16: 1.5e-2}


def rel_err(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(ref * ref)))
    return float(np.max(np.abs(x - ref))) / max(1.0, rms)


class ErrAcc:
    """rel_err over a tensor compared piece by piece: the max of |x - ref| and
    the rms of ref are taken over every piece seen, as rel_err takes them over
    the whole tensor."""

    def __init__(self):
        self.maxabs, self.ss, self.count = 0.0, 0.0, 0

    def add(self, x, ref):
        x = np.asarray(x, dtype=np.float64)
        ref = np.asarray(ref, dtype=np.float64)
        if ref.size == 0:
            return
        self.maxabs = max(self.maxabs, float(np.max(np.abs(x - ref))))
        self.ss += float(np.sum(ref * ref))
        self.count += ref.size

    def err(self):
        if self.count == 0:
            return 0.0
        return self.maxabs / max(1.0, float(np.sqrt(self.ss / self.count)))


def to_np(t):
    return t.detach().to("cpu", torch.float64).numpy() if t is not None else None


def oracle_run(inp, heads=None, threads=None, dump_vnew=False):
    """Oracle on the same tensors.  `heads` restricts to a list of state
    heads (with their q/k heads), returning results for those heads only."""
    q, k, v = inp["q"], inp["k"], inp["v"]
    g, b = inp["g_log"], inp["beta"]
    s0 = inp.get("initial_state")
    cache = inp.get("state_cache")
    Hv, Hqk = v.shape[1], q.shape[1]
    grp = Hv // Hqk
    if heads is not None:
        heads = list(heads)
        qk_heads = sorted({h // grp for h in heads})
        # keep the grouping: the selected state heads must cover whole groups
        assert len(heads) == len(qk_heads) * grp and all(h // grp in qk_heads for h in heads)
        q = q[:, qk_heads]
        k = k[:, qk_heads]
        v = v[:, heads]
        g = g[:, heads]
        b = b[:, heads]
        s0 = s0[:, heads] if s0 is not None else None
        cache = cache[:, heads] if cache is not None else None
    return oracle.prefill(to_np(q), to_np(k), to_np(v), to_np(g), to_np(b), inp["num_householder"],
                          inp["cu_seqlens"].cpu().numpy(), scale=inp.get("scale"),
                          initial_state=to_np(s0), use_qk_l2norm=inp.get("use_qk_l2norm", False),
                          return_chunk_states=inp.get("return_chunk_states", False),
                          state_cache=to_np(cache), state_indices=(
                              inp["state_indices"].cpu().numpy() if inp.get("state_indices") is not None else None),
                          dump_vnew=dump_vnew, threads=threads)


def to_device(inp, device="cuda"):
    out = {}
    for key, val in inp.items():
        out[key] = val.to(device) if isinstance(val, torch.Tensor) else val
    return out
