"""Throughput of chunked Gated DeltaProduct prefill on one MI355X.

Workload: the long-context prefill -- 8 sequences x 65536 tokens (524,288 real
tokens), n = 2 Householder rows per token, 16 q/k heads shared by 32 state
heads, K = V = 128, bf16 q/k/v, fp32 g/beta/state, q/k L2-normalised in the
kernel, random initial state, final state returned.  Inputs are seeded
synthetic tensors resident in HBM before timing starts.

One step = one whole forward pass over the batch: the descriptor build and
the prefill (both C-ABI calls, on torch's current stream).
Prints one JSON line (metric, throughput in real tokens/s, roofline of the
dominant kernel measured with HIP events on its stream, and the CPU oracle's
rate on a bounded sample).
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_long_context_traffic.json")
KERNEL_SOURCES = [os.path.join(ROOT, "gated_deltaproduct_recurrence_amd", "csrc", f)
                  for f in ("gdp_kernels.hip", "gdp_common.h")]


def algorithmic_bytes(w, slots=None):
    """Each input read once, each output written once, no intermediates.
    Per real token: q, k (Hqk*K*(1+n) bf16), v, o (Hv*V*(1+n) bf16), g, beta
    (Hv*(1+n) fp32); per sequence: initial and final state (Hv*K*V fp32 each);
    per 64-token chunk when chunk states are returned, and per cache slot
    written (a state index >= 0), one more Hv*K*V fp32 state."""
    es = 2 if str(w.dtype).endswith("bfloat16") else 4
    state = 4 * w.Hv * w.K * w.V
    per_tok = es * w.K * w.Hqk * (1 + w.n) + es * w.V * w.Hv * (1 + w.n) + 4 * w.Hv * (1 + w.n)
    per_seq = state * ((1 if w.init_std > 0 else 0) + (1 if w.output_final_state else 0))
    total = per_tok * w.T + per_seq * w.N
    if w.return_chunk_states:
        total += state * sum((L + 63) // 64 for L in w.lens)
    if slots is not None:
        total += state * int(sum(1 for s in slots if 0 <= s < w.state_cache_slots))
    return total


# parity bar of the oracle checks: max|x - ref| / max(1, rms(ref)) over the sample
TOL = {"f32": 1e-4, "bf16": 1.5e-2}


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or the platform's processor string."""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def check_against_oracle(what, err, tol):
    """A GPU result outside the parity bar fails the run (no JSON line is printed)."""
    print(f"bench: {what} vs oracle err {err:.3e} (tolerance {tol:.1e})", file=sys.stderr)
    if not err <= tol:
        print(f"bench: {what} is outside the tolerance: the run fails", file=sys.stderr)
        sys.exit(1)


def source_hash():
    """Hash of the fused kernel's sources and of the compiler flags they are built with."""
    from gated_deltaproduct_recurrence_amd import build as kbuild
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    h.update(" ".join(kbuild.DEVICE_FLAGS + kbuild.SOURCE_FLAGS.get("gdp_kernels.hip", [])).encode())
    return h.hexdigest()[:16]


def measured_traffic(wid):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary, if it was taken on the current kernel source and on this workload
    (the counters were taken on the long-context prefill, workload 4); else None."""
    if wid != 4:
        return None
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != source_hash():
        return None
    return rec.get("traffic_bytes_per_launch")


def kernel_label(w):
    """Kernel(s) the library runs for this workload (the same rule as the
    library's path choice; GDP_PREFILL_PATH=fused|split|segmented forces one):
    the fused single kernel for bf16 inputs with at least 256 (sequence, state
    head) chains; for fewer chains of long sequences (bf16, K == V) the fused
    kernel on segments plus the segment combine; otherwise the WY + scan pair."""
    import torch
    forced = os.environ.get("GDP_PREFILL_PATH")
    bf16 = w.dtype == torch.bfloat16
    chains = w.N * w.Hv
    if bf16 and w.K == w.V and w.K in (64, 128) and forced not in ("fused", "split"):
        avg = -(-w.T // max(w.N, 1))
        target = max(2, 256 // max(chains, 1))
        L = max(256, (-(-avg // target) + 63) // 64 * 64)
        if forced == "segmented" or (chains < 256 and avg >= 2 * L):
            return "gdp_fused_kernel on segments + gdp_combine_kernel"
    fused = bf16 and (forced == "fused" or (forced != "split" and chains >= 256))
    return "gdp_fused_kernel" if fused else "gdp_wy_kernel + gdp_scan_kernel"


def copy_bandwidth(dev, reps=5):
    """Read + write bytes per second of a plain 1 GiB device-to-device copy on
    this GPU (torch's copy kernel), timed with HIP events: a practical ceiling
    next to the 8 TB/s peak."""
    import torch
    src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbs = 2.0 * src.numel() * 4 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return gbs


def cpu_baseline(inp, w, tokens_per_seq, threads):
    """The fp64 oracle on the first `tokens_per_seq` tokens of every sequence
    (all heads), timed on the host cores; returns (record, oracle outputs)."""
    import torch

    import oracle
    n = w.n
    cu = inp["cu_seqlens"].cpu().numpy()
    idx_t, idx_s = [], []
    for i in range(w.N):
        t0 = int(cu[i])
        L = min(tokens_per_seq, int(cu[i + 1]) - t0)
        idx_t.append(np.arange(t0, t0 + L))
        idx_s.append(np.arange(t0 * n, (t0 + L) * n))
    it = torch.tensor(np.concatenate(idx_t), device=inp["q"].device)
    isub = torch.tensor(np.concatenate(idx_s), device=inp["q"].device)

    def host(x, rows):
        return x.index_select(0, rows).to("cpu", torch.float64).numpy()

    q, k, v = host(inp["q"], it), host(inp["k"], isub), host(inp["v"], isub)
    g, b = host(inp["g_log"], it), host(inp["beta"], isub)
    lens = [len(x) for x in idx_t]
    cus = np.concatenate([[0], np.cumsum(lens)])
    s0 = inp["initial_state"].cpu().double().numpy() if inp["initial_state"] is not None else None
    t_start = time.perf_counter()
    ref = oracle.prefill(q, k, v, g, b, n, cus, initial_state=s0, use_qk_l2norm=w.l2norm_in_kernel,
                         threads=threads)
    dt = time.perf_counter() - t_start
    rec = {"value": float(cus[-1] / dt), "unit": "tokens/s", "cores": threads, "cpu_model": cpu_model(), "kind": "oracle",
           "sample": f"first {tokens_per_seq} tokens of each of the {w.N} sequences, all {w.Hv} heads "
                     f"({int(cus[-1])} real tokens), fp64 token loop, {dt:.2f} s"}
    return rec, ref, it


def bench_decode(args, gdp, workloads):
    """One decode step per timed step on the serving batch; HBM-bound (each live
    entry reads and writes its Hv K x V fp32 states once)."""
    import torch
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    N, n, Hqk, Hv, K, V, S, pad = 256, 2, 16, 32, 128, 128, 1024, 8
    inp = workloads.decode_batch(N, n, Hqk, Hv, K, V, S, pad=pad, dtype=torch.bfloat16, l2norm_in_kernel=True,
                                 g_shift=3.0, seed=2024, device="cuda")
    o = torch.empty((N, Hv, V), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        gdp.gdp_recurrent_decode(inp["q"], inp["k"], inp["v"], inp["g_log"], inp["beta"], n, 0.0, True,
                                 inp["state_cache"], inp["state_indices"], o, stream=stream.cuda_stream)

    rec = None
    if not args.no_cpu_baseline:
        # the oracle on every live entry of the step, with the cache cut down to
        # their slots; the GPU output of the same step (from the same cache) is
        # checked against it before the timed steps change the cache
        import oracle
        idx = inp["state_indices"]
        sel = torch.nonzero(idx >= 0).flatten()
        rows = (sel[:, None] * n + torch.arange(n, device=dev)).flatten()
        f64 = lambda x: x.to("cpu", torch.float64).numpy()
        args_o = (f64(inp["q"][sel]), f64(inp["k"][rows]), f64(inp["v"][rows]), f64(inp["g_log"][sel]),
                  f64(inp["beta"][rows]), n, f64(inp["state_cache"][idx[sel].long()]),
                  np.arange(sel.numel(), dtype=np.int32))
        step()
        torch.cuda.synchronize()
        got = o.index_select(0, sel).to("cpu", torch.float64).numpy()
        threads = args.cpu_threads or max(1, min(16, os.cpu_count() or 1))
        reps = 10  # the step is small: repeated for a stable rate
        t0 = time.perf_counter()
        for _ in range(reps):
            ref = oracle.decode(*args_o, use_qk_l2norm=True, threads=threads)
        dt = (time.perf_counter() - t0) / reps
        err = float(np.max(np.abs(got - ref["o"]))) / max(1.0, float(np.sqrt(np.mean(ref["o"] ** 2))))
        check_against_oracle("decode outputs", err, TOL["bf16"])
        rec = {"value": sel.numel() / dt, "unit": "entries/s", "cores": threads, "cpu_model": cpu_model(),
               "kind": "oracle",
               "sample": f"all {sel.numel()} live entries of one step, all {Hv} heads, fp64 "
                         f"(cache cut to their slots), {reps} runs of {dt:.2f} s"}

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    kern_ms = e0.elapsed_time(e1) / args.steps
    live = N - pad
    alg = live * Hv * (2 * K * V * 4 + 4 + 4 * n) + live * (2 * K * Hqk * (1 + n)) + live * Hv * 2 * V * (n + 1)
    achieved = alg / (kern_ms * 1e-3) / 1e9
    line = {"metric": "decode entries/s, single-token GDP decode step on the state cache (bf16, d=128) + % of HBM roofline",
            "value": live / (wall / args.steps), "unit": "entries/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": wall * 1e3 / args.steps, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "serving decode step: 256 entries (8 padding), n=2, Hqk=16 / Hv=32, K=V=128, "
                                   "bf16, in-kernel L2 norm, 1024 cache slots", "entries": N, "padding": pad},
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": achieved / HBM_PEAK_GBS, "traffic": None, "kernel": "gdp_decode_kernel",
                         "kernel_ms": kern_ms, "algorithmic_bytes_per_launch": alg},
            "cpu_baseline": rec}
    print(json.dumps(line), flush=True)


def backward_cpu_baseline(args, inp, w, d_o, grads, M=2048, seq=7, hq=5):
    """The fp64 autograd oracle on the last M tokens of sequence `seq` for the
    two state heads of q/k head `hq` (given the state entering the suffix, from
    the forward oracle over the prefix, which is not timed), scaled to all
    heads; also checks the GPU gradients of that sample."""
    import torch

    import oracle
    from oracle import backward as obwd
    n, grp = w.n, w.Hv // w.Hqk
    cu = inp["cu_seqlens"].cpu().numpy()
    t0, t1 = int(cu[seq]), int(cu[seq + 1])
    ts = t1 - M
    heads = list(range(grp * hq, grp * hq + grp))
    f64 = lambda x: x.to("cpu", torch.float64).numpy()
    pre = oracle.prefill(f64(inp["q"][t0:ts, hq:hq + 1]), f64(inp["k"][t0 * n:ts * n, hq:hq + 1]),
                         f64(inp["v"][t0 * n:ts * n, heads]), f64(inp["g_log"][t0:ts, heads]),
                         f64(inp["beta"][t0 * n:ts * n, heads]), n, np.array([0, ts - t0]),
                         initial_state=f64(inp["initial_state"][seq:seq + 1, heads]), use_qk_l2norm=True)
    sub = (f64(inp["q"][ts:t1, hq:hq + 1]), f64(inp["k"][ts * n:t1 * n, hq:hq + 1]), f64(inp["v"][ts * n:t1 * n, heads]),
           f64(inp["g_log"][ts:t1, heads]), f64(inp["beta"][ts * n:t1 * n, heads]), n, np.array([0, M]),
           f64(d_o[ts:t1, heads]), None)
    if args.cpu_threads:
        torch.set_num_threads(args.cpu_threads)
    threads = torch.get_num_threads()
    t_start = time.perf_counter()
    ref = obwd.backward(*sub, initial_state=pre["final_state"], use_qk_l2norm=True)
    dt = time.perf_counter() - t_start
    got = {"dq": grads["dq"][ts:t1, hq:hq + 1], "dk": grads["dk"][ts * n:t1 * n, hq:hq + 1],
           "dv": grads["dv"][ts * n:t1 * n, heads], "dg_log": grads["dg_log"][ts:t1, heads],
           "dbeta": grads["dbeta"][ts * n:t1 * n, heads]}
    for name, x in got.items():
        r = ref[name]
        e = float(np.max(np.abs(f64(x) - r))) / max(1.0, float(np.sqrt(np.mean(r ** 2))))
        check_against_oracle(name, e, TOL["bf16"])
    groups = w.Hqk
    return {"value": M / (dt * groups), "unit": "tokens/s", "cores": threads, "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"last {M} tokens of sequence {seq}, the {grp} state heads of q/k head {hq} (one of {groups} "
                      f"groups; the rate is scaled to all {w.Hv} heads), fp64 autograd token loop given the state "
                      f"entering the suffix, {dt:.2f} s"}


def bench_flashinfer(args, gdp, workloads):
    """The long-context prefill through the FlashInfer-convention entry point:
    linear decays alpha, float32 betas, V-major float32 initial and final states
    (restated by the front end's small kernels around the prefill kernels)."""
    import torch
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lens, n, Hq, Hv, d = [65536] * 8, 2, 16, 32, 128
    inp = workloads.flashinfer_batch(lens, n, Hq, Hq, Hv, d, dtype=torch.bfloat16, l2norm_in_kernel=True,
                                     g_shift=3.0, init_std=0.1, seed=1004, device=dev)
    T, N = sum(lens), len(lens)
    out = torch.empty((T, Hv, d), dtype=torch.bfloat16, device=dev)
    fs = torch.empty((N, Hv, d, d), dtype=torch.float32, device=dev)
    ws = torch.empty(gdp.gdp_fi_workspace_bytes(T, N, n, Hq, Hv, d, torch.bfloat16, True, True), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        gdp.gdp_chunk_gated_delta_product(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], n, None,
                                          inp["initial_state"], True, inp["cu_seqlens"], True, out, fs, ws,
                                          stream=stream.cuda_stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    kern_ms = e0.elapsed_time(e1) / args.steps
    # the op's own bytes: q, k, v, o (bf16), alpha, beta (float32), initial and final states (float32)
    alg = T * (2 * d * Hq * (1 + n) + 2 * d * Hv * (1 + n) + 4 * Hv * (1 + n)) + 2 * 4 * N * Hv * d * d
    achieved = alg / (kern_ms * 1e-3) / 1e9
    line = {"metric": "real tokens/s, chunked GDP prefill in the FlashInfer convention (bf16, d=128) + % of HBM roofline",
            "value": T / (wall / args.steps), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": wall * 1e3 / args.steps, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "long-context prefill in the FlashInfer convention: 8 x 65536 tokens, n=2, "
                                   "Hq=Hk=16 / Hv=32, d=128, bf16, linear alpha, V-major float32 states, "
                                   "in-kernel L2 norm", "real_tokens": T},
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                         "kernel": "gdp_chunk_gated_delta_product (gate and state kernels + gdp_fused_kernel)",
                         "kernel_ms": kern_ms, "algorithmic_bytes_per_launch": alg},
            "cpu_baseline": None}
    copy_gbs = copy_bandwidth(dev)
    line["copy_bound"] = {"copy_GBs": copy_gbs, "achieved_GBs": achieved, "frac": achieved / copy_gbs,
                          "what": "1 GiB device-to-device copy on this GPU, read + write bytes per second"}
    if not args.no_cpu_baseline:
        # the FlashInfer-convention oracle on the first L tokens of every sequence
        # (outputs depend only on the tokens before them), all heads
        import oracle
        L = min(args.cpu_tokens, 32768)
        it = torch.cat([torch.arange(i * lens[0], i * lens[0] + L, device=dev) for i in range(N)])
        isub = torch.cat([torch.arange(i * lens[0] * n, (i * lens[0] + L) * n, device=dev) for i in range(N)])
        host = lambda x, rows: x.index_select(0, rows).to("cpu", torch.float64).numpy()
        sub = (host(inp["q"], it), host(inp["k"], isub), host(inp["v"], isub), host(inp["g"], it),
               host(inp["beta"], isub))
        threads = args.cpu_threads or max(1, min(16, os.cpu_count() or 1))
        t0 = time.perf_counter()
        ref = oracle.prefill_flashinfer(*sub, num_householder=n, initial_state=inp["initial_state"].cpu().double().numpy(),
                                        cu_seqlens=np.arange(N + 1) * L, use_qk_l2norm_in_kernel=True, threads=threads)
        dt = time.perf_counter() - t0
        got = out.index_select(0, it).to("cpu", torch.float64).numpy()
        err = float(np.max(np.abs(got - ref["o"]))) / max(1.0, float(np.sqrt(np.mean(ref["o"] ** 2))))
        check_against_oracle("sampled outputs", err, TOL["bf16"])
        line["cpu_baseline"] = {"value": N * L / dt, "unit": "tokens/s", "cores": threads, "cpu_model": cpu_model(),
                                "kind": "oracle",
                                "sample": f"first {L} tokens of each of the {N} sequences, all {Hv} heads, fp64 "
                                          f"token loop (FlashInfer convention), {dt:.2f} s"}
    print(json.dumps(line), flush=True)


def bench_backward(args, gdp, workloads):
    """Gradients of the long-context prefill (its shape and inputs, one call per
    step: the chunked path's prep, state walk, reverse state-gradient walk and
    per-chunk gradient kernels, or with GDP_BACKWARD_PATH=recurrent the forward
    rerun and the per-token reverse kernel).  The line reports the algorithmic
    HBM bytes (inputs read once, float32 gradients written once) so that the
    fraction shows how far the call is from the bandwidth bound; the chunked
    path also moves the per-chunk states and state gradients through HBM."""
    import torch
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = workloads.workload(4)
    inp = workloads.generate(w, dev)
    T, N, n, Hqk, Hv, K, V = w.T, w.N, w.n, w.Hqk, w.Hv, w.K, w.V
    gen = torch.Generator(device=dev).manual_seed(4242)
    d_o = torch.randn(T, Hv, V, generator=gen, device=dev).to(torch.bfloat16)
    f32 = dict(dtype=torch.float32, device=dev)
    dq, dk = torch.empty((T, Hqk, K), **f32), torch.empty((T * n, Hqk, K), **f32)
    dv, dg, db = torch.empty((T * n, Hv, V), **f32), torch.empty((T, Hv), **f32), torch.empty((T * n, Hv), **f32)
    ds0 = torch.empty((N, Hv, K, V), **f32)
    ws = torch.empty(gdp.gdp_backward_workspace_bytes(T, N, n, Hqk, Hv, K, V), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        gdp.gdp_chunk_prefill_backward(inp["q"], inp["k"], inp["v"], inp["g_log"], inp["beta"], n, inp["cu_seqlens"],
                                       0.0, inp["initial_state"], True, d_o, None, dq, dk, dv, dg, db, ds0, ws,
                                       stream=stream.cuda_stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    kern_ms = e0.elapsed_time(e1) / args.steps
    # read: q, k, v, do (bf16), g, beta, s0; written: dq, dk, dv, dg, dbeta, ds0 (float32)
    alg = (T * (2 * K * Hqk * (1 + n) + 2 * V * Hv * (1 + n) + 4 * Hv * (1 + n)) + 4 * N * Hv * K * V +
           T * 4 * (K * Hqk * (1 + n) + V * Hv * n + Hv * (1 + n)) + 4 * N * Hv * K * V)
    achieved = alg / (kern_ms * 1e-3) / 1e9
    line = {"metric": "real tokens/s, gradients of the chunked GDP prefill (bf16 inputs, float32 gradients) + % of HBM roofline",
            "value": T / (wall / args.steps), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": wall * 1e3 / args.steps, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "backward of the long-context prefill: 8 x 65536 tokens, n=2, Hqk=16 / Hv=32, "
                                   "K=V=128, bf16, in-kernel L2 norm", "real_tokens": T},
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                         "kernel": ("gdp_chunk_prefill_backward (forward rerun + gdp_backward_kernel)"
                                    if os.environ.get("GDP_BACKWARD_PATH") == "recurrent" else
                                    "gdp_chunk_prefill_backward (gdp_bwd_prep, gdp_bwd_state, gdp_bwd_adjoint, "
                                    "gdp_bwd_grad kernels)"),
                         "kernel_ms": kern_ms, "algorithmic_bytes_per_launch": alg},
            "cpu_baseline": None}
    if not args.no_cpu_baseline:
        grads = {"dq": dq, "dk": dk, "dv": dv, "dg_log": dg, "dbeta": db}
        line["cpu_baseline"] = backward_cpu_baseline(args, inp, w, d_o, grads)
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=4, help="workload id (4 = long-context prefill)")
    ap.add_argument("--cpu-tokens", type=int, default=65536, help="oracle sample: tokens per sequence")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="host threads of the oracle baseline (default: the cores, at most 16)")
    ap.add_argument("--graph", action="store_true",
                    help="also capture one step (descriptor build + prefill) in a HIP graph and time its "
                         "replays; the replayed output is checked against the eager one bit for bit")
    ap.add_argument("--decode", action="store_true",
                    help="measure the single-token decode step on the state cache instead of the prefill "
                         "(serving batch: 256 entries with 8 padding, n=2, Hqk=16 / Hv=32, K=V=128, bf16, "
                         "1024 cache slots)")
    ap.add_argument("--flashinfer", action="store_true",
                    help="time the FlashInfer-convention entry point on the long-context shape instead")
    ap.add_argument("--backward", action="store_true",
                    help="measure the gradients of the long-context prefill instead of the forward pass")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (three times); used to scale the "
                         "FETCH_SIZE / WRITE_SIZE counters to bytes")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU; --gpus {args.gpus} is not supported "
              "(the op shards across GPUs by sequence or head with no exchange, which is not built here)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")  # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_each_way": src.numel() * 4, "launches": 3}))
        return

    from gated_deltaproduct_recurrence_amd import binding as gdp
    from gated_deltaproduct_recurrence_amd import workloads

    if args.decode:
        bench_decode(args, gdp, workloads)
        return
    if args.backward:
        bench_backward(args, gdp, workloads)
        return
    if args.flashinfer:
        bench_flashinfer(args, gdp, workloads)
        return

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = workloads.workload(args.workload)
    inp = workloads.generate(w, dev)
    T, N, n = w.T, w.N, w.n
    Hqk, Hv, K, V = w.Hqk, w.Hv, w.K, w.V
    o = torch.empty((T, Hv, V), dtype=w.dtype, device=dev)
    fs = torch.empty((N, Hv, K, V), dtype=torch.float32, device=dev) if w.output_final_state else None
    cache = inp["state_cache"]
    cs = None
    nt_cap, ntdp_cap = gdp.gdp_descriptor_capacity(T, N, n)
    if w.return_chunk_states:
        cs = torch.empty((nt_cap, Hv, K, V), dtype=torch.float32, device=dev)
    desc = {"chunk_indices": torch.empty((max(nt_cap, 1), 2), dtype=torch.int32, device=dev),
            "chunk_indices_dp": torch.empty((max(ntdp_cap, 1), 2), dtype=torch.int32, device=dev),
            "chunk_offsets": torch.empty(N + 1, dtype=torch.int32, device=dev),
            "chunk_offsets_dp": torch.empty(N + 1, dtype=torch.int32, device=dev)}
    d = gdp._descs(desc, nt_cap, ntdp_cap)
    ws = torch.empty(gdp.gdp_workspace_bytes(T, N, n, Hqk, Hv, K, V, w.dtype), dtype=torch.uint8, device=dev)
    cu_t = gdp.as_gdp_tensor(inp["cu_seqlens"])
    import ctypes
    stream = torch.cuda.current_stream(dev)

    def build_desc(st=stream):
        rc = gdp.LIB.gdp_build_descriptors(ctypes.byref(cu_t), n, T, ctypes.byref(d), st.cuda_stream)
        if rc != 0:
            raise gdp.GdpError(rc, gdp.gdp_last_error())

    def prefill(st=stream):
        gdp.gdp_chunk_prefill(inp["q"], inp["k"], inp["v"], inp["g_log"], inp["beta"], n, inp["cu_seqlens"],
                              inp["scale"] or 0.0, inp["initial_state"], w.output_final_state,
                              w.l2norm_in_kernel, cache, inp["state_indices"], w.return_chunk_states, o, fs, cs,
                              desc, ws, stream=st.cuda_stream)

    for _ in range(args.warmup):
        build_desc()
        prefill()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for s in range(args.steps):
        ev[s][0].record(stream)
        build_desc()
        ev[s][1].record(stream)
        prefill()
        ev[s][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    step_ms = [e[0].elapsed_time(e[2]) for e in ev]
    fused_ms = [e[1].elapsed_time(e[2]) for e in ev]
    desc_ms = [e[0].elapsed_time(e[1]) for e in ev]
    ms_per_step = wall * 1e3 / args.steps
    value = T / (ms_per_step * 1e-3)

    graph_detail = None
    if args.graph:
        # one step captured (every grid depends only on host-known sizes), then
        # replayed; the outputs must equal the eager step's
        o_eager = o.clone()
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            build_desc(side)
            prefill(side)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            cap = torch.cuda.current_stream(dev)
            build_desc(cap)
            prefill(cap)
        torch.cuda.synchronize()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t_g = time.perf_counter()
        g0.record(stream)
        for _ in range(args.steps):
            graph.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        wall_g = time.perf_counter() - t_g
        same = bool(torch.equal(o, o_eager))
        if not same:
            print("bench: graph replay output differs from the eager output: the run fails", file=sys.stderr)
            sys.exit(1)
        graph_detail = {"graph_replay_ms_per_step": wall_g * 1e3 / args.steps,
                        "graph_replay_event_ms": g0.elapsed_time(g1) / args.steps,
                        "graph_replay_equals_eager": same}

    alg = algorithmic_bytes(w, None if inp["state_indices"] is None else inp["state_indices"].cpu().tolist())
    fused_avg_s = float(np.mean(fused_ms)) * 1e-3
    achieved = alg / fused_avg_s / 1e9
    traffic = measured_traffic(args.workload)

    line = {
        "metric": "real tokens/s, chunked GDP prefill (bf16, d=128) + % of MFMA/HBM roofline",
        "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.dtype == torch.bfloat16 else "f32", "data": "synthetic",
        "config": {"workload": w.name, "sequences": N, "tokens_per_sequence": w.lens[0] if N else 0,
                   "real_tokens": T, "num_householder": n, "q_k_heads": Hqk, "state_heads": Hv, "K": K,
                   "V": V, "use_qk_l2norm": w.l2norm_in_kernel, "initial_state": w.init_std > 0,
                   "output_final_state": w.output_final_state},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": f"gdp_chunk_prefill ({kernel_label(w)})", "kernel_ms": float(np.mean(fused_ms)),
                     "algorithmic_bytes_per_launch": alg},
        "timing_detail": {"event_step_ms_median": float(np.median(step_ms)),
                          "descriptor_kernel_ms": float(np.mean(desc_ms))},
    }
    if graph_detail is not None:
        line["timing_detail"].update(graph_detail)
    copy_gbs = copy_bandwidth(dev)
    line["copy_bound"] = {"copy_GBs": copy_gbs, "achieved_GBs": achieved, "frac": achieved / copy_gbs,
                          "what": "1 GiB device-to-device copy on this GPU, read + write bytes per second"}
    if not args.no_cpu_baseline:
        threads = args.cpu_threads or max(1, min(16, os.cpu_count() or 1))
        rec, ref, it = cpu_baseline(inp, w, args.cpu_tokens, threads)
        line["cpu_baseline"] = rec
        got = o.index_select(0, it).to("cpu", torch.float64).numpy()
        err = float(np.max(np.abs(got - ref["o"]))) / max(1.0, float(np.sqrt(np.mean(ref["o"] ** 2))))
        check_against_oracle("sampled outputs", err, TOL["bf16" if w.dtype == torch.bfloat16 else "f32"])
        rec["oracle_check_err"] = err
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
