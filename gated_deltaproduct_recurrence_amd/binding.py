"""ctypes binding of libgdp.so (include/gdp.h), same names as the C ABI.

Argument marshalling only: torch supplies device memory and the current
stream; every step of the computation runs in the library's HIP kernels.  If
the library is missing this module raises on import -- there is no fallback.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# GDP_LIBRARY names another build of the library (the host-sanitized check
# build of the CPU sanitizer run); by default the in-tree libgdp.so
LIB_PATH = os.environ.get("GDP_LIBRARY") or os.path.join(_HERE, "libgdp.so")

GDP_F32, GDP_BF16, GDP_I32, GDP_I64, GDP_F16 = 0, 1, 2, 3, 4
GDP_OK, GDP_EINVAL, GDP_EUNSUPPORTED, GDP_EALIAS, GDP_EWORKSPACE, GDP_EHIP = 0, -1, -2, -3, -4, -5
GDP_DBG_CU, GDP_DBG_SLOT, GDP_DBG_DUP = 1, 2, 4
STATUS_NAMES = {GDP_EINVAL: "GDP_EINVAL", GDP_EUNSUPPORTED: "GDP_EUNSUPPORTED", GDP_EALIAS: "GDP_EALIAS",
                GDP_EWORKSPACE: "GDP_EWORKSPACE", GDP_EHIP: "GDP_EHIP"}

EXPORTED = ("gdp_descriptor_capacity", "gdp_build_descriptors", "gdp_workspace_bytes",
            "gdp_chunk_prefill", "gdp_recurrent_decode", "gdp_fi_workspace_bytes",
            "gdp_chunk_gated_delta_product", "gdp_backward_workspace_bytes", "gdp_chunk_prefill_backward",
            "gdp_debug_status", "gdp_last_error", "gdp_version", "gdp_chunk_prefill_noalloc")


class gdp_tensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4), ("stride", ctypes.c_int64 * 4)]


class gdp_descriptors(ctypes.Structure):
    _fields_ = [("chunk_indices", ctypes.c_void_p), ("chunk_indices_dp", ctypes.c_void_p),
                ("chunk_offsets", ctypes.c_void_p), ("chunk_offsets_dp", ctypes.c_void_p),
                ("nt_cap", ctypes.c_int64), ("ntdp_cap", ctypes.c_int64)]


class GdpError(RuntimeError):
    def __init__(self, code, message):
        super().__init__(f"{STATUS_NAMES.get(code, code)}: {message}")
        self.code = code


def _load(path=LIB_PATH):
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run __graft_entry__.build() "
                          "(gated_deltaproduct_recurrence_amd/build.py)")
    lib = ctypes.CDLL(path)
    T = ctypes.POINTER(gdp_tensor)
    D = ctypes.POINTER(gdp_descriptors)
    lib.gdp_descriptor_capacity.restype = ctypes.c_int
    lib.gdp_descriptor_capacity.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                            ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64)]
    lib.gdp_build_descriptors.restype = ctypes.c_int
    lib.gdp_build_descriptors.argtypes = [T, ctypes.c_int32, ctypes.c_int64, D, ctypes.c_void_p]
    lib.gdp_workspace_bytes.restype = ctypes.c_size_t
    lib.gdp_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
    lib.gdp_chunk_prefill.restype = ctypes.c_int
    lib.gdp_chunk_prefill.argtypes = [T, T, T, T, T, ctypes.c_int32, T, ctypes.c_float, T, ctypes.c_int32,
                                      ctypes.c_int32, T, T, ctypes.c_int32, T, T, T, D, ctypes.c_void_p,
                                      ctypes.c_size_t, ctypes.c_void_p]
    lib.gdp_chunk_prefill_noalloc.restype = ctypes.c_int
    lib.gdp_chunk_prefill_noalloc.argtypes = [T, T, T, T, T, ctypes.c_int32, T, ctypes.c_float, T, ctypes.c_int32,
                                              ctypes.c_int32, T, T, ctypes.c_int32, T, T, T, D, ctypes.c_void_p]
    lib.gdp_recurrent_decode.restype = ctypes.c_int
    lib.gdp_recurrent_decode.argtypes = [T, T, T, T, T, ctypes.c_int32, ctypes.c_float, ctypes.c_int32, T, T, T,
                                         ctypes.c_void_p]
    lib.gdp_fi_workspace_bytes.restype = ctypes.c_size_t
    lib.gdp_fi_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_int32]
    lib.gdp_chunk_gated_delta_product.restype = ctypes.c_int
    lib.gdp_chunk_gated_delta_product.argtypes = [T, T, T, T, T, ctypes.c_int32, ctypes.c_float, T,
                                                  ctypes.c_int32, T, ctypes.c_int32, T, T, ctypes.c_void_p,
                                                  ctypes.c_size_t, ctypes.c_void_p]
    lib.gdp_backward_workspace_bytes.restype = ctypes.c_size_t
    lib.gdp_backward_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                                 ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
    lib.gdp_chunk_prefill_backward.restype = ctypes.c_int
    lib.gdp_chunk_prefill_backward.argtypes = [T, T, T, T, T, ctypes.c_int32, T, ctypes.c_float, T, ctypes.c_int32,
                                               T, T, T, T, T, T, T, T, ctypes.c_void_p, ctypes.c_size_t,
                                               ctypes.c_void_p]
    lib.gdp_debug_status.restype = ctypes.c_int
    lib.gdp_debug_status.argtypes = [ctypes.POINTER(ctypes.c_uint32), ctypes.c_int32, ctypes.c_void_p]
    lib.gdp_last_error.restype = ctypes.c_char_p
    lib.gdp_last_error.argtypes = []
    lib.gdp_version.restype = ctypes.c_char_p
    lib.gdp_version.argtypes = []
    return lib


LIB = _load()

_DT = {torch.float32: GDP_F32, torch.bfloat16: GDP_BF16, torch.int32: GDP_I32, torch.int64: GDP_I64,
       torch.float16: GDP_F16}


def as_gdp_tensor(t):
    """gdp_tensor view of a torch tensor (None -> absent)."""
    g = gdp_tensor()
    if t is None:
        return g
    if t.dim() > 4:
        raise ValueError("at most 4 dims")
    if t.dtype not in _DT:
        raise ValueError(f"unsupported dtype {t.dtype}")
    g.data = t.data_ptr() if t.numel() > 0 else None
    g.dtype = _DT[t.dtype]
    g.ndim = t.dim()
    for d in range(t.dim()):
        g.shape[d] = t.shape[d]
        g.stride[d] = t.stride(d)
    if t.numel() == 0:
        # an empty tensor is still "present"; give it a non-null dummy address
        g.data = 16
    return g


def _check(rc):
    if rc != GDP_OK:
        raise GdpError(rc, LIB.gdp_last_error().decode())


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


# ---------------------------------------------------------------- C ABI names

def gdp_version():
    return LIB.gdp_version().decode()


def gdp_last_error():
    return LIB.gdp_last_error().decode()


def gdp_debug_status(clear=True, device=None):
    """The current device's debug-validation word (GDP_DBG_* bits) after the work
    queued on the current stream; cleared afterwards when `clear`.  The checks run
    only with GDP_DEBUG_VALIDATE=1 in the environment."""
    word = ctypes.c_uint32(0)
    _check(LIB.gdp_debug_status(ctypes.byref(word), 1 if clear else 0, _stream(device)))
    return int(word.value)


def gdp_descriptor_capacity(T, N, num_householder):
    a, b = ctypes.c_int64(), ctypes.c_int64()
    _check(LIB.gdp_descriptor_capacity(T, N, num_householder, ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def gdp_workspace_bytes(T, N, num_householder, Hqk, Hv, K, V, dtype=torch.bfloat16):
    return int(LIB.gdp_workspace_bytes(T, N, num_householder, Hqk, Hv, K, V, _DT[dtype]))


def gdp_build_descriptors(cu_seqlens, num_householder, T, nt_cap=None, ntdp_cap=None, out=None):
    """Device-built descriptors of both chunkings (int32 tensors), padded to capacity.

    ``out``: a dict of caller-allocated buffers (as this function returns) to
    build into, with the capacities their row counts give; nothing is then
    allocated, so the call can be captured in a graph."""
    N = cu_seqlens.shape[0] - 1
    dev = cu_seqlens.device
    if out is None:
        ct, cd = gdp_descriptor_capacity(T, N, num_householder)
        nt_cap = ct if nt_cap is None else nt_cap
        ntdp_cap = cd if ntdp_cap is None else ntdp_cap
        out = {"chunk_indices": torch.empty((max(nt_cap, 1), 2), dtype=torch.int32, device=dev),
               "chunk_indices_dp": torch.empty((max(ntdp_cap, 1), 2), dtype=torch.int32, device=dev),
               "chunk_offsets": torch.empty(N + 1, dtype=torch.int32, device=dev),
               "chunk_offsets_dp": torch.empty(N + 1, dtype=torch.int32, device=dev)}
    else:
        nt_cap, ntdp_cap = out["chunk_indices"].shape[0], out["chunk_indices_dp"].shape[0]
    d = _descs(out, nt_cap, ntdp_cap)
    cu = as_gdp_tensor(cu_seqlens)
    _check(LIB.gdp_build_descriptors(ctypes.byref(cu), num_householder, T, ctypes.byref(d), _stream(dev)))
    out["chunk_indices"] = out["chunk_indices"][:nt_cap]
    out["chunk_indices_dp"] = out["chunk_indices_dp"][:ntdp_cap]
    return out


def _descs(dct, nt_cap, ntdp_cap):
    d = gdp_descriptors()
    d.chunk_indices = dct["chunk_indices"].data_ptr()
    d.chunk_indices_dp = dct["chunk_indices_dp"].data_ptr()
    d.chunk_offsets = dct["chunk_offsets"].data_ptr()
    d.chunk_offsets_dp = dct["chunk_offsets_dp"].data_ptr()
    d.nt_cap = nt_cap
    d.ntdp_cap = ntdp_cap
    return d


def gdp_chunk_prefill(q, k, v, g_log, beta, num_householder, cu_seqlens, scale=0.0, initial_state=None,
                      output_final_state=False, use_qk_l2norm=False, state_cache=None, state_indices=None,
                      return_chunk_states=False, o=None, final_state=None, chunk_states=None,
                      descriptors=None, workspace=None, stream=None):
    """Direct call of the C entry point with caller-allocated outputs (all torch tensors).

    ``descriptors`` is a dict as returned by gdp_build_descriptors or None;
    ``workspace`` is a uint8 device tensor of at least gdp_workspace_bytes(...)
    bytes."""
    args = [as_gdp_tensor(x) for x in (q, k, v, g_log, beta)]
    cu = as_gdp_tensor(cu_seqlens)
    s0 = as_gdp_tensor(initial_state)
    cache = as_gdp_tensor(state_cache)
    slots = as_gdp_tensor(state_indices)
    ot, ft, ct = as_gdp_tensor(o), as_gdp_tensor(final_state), as_gdp_tensor(chunk_states)
    dptr = None
    if descriptors is not None:
        d = _descs(descriptors, descriptors["chunk_indices"].shape[0], descriptors["chunk_indices_dp"].shape[0])
        dptr = ctypes.byref(d)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = _stream(q.device) if stream is None else stream
    rc = LIB.gdp_chunk_prefill(*[ctypes.byref(a) for a in args], int(num_householder), ctypes.byref(cu),
                               float(scale or 0.0), ctypes.byref(s0), int(bool(output_final_state)),
                               int(bool(use_qk_l2norm)), ctypes.byref(cache), ctypes.byref(slots),
                               int(bool(return_chunk_states)), ctypes.byref(ot), ctypes.byref(ft),
                               ctypes.byref(ct), dptr, ws_ptr, ws_bytes, st)
    _check(rc)


def gdp_chunk_prefill_noalloc(q, k, v, g_log, beta, num_householder, cu_seqlens, scale=0.0, initial_state=None,
                              output_final_state=False, use_qk_l2norm=False, state_cache=None, state_indices=None,
                              return_chunk_states=False, o=None, final_state=None, chunk_states=None,
                              descriptors=None, stream=None):
    """Direct call of the C entry point that takes no workspace (its scratch is
    the library's static per-GPU array); outputs are caller-allocated."""
    args = [as_gdp_tensor(x) for x in (q, k, v, g_log, beta)]
    cu = as_gdp_tensor(cu_seqlens)
    s0 = as_gdp_tensor(initial_state)
    cache = as_gdp_tensor(state_cache)
    slots = as_gdp_tensor(state_indices)
    ot, ft, ct = as_gdp_tensor(o), as_gdp_tensor(final_state), as_gdp_tensor(chunk_states)
    dptr = None
    if descriptors is not None:
        d = _descs(descriptors, descriptors["chunk_indices"].shape[0], descriptors["chunk_indices_dp"].shape[0])
        dptr = ctypes.byref(d)
    st = _stream(q.device) if stream is None else stream
    rc = LIB.gdp_chunk_prefill_noalloc(*[ctypes.byref(a) for a in args], int(num_householder), ctypes.byref(cu),
                                       float(scale or 0.0), ctypes.byref(s0), int(bool(output_final_state)),
                                       int(bool(use_qk_l2norm)), ctypes.byref(cache), ctypes.byref(slots),
                                       int(bool(return_chunk_states)), ctypes.byref(ot), ctypes.byref(ft),
                                       ctypes.byref(ct), dptr, st)
    _check(rc)


def gdp_recurrent_decode(q, k, v, g_log, beta, num_householder, scale, use_qk_l2norm, state_cache,
                         state_indices, o, stream=None):
    """Direct call of the C entry point; o is caller-allocated, state_cache is updated in place."""
    args = [as_gdp_tensor(x) for x in (q, k, v, g_log, beta)]
    cache, slots, ot = as_gdp_tensor(state_cache), as_gdp_tensor(state_indices), as_gdp_tensor(o)
    st = _stream(q.device) if stream is None else stream
    _check(LIB.gdp_recurrent_decode(*[ctypes.byref(a) for a in args], int(num_householder), float(scale or 0.0),
                                    int(bool(use_qk_l2norm)), ctypes.byref(cache), ctypes.byref(slots),
                                    ctypes.byref(ot), st))


def gdp_fi_workspace_bytes(T, N, num_householder, Hq, Hv, head_size, dtype=torch.bfloat16,
                           with_initial_state=False, output_final_state=False):
    return int(LIB.gdp_fi_workspace_bytes(T, N, num_householder, Hq, Hv, head_size, _DT[dtype],
                                          int(bool(with_initial_state)), int(bool(output_final_state))))


def gdp_chunk_gated_delta_product(q, k, v, g, beta, num_householder, scale, initial_state, output_final_state,
                                  cu_seqlens, use_qk_l2norm_in_kernel, output, output_state, workspace,
                                  stream=None):
    """Direct call of the FlashInfer-convention C entry point (caller-allocated
    output, output_state and workspace)."""
    ts = [as_gdp_tensor(x) for x in (q, k, v, g, beta)]
    s0, cu = as_gdp_tensor(initial_state), as_gdp_tensor(cu_seqlens)
    ot, st_out = as_gdp_tensor(output), as_gdp_tensor(output_state)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = _stream(q.device) if stream is None else stream
    _check(LIB.gdp_chunk_gated_delta_product(*[ctypes.byref(a) for a in ts], int(num_householder),
                                             float(scale or 0.0), ctypes.byref(s0), int(bool(output_final_state)),
                                             ctypes.byref(cu), int(bool(use_qk_l2norm_in_kernel)),
                                             ctypes.byref(ot), ctypes.byref(st_out), ws_ptr, ws_bytes, st))


def gdp_backward_workspace_bytes(T, N, num_householder, Hqk, Hv, K, V, dtype=torch.bfloat16):
    return int(LIB.gdp_backward_workspace_bytes(T, N, num_householder, Hqk, Hv, K, V, _DT[dtype]))


def gdp_chunk_prefill_backward(q, k, v, g_log, beta, num_householder, cu_seqlens, scale, initial_state,
                               use_qk_l2norm, d_o, d_final_state, dq, dk, dv, dg_log, dbeta, d_initial_state,
                               workspace, stream=None):
    """Direct call of the backward C entry point (caller-allocated gradients and workspace)."""
    ts = [as_gdp_tensor(x) for x in (q, k, v, g_log, beta)]
    cu, s0 = as_gdp_tensor(cu_seqlens), as_gdp_tensor(initial_state)
    dts = [as_gdp_tensor(x) for x in (d_o, d_final_state, dq, dk, dv, dg_log, dbeta, d_initial_state)]
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = _stream(q.device) if stream is None else stream
    _check(LIB.gdp_chunk_prefill_backward(*[ctypes.byref(a) for a in ts], int(num_householder), ctypes.byref(cu),
                                          float(scale or 0.0), ctypes.byref(s0), int(bool(use_qk_l2norm)),
                                          *[ctypes.byref(a) for a in dts], ws_ptr, ws_bytes, st))


# ---------------------------------------------------------------- convenience wrapper

def chunk_prefill(q, k, v, g_log, beta, num_householder, cu_seqlens, scale=None, initial_state=None,
                  output_final_state=False, use_qk_l2norm=False, state_cache=None, state_indices=None,
                  return_chunk_states=False, descriptors=None, out=None):
    """Allocating front end in the Megatron Core argument order.

    Accepts an optional leading batch dim of 1 on q/k/v/g/beta (THD packing).
    Returns (o, final_state or None) or, with return_chunk_states,
    (o, final_state or None, chunk_states, chunk_offsets): chunk_states has the
    capacity row count; rows >= chunk_offsets[N] are unwritten padding.
    """
    squeeze = q.dim() == 4
    if squeeze:
        q, k, v, g_log, beta = q[0], k[0], v[0], g_log[0], beta[0]
    T, Hqk, K = q.shape
    Hv, V = v.shape[1], v.shape[2]
    N = cu_seqlens.shape[0] - 1
    dev = q.device
    o = out if out is not None else torch.empty((T, Hv, V), dtype=q.dtype, device=dev)
    fs = torch.empty((N, Hv, K, V), dtype=torch.float32, device=dev) if output_final_state else None
    cs = None
    if return_chunk_states and descriptors is None:
        descriptors = gdp_build_descriptors(cu_seqlens, num_householder, T)
    ws = torch.empty(max(gdp_workspace_bytes(T, N, num_householder, Hqk, Hv, K, V, q.dtype), 256),
                     dtype=torch.uint8, device=dev)
    if return_chunk_states:
        nt_cap, _ = gdp_descriptor_capacity(T, N, num_householder)
        cs = torch.empty((max(nt_cap, 1), Hv, K, V), dtype=torch.float32, device=dev)
    gdp_chunk_prefill(q, k, v, g_log, beta, num_householder, cu_seqlens, scale or 0.0, initial_state,
                      output_final_state, use_qk_l2norm, state_cache, state_indices, return_chunk_states,
                      o, fs, cs, descriptors, ws)
    if squeeze:
        o = o.unsqueeze(0)
    if return_chunk_states:
        return o, fs, cs, descriptors["chunk_offsets"]
    return o, fs


def recurrent_decode(q, k, v, g_log, beta, num_householder, state_cache, state_indices, scale=None,
                     use_qk_l2norm=False, out=None):
    """Allocating front end of the decode step: returns o [N, Hv, V]; the state
    cache is updated in place."""
    N = q.shape[0]
    Hv, V = v.shape[1], v.shape[2]
    o = out if out is not None else torch.empty((N, Hv, V), dtype=q.dtype, device=q.device)
    gdp_recurrent_decode(q, k, v, g_log, beta, num_householder, scale or 0.0, use_qk_l2norm, state_cache,
                         state_indices, o)
    return o


def chunk_gated_delta_product(q, k, v, g=None, beta=None, num_householder=1, scale=None, initial_state=None,
                              output_final_state=False, cu_seqlens=None, use_qk_l2norm_in_kernel=False,
                              output=None, output_state=None):
    """Allocating front end in the FlashInfer convention (FlashInfer docs,
    "flashinfer.gdp_prefill.chunk_gated_delta_product", parameter list): linear
    decays g (None: no decay), beta (None: ones), V-major states.  Returns
    output, or (output, final_state) when output_final_state."""
    if cu_seqlens is None:
        raise ValueError("cu_seqlens is required (varlen input only)")
    T, Hq, d = q.shape
    Hv = v.shape[1]
    N = cu_seqlens.shape[0] - 1
    dev = q.device
    out = output if output is not None else torch.empty((T, Hv, d), dtype=q.dtype, device=dev)
    fs = None
    if output_final_state:
        fs = output_state if output_state is not None else torch.empty(
            (N, Hv, d, d), dtype=initial_state.dtype if initial_state is not None else torch.float32, device=dev)
    ws = torch.empty(max(gdp_fi_workspace_bytes(T, N, num_householder, Hq, Hv, d, q.dtype, initial_state is not None,
                                                output_final_state), 256), dtype=torch.uint8, device=dev)
    gdp_chunk_gated_delta_product(q, k, v, g, beta, num_householder, scale, initial_state, output_final_state,
                                  cu_seqlens, use_qk_l2norm_in_kernel, out, fs, ws)
    return (out, fs) if output_final_state else out


def chunk_prefill_backward(q, k, v, g_log, beta, num_householder, cu_seqlens, d_o, d_final_state=None, scale=None,
                           initial_state=None, use_qk_l2norm=False):
    """Allocating front end of the gradients: returns a dict of float32 tensors
    dq, dk, dv, dg_log, dbeta and d_initial_state (None without an initial state)."""
    T, Hqk, K = q.shape
    Hk, Hv, V = k.shape[1], v.shape[1], v.shape[2]
    N = cu_seqlens.shape[0] - 1
    n = int(num_householder)
    dev = q.device
    f32 = dict(dtype=torch.float32, device=dev)
    dq, dk = torch.empty((T, Hqk, K), **f32), torch.empty((T * n, Hk, K), **f32)
    dv, dg = torch.empty((T * n, Hv, V), **f32), torch.empty((T, Hv), **f32)
    db = torch.empty((T * n, Hv), **f32)
    ds0 = torch.empty((N, Hv, K, V), **f32) if initial_state is not None else None
    ws = torch.empty(max(gdp_backward_workspace_bytes(T, N, n, Hqk, Hv, K, V, q.dtype), 256), dtype=torch.uint8,
                     device=dev)
    gdp_chunk_prefill_backward(q, k, v, g_log, beta, n, cu_seqlens, scale, initial_state, use_qk_l2norm, d_o,
                               d_final_state, dq, dk, dv, dg, db, ds0, ws)
    return {"dq": dq, "dk": dk, "dv": dv, "dg_log": dg, "dbeta": db, "d_initial_state": ds0}
