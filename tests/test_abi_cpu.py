"""C-ABI checks that need no GPU: the library loads, exports every function
include/gdp.h declares, and rejects bad arguments on the host (shapes, dtypes,
strides, aliasing, workspace) before any launch.  Device pointers here are
fake, well-aligned addresses that are never dereferenced: every case below
fails validation, which reads shapes and pointer ranges only."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdp.h")


@pytest.fixture(scope="module")
def b():
    from gated_deltaproduct_recurrence_amd import binding
    return binding


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdp_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(b):
    names = declared_functions()
    assert set(names) == set(b.EXPORTED), names
    for name in names:
        assert hasattr(b.LIB, name), f"{name} not exported"
    assert "gfx950" in b.gdp_version()


def test_capacity_and_workspace(b):
    assert b.gdp_descriptor_capacity(812, 4, 2) == (16, 29)
    assert b.gdp_descriptor_capacity(524288, 8, 2) == (8199, 16391)
    assert b.gdp_workspace_bytes(812, 4, 2, 4, 4, 128, 128) >= 29 * 4 * 64 * 64 * 2 + (16 + 29) * 8 + 2 * 5 * 4
    import torch
    assert b.gdp_workspace_bytes(812, 4, 2, 4, 4, 64, 64, torch.float32) >= 29 * 4 * 64 * 64 * 4
    with pytest.raises(b.GdpError):
        b.gdp_descriptor_capacity(10, 1, 0)


class Fake:
    """Allocates fake 4 KiB-aligned, non-overlapping "device" ranges."""

    def __init__(self):
        self.next = 1 << 40

    def tensor(self, b, dtype, shape, strides=None, data=None):
        t = b.gdp_tensor()
        es = {b.GDP_F32: 4, b.GDP_BF16: 2, b.GDP_I32: 4, b.GDP_I64: 8, b.GDP_F16: 2}[dtype]
        if strides is None:
            strides, acc = [], 1
            for d in reversed(shape):
                strides.insert(0, acc)
                acc *= d
        size = es
        for d, s in zip(shape, strides):
            size += (d - 1) * s * es if d > 0 else 0
        if data is None:
            data = self.next
            self.next += (size + 4095) // 4096 * 4096 + 4096
        t.data = data
        t.dtype = dtype
        t.ndim = len(shape)
        for i, (d, s) in enumerate(zip(shape, strides)):
            t.shape[i] = d
            t.stride[i] = s
        return t


def base_args(b, T=100, N=2, n=2, Hqk=2, Hv=4, K=128, V=128, dt=None):
    f = Fake()
    dt = b.GDP_BF16 if dt is None else dt
    a = dict(
        q=f.tensor(b, dt, [T, Hqk, K]), k=f.tensor(b, dt, [T * n, Hqk, K]), v=f.tensor(b, dt, [T * n, Hv, V]),
        g_log=f.tensor(b, b.GDP_F32, [T, Hv]), beta=f.tensor(b, b.GDP_F32, [T * n, Hv]), n=n,
        cu=f.tensor(b, b.GDP_I32, [N + 1]), scale=0.0, s0=f.tensor(b, b.GDP_F32, [N, Hv, K, V]), ofs=1, l2=0,
        cache=b.gdp_tensor(), slots=b.gdp_tensor(), rcs=0, o=f.tensor(b, dt, [T, Hv, V]),
        fs=f.tensor(b, b.GDP_F32, [N, Hv, K, V]), cs=b.gdp_tensor(), desc=None, ws=f.next, wsb=1 << 30)
    a["fake"] = f
    return a


def call(b, a):
    r = ctypes.byref
    return b.LIB.gdp_chunk_prefill(r(a["q"]), r(a["k"]), r(a["v"]), r(a["g_log"]), r(a["beta"]), a["n"], r(a["cu"]),
                                   a["scale"], r(a["s0"]), a["ofs"], a["l2"], r(a["cache"]), r(a["slots"]),
                                   a["rcs"], r(a["o"]), r(a["fs"]), r(a["cs"]), a["desc"], a["ws"], a["wsb"], None)


def expect(b, a, code, fragment):
    rc = call(b, a)
    assert rc == code, (rc, b.gdp_last_error())
    assert fragment in b.gdp_last_error(), b.gdp_last_error()


def test_missing_required(b):
    a = base_args(b)
    a["cu"] = b.gdp_tensor()
    expect(b, a, b.GDP_EINVAL, "cu_seqlens is required")
    a = base_args(b)
    a["q"] = b.gdp_tensor()
    expect(b, a, b.GDP_EINVAL, "required")


def test_householder_count(b):
    a = base_args(b)
    a["n"] = 0
    expect(b, a, b.GDP_EINVAL, "num_householder")


def test_head_grouping(b):
    a = base_args(b, Hqk=3, Hv=4)
    expect(b, a, b.GDP_EINVAL, "multiple of Hqk")


def test_shape_mismatch(b):
    a = base_args(b)
    a["k"] = a["fake"].tensor(b, b.GDP_BF16, [150, 2, 128])
    expect(b, a, b.GDP_EINVAL, "k: dim 0")
    a = base_args(b)
    a["beta"] = a["fake"].tensor(b, b.GDP_F32, [100, 4])
    expect(b, a, b.GDP_EINVAL, "beta: dim 0")


def test_dtype_rules(b):
    a = base_args(b)
    a["k"] = a["fake"].tensor(b, b.GDP_F32, [200, 2, 128])
    expect(b, a, b.GDP_EUNSUPPORTED, "share one dtype")
    a = base_args(b)
    a["beta"] = a["fake"].tensor(b, b.GDP_BF16, [200, 4])
    expect(b, a, b.GDP_EUNSUPPORTED, "float32")


def test_unsupported_head_dims(b):
    a = base_args(b, K=96, V=96)
    expect(b, a, b.GDP_EUNSUPPORTED, "K=96")
    a = base_args(b, K=128, V=128, dt=b.GDP_F32)
    expect(b, a, b.GDP_EUNSUPPORTED, "f32")


def test_inner_stride(b):
    a = base_args(b)
    a["q"] = a["fake"].tensor(b, b.GDP_BF16, [100, 2, 128], strides=[512, 256, 2])
    expect(b, a, b.GDP_EINVAL, "innermost")


def test_misaligned_row_stride(b):
    a = base_args(b)
    a["q"] = a["fake"].tensor(b, b.GDP_BF16, [100, 2, 128], strides=[260, 130, 1])
    expect(b, a, b.GDP_EUNSUPPORTED, "16-byte")


def test_final_state_aliasing_initial_state(b):
    a = base_args(b)
    a["fs"] = a["fake"].tensor(b, b.GDP_F32, [2, 4, 128, 128], data=a["s0"].data)
    expect(b, a, b.GDP_EALIAS, "final_state overlaps input initial_state")


def test_output_overlaps_input(b):
    a = base_args(b)
    a["o"] = a["fake"].tensor(b, b.GDP_BF16, [100, 4, 128], data=a["v"].data + 64)
    expect(b, a, b.GDP_EALIAS, "o overlaps input v")


def test_outputs_overlap_each_other(b):
    a = base_args(b)
    a["cache"] = a["fake"].tensor(b, b.GDP_F32, [4, 4, 128, 128], data=a["fs"].data)
    a["slots"] = a["fake"].tensor(b, b.GDP_I32, [2])
    expect(b, a, b.GDP_EALIAS, "overlaps")


def test_cache_needs_indices(b):
    a = base_args(b)
    a["cache"] = a["fake"].tensor(b, b.GDP_F32, [4, 4, 128, 128])
    expect(b, a, b.GDP_EINVAL, "go together")


def test_final_state_buffer_required(b):
    a = base_args(b)
    a["fs"] = b.gdp_tensor()
    expect(b, a, b.GDP_EINVAL, "final_state buffer")


def test_chunk_states_capacity(b):
    a = base_args(b)
    a["rcs"] = 1
    a["cs"] = a["fake"].tensor(b, b.GDP_F32, [2, 4, 128, 128])
    expect(b, a, b.GDP_EINVAL, "rows")


def test_workspace_too_small(b):
    a = base_args(b)
    a["wsb"] = 8
    expect(b, a, b.GDP_EWORKSPACE, "workspace")
    a = base_args(b)
    a["ws"] = None
    expect(b, a, b.GDP_EWORKSPACE, "workspace")


def test_build_descriptors_capacity_check(b):
    f = Fake()
    cu = f.tensor(b, b.GDP_I32, [5])
    d = b.gdp_descriptors()
    d.chunk_indices = d.chunk_indices_dp = d.chunk_offsets = d.chunk_offsets_dp = f.next
    d.nt_cap, d.ntdp_cap = 15, 29
    rc = b.LIB.gdp_build_descriptors(ctypes.byref(cu), 2, 812, ctypes.byref(d), None)
    assert rc == b.GDP_EINVAL and "below the bound" in b.gdp_last_error()


@pytest.mark.parametrize("caps", [(2, 5), (3, 4)], ids=["token-capacity", "expanded-capacity"])
def test_caller_descriptors_below_the_bound(b, caps):
    """Caller descriptors built for a smaller T (or another n) would leave
    chunks out of the grids: their capacities are checked against the bound
    of (T, N, n) = (100, 2, 2), which is (3, 5)."""
    assert b.gdp_descriptor_capacity(100, 2, 2) == (3, 5)
    a = base_args(b)
    f = a["fake"]
    d = b.gdp_descriptors()
    d.chunk_indices = d.chunk_indices_dp = d.chunk_offsets = d.chunk_offsets_dp = f.next
    d.nt_cap, d.ntdp_cap = caps
    a["desc"] = ctypes.byref(d)
    expect(b, a, b.GDP_EINVAL, "below the bounds")


# ---------------------------------------------------------------- decode step

def decode_args(b, N=8, n=2, Hqk=2, Hv=4, K=128, V=128, S=16, dt=None):
    f = Fake()
    dt = b.GDP_BF16 if dt is None else dt
    a = dict(q=f.tensor(b, dt, [N, Hqk, K]), k=f.tensor(b, dt, [N * n, Hqk, K]), v=f.tensor(b, dt, [N * n, Hv, V]),
             g_log=f.tensor(b, b.GDP_F32, [N, Hv]), beta=f.tensor(b, b.GDP_F32, [N * n, Hv]), n=n, scale=0.0, l2=0,
             cache=f.tensor(b, b.GDP_F32, [S, Hv, K, V]), slots=f.tensor(b, b.GDP_I32, [N]),
             o=f.tensor(b, dt, [N, Hv, V]))
    a["fake"] = f
    return a


def decode_expect(b, a, code, fragment):
    r = ctypes.byref
    rc = b.LIB.gdp_recurrent_decode(r(a["q"]), r(a["k"]), r(a["v"]), r(a["g_log"]), r(a["beta"]), a["n"],
                                    a["scale"], a["l2"], r(a["cache"]), r(a["slots"]), r(a["o"]), None)
    assert rc == code, (rc, b.gdp_last_error())
    assert fragment in b.gdp_last_error(), b.gdp_last_error()


def test_decode_requires_cache(b):
    a = decode_args(b)
    a["cache"] = b.gdp_tensor()
    decode_expect(b, a, b.GDP_EINVAL, "state_cache and state_indices are required")


def test_decode_shapes_and_dtypes(b):
    a = decode_args(b)
    a["k"] = a["fake"].tensor(b, b.GDP_BF16, [8, 2, 128])
    decode_expect(b, a, b.GDP_EINVAL, "k: dim 0")
    a = decode_args(b)
    a["cache"] = a["fake"].tensor(b, b.GDP_F32, [16, 4, 128, 64])
    decode_expect(b, a, b.GDP_EINVAL, "state_cache: dim 3")
    a = decode_args(b)
    a["cache"] = a["fake"].tensor(b, b.GDP_BF16, [16, 4, 128, 128])
    decode_expect(b, a, b.GDP_EUNSUPPORTED, "float32")
    a = decode_args(b)
    a["slots"] = a["fake"].tensor(b, b.GDP_F32, [8])
    decode_expect(b, a, b.GDP_EINVAL, "int32 or int64")
    a = decode_args(b, K=96, V=96)
    decode_expect(b, a, b.GDP_EUNSUPPORTED, "K=96")
    a = decode_args(b, Hqk=3, Hv=4)
    decode_expect(b, a, b.GDP_EINVAL, "multiple of Hqk")
    a = decode_args(b)
    a["n"] = 0
    decode_expect(b, a, b.GDP_EINVAL, "num_householder")


def test_decode_aliasing(b):
    a = decode_args(b)
    a["o"] = a["fake"].tensor(b, b.GDP_BF16, [8, 4, 128], data=a["v"].data)
    decode_expect(b, a, b.GDP_EALIAS, "o overlaps input v")
    a = decode_args(b)
    a["cache"] = a["fake"].tensor(b, b.GDP_F32, [16, 4, 128, 128], data=a["k"].data)
    decode_expect(b, a, b.GDP_EALIAS, "state_cache overlaps input k")
    a = decode_args(b)
    a["o"] = a["fake"].tensor(b, b.GDP_BF16, [8, 4, 128], data=a["cache"].data + 4096)
    decode_expect(b, a, b.GDP_EALIAS, "o overlaps state_cache")


# ---------------------------------------------------------------- FlashInfer-convention entry point

def fi_args(b, T=100, N=2, n=2, Hq=2, Hk=2, Hv=4, d=128, dt=None):
    f = Fake()
    dt = b.GDP_BF16 if dt is None else dt
    a = dict(q=f.tensor(b, dt, [T, Hq, d]), k=f.tensor(b, dt, [T * n, Hk, d]), v=f.tensor(b, dt, [T * n, Hv, d]),
             g=f.tensor(b, b.GDP_F32, [T, Hv]), beta=f.tensor(b, b.GDP_F32, [T * n, Hv]), n=n, scale=0.0,
             s0=f.tensor(b, b.GDP_F32, [N, Hv, d, d]), ofs=1, cu=f.tensor(b, b.GDP_I32, [N + 1]), l2=0,
             o=f.tensor(b, dt, [T, Hv, d]), fs=f.tensor(b, b.GDP_F32, [N, Hv, d, d]), ws=None, wsb=0)
    a["fake"] = f
    return a


def fi_expect(b, a, code, fragment):
    r = ctypes.byref
    rc = b.LIB.gdp_chunk_gated_delta_product(r(a["q"]), r(a["k"]), r(a["v"]), r(a["g"]), r(a["beta"]), a["n"],
                                             a["scale"], r(a["s0"]), a["ofs"], r(a["cu"]), a["l2"], r(a["o"]),
                                             r(a["fs"]), a["ws"], a["wsb"], None)
    assert rc == code, (rc, b.gdp_last_error())
    assert fragment in b.gdp_last_error(), b.gdp_last_error()


def test_fi_validation(b):
    fi_expect(b, fi_args(b), b.GDP_EWORKSPACE, "workspace")
    a = fi_args(b)
    a["fs"] = a["fake"].tensor(b, b.GDP_F32, [2, 4, 128, 128], data=a["s0"].data)
    fi_expect(b, a, b.GDP_EALIAS, "output_state overlaps initial_state")
    fi_expect(b, fi_args(b, dt=b.GDP_F32), b.GDP_EUNSUPPORTED, "bfloat16 or float16")
    a = fi_args(b, dt=b.GDP_F16)
    a["q"] = a["fake"].tensor(b, b.GDP_F16, [100, 2, 128], strides=[260, 130, 1])
    a["ws"], a["wsb"] = a["fake"].next, 1 << 34
    fi_expect(b, a, b.GDP_EUNSUPPORTED, "multiples of 8")
    fi_expect(b, fi_args(b, Hk=3), b.GDP_EINVAL, "Hq or Hv heads")
    fi_expect(b, fi_args(b, Hq=4, Hk=4, Hv=2), b.GDP_EUNSUPPORTED, "more q heads")
    fi_expect(b, fi_args(b, d=96), b.GDP_EUNSUPPORTED, "head size")
    a = fi_args(b)
    a["g"] = a["fake"].tensor(b, b.GDP_I32, [100, 4])
    fi_expect(b, a, b.GDP_EUNSUPPORTED, "g must be")
    a = fi_args(b)
    a["beta"] = a["fake"].tensor(b, b.GDP_F16, [200, 4])
    fi_expect(b, a, b.GDP_EUNSUPPORTED, "beta must be")
    a = fi_args(b)
    a["fs"] = b.gdp_tensor()
    fi_expect(b, a, b.GDP_EINVAL, "output_state is required")
    a = fi_args(b)
    a["o"] = a["fake"].tensor(b, b.GDP_BF16, [100, 2, 128])
    fi_expect(b, a, b.GDP_EINVAL, "output: dim 1")


def test_fi_workspace_bytes(b):
    import torch
    base = b.gdp_workspace_bytes(100, 2, 2, 2, 4, 128, 128)
    ws = b.gdp_fi_workspace_bytes(100, 2, 2, 2, 4, 128, torch.bfloat16, True, True)
    assert ws >= base + 4 * 3 * 100 * 4 + 2 * 2 * 4 * 128 * 128 * 4
    assert b.gdp_fi_workspace_bytes(100, 2, 2, 2, 4, 128, torch.float16) >= b.gdp_fi_workspace_bytes(
        100, 2, 2, 2, 4, 128, torch.bfloat16) + 2 * (100 * 2 + 2 * 2 * 100 * 4 + 100 * 4) * 128
    assert b.gdp_fi_workspace_bytes(100, 2, 2, 2, 4, 128, torch.float32) == 0


def test_prefill_accepts_k_per_state_head(b):
    a = base_args(b)
    a["k"] = a["fake"].tensor(b, b.GDP_BF16, [200, 3, 128])
    expect(b, a, b.GDP_EINVAL, "Hqk or Hv heads")


def test_debug_status_requires_a_word(b):
    """The word pointer is checked before any runtime call."""
    assert b.LIB.gdp_debug_status(None, 0, None) == b.GDP_EINVAL
    assert "word" in b.gdp_last_error()


def test_debug_bits_match_the_header(b):
    text = open(HEADER).read()
    for name, val in (("GDP_DBG_CU", b.GDP_DBG_CU), ("GDP_DBG_SLOT", b.GDP_DBG_SLOT), ("GDP_DBG_DUP", b.GDP_DBG_DUP)):
        assert re.search(rf"\b{name}\s*=\s*{val}\b", text), name


# ---------------------------------------------------------------- entry point without a workspace

def call_noalloc(b, a):
    r = ctypes.byref
    return b.LIB.gdp_chunk_prefill_noalloc(r(a["q"]), r(a["k"]), r(a["v"]), r(a["g_log"]), r(a["beta"]), a["n"],
                                           r(a["cu"]), a["scale"], r(a["s0"]), a["ofs"], a["l2"], r(a["cache"]),
                                           r(a["slots"]), a["rcs"], r(a["o"]), r(a["fs"]), r(a["cs"]), a["desc"],
                                           None)


def test_noalloc_validates_like_the_workspace_entry(b):
    """The entry point without a workspace runs the same host checks first."""
    a = base_args(b)
    a["n"] = 0
    assert call_noalloc(b, a) == b.GDP_EINVAL and "num_householder" in b.gdp_last_error()
    a = base_args(b)
    a["fs"] = a["s0"]
    assert call_noalloc(b, a) == b.GDP_EALIAS


def test_noalloc_rejects_calls_beyond_its_scratch(b, monkeypatch):
    """A call whose workspace need exceeds the static scratch array (here the
    float32 split path's WY matrices, 16 KiB per expanded chunk and state head:
    about 200 MB for 100,000 tokens, n=2, four heads) is refused before any
    device call, with the size it needs."""
    monkeypatch.delenv("GDP_PREFILL_PATH", raising=False)
    a = base_args(b, T=100000, N=1, n=2, Hqk=1, Hv=4, K=64, V=64, dt=b.GDP_F32)
    rc = call_noalloc(b, a)
    assert rc == b.GDP_EWORKSPACE, (rc, b.gdp_last_error())
    msg = b.gdp_last_error()
    assert "noalloc" in msg and str(64 << 20) in msg, msg
