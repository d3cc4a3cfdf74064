"""Oracle-side chunk descriptors against hand-worked values and closed forms (CPU only).

Megatron Core API docs, core.ssm.ops.gdp.chunk: a sequence of L real tokens
has ceil(L/64) token chunks and ceil(L*M/64) Householder-expanded chunks, and
the second count is not M times the first unless 64 divides L.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "descriptors_varlen4_n2.json")


def test_golden_varlen4():
    gold = json.load(open(GOLDEN))
    d = oracle.descriptors(gold["cu_seqlens"], gold["num_householder"])
    assert d["chunk_indices"].tolist() == gold["chunk_indices"]
    assert d["chunk_indices_dp"].tolist() == gold["chunk_indices_dp"]
    assert d["chunk_offsets"].tolist() == gold["chunk_offsets"]
    assert d["chunk_offsets_dp"].tolist() == gold["chunk_offsets_dp"]
    T, N = gold["cu_seqlens"][-1], len(gold["cu_seqlens"]) - 1
    assert oracle.descriptor_capacity(T, N, 2) == (gold["nt_cap"], gold["ntdp_cap"])
    # the witness: expanded count differs from M * token count
    assert gold["NT_dp"] != 2 * gold["NT"]


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("n", [1, 2, 3, 5])
def test_random_lengths_closed_form(seed, n):
    rng = np.random.default_rng(seed)
    N = int(rng.integers(1, 40))
    lens = rng.integers(0, 300, size=N)
    lens[rng.random(N) < 0.2] = 0
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1])
    d = oracle.descriptors(cu, n)
    ct = [-(-int(L) // 64) for L in lens]
    cd = [-(-int(L) * n // 64) for L in lens]
    assert d["chunk_offsets"].tolist() == np.concatenate([[0], np.cumsum(ct)]).tolist()
    assert d["chunk_offsets_dp"].tolist() == np.concatenate([[0], np.cumsum(cd)]).tolist()
    cap_t, cap_d = oracle.descriptor_capacity(T, N, n)
    assert sum(ct) <= cap_t and sum(cd) <= cap_d
    rows = [(i, c) for i in range(N) for c in range(ct[i])]
    rows += [(-1, -1)] * (cap_t - len(rows))
    assert [tuple(r) for r in d["chunk_indices"].tolist()] == rows
    rows = [(i, c) for i in range(N) for c in range(cd[i])]
    rows += [(-1, -1)] * (cap_d - len(rows))
    assert [tuple(r) for r in d["chunk_indices_dp"].tolist()] == rows


def test_capacity_is_tight():
    # all lengths = 1 (mod 64) reach the bound floor((T + 63 N)/64) exactly
    lens = [65, 1, 129]
    cu = np.concatenate([[0], np.cumsum(lens)])
    cap_t, _ = oracle.descriptor_capacity(int(cu[-1]), 3, 1)
    assert cap_t == sum(-(-L // 64) for L in lens)


def test_capacity_too_small_rejected():
    with pytest.raises(ValueError):
        oracle.descriptors([0, 100], 2, nt_cap=1, ntdp_cap=4)
