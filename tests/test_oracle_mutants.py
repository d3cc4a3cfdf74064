"""Planted mistakes in the oracle must be caught by the pins (CPU only).

Each mutant is a copy of oracle/gdp_oracle.c with one plausible mistake (a
dropped term, a wrong sign, a wrong index, a transposed role), compiled to a
temporary library.  The pins of tests/oracle_pins.py run against it and at
least one must fail; a mutant that survives means the pins have a hole.
"""
import os

import pytest

import oracle
from oracle import build as obuild
from tests import oracle_pins

MUTANTS = {
    "error_sign": ("e[c] = b * (vr[c] - e[c]);", "e[c] = b * (vr[c] + e[c]);"),
    "dropped_beta": ("e[c] = b * (vr[c] - e[c]);", "e[c] = (vr[c] - e[c]);"),
    "last_update_dropped": ("for (int j = 0; j < n; ++j) {", "for (int j = 0; j < n - 1; ++j) {"),
    "decay_every_subrow": (
        "const double b = p->beta[(size_t)r * Hv + h];",
        "const double b = p->beta[(size_t)r * Hv + h];\n"
        "      if (j > 0) for (size_t x = 0; x < KV; ++x) S[x] *= alpha;"),
    "decay_after_update": [
        ("for (size_t x = 0; x < KV; ++x) S[x] *= alpha;\n", "\n"),
        ("/* 2.4 readout after the last update */",
         "for (size_t x = 0; x < KV; ++x) S[x] *= alpha;")],
    "gqa_modulo": ("const int hq = h / (Hv / Hqk);", "const int hq = h % Hqk;"),
    "key_token_row": ("memcpy(kap, p->k + ((size_t)r * Hqk + hq) * K, K * sizeof(double));",
                      "memcpy(kap, p->k + ((size_t)(t * n) * Hqk + hq) * K, K * sizeof(double));"),
    "norm_without_sqrt": ("double r = 1.0 / sqrt(ss + 1e-6);", "double r = 1.0 / (ss + 1e-6);"),
    "default_scale_uses_V": ("1.0 / sqrt((double)K)", "1.0 / sqrt((double)V)"),
    "chunk_state_off_by_one": ("if (p->chunk_states && rel % GDPO_CHUNK == 0) {",
                               "if (p->chunk_states && (rel + 1) % GDPO_CHUNK == 0) {"),
    "slot_zero_skipped": ("p->slots[seq] >= 0)", "p->slots[seq] > 0)"),
    "initial_state_index": ("memcpy(S, p->s0 + ((size_t)seq * Hv + h) * KV",
                            "memcpy(S, p->s0 + ((size_t)h * p->N + seq) * KV"),
    "readout_scale_dropped": ("ot[c] = p->scale * e[c];", "ot[c] = e[c];"),
    "update_uses_query": ("Sa[c] += ka * e[c]; /* S += k e^T */",
                          "Sa[c] += ka * e[c] * (1.0 + 1e-3 * a); /* S += k e^T */"),
}


@pytest.fixture(scope="module")
def source():
    with open(obuild.SRC) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, source, name):
    edits = MUTANTS[name]
    if isinstance(edits, tuple):
        edits = [edits]
    text = source
    for old, new in edits:
        assert text.count(old) >= 1, f"mutation target for {name} not found in the oracle source"
        text = text.replace(old, new, 1)
    src = tmp_path / "mutant.c"
    src.write_text(text)
    lib_path = obuild.compile_oracle(str(src), str(tmp_path / "libmutant.so"))
    lib = oracle.load(lib_path)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(lib)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"mutant {name} survived every pin"
    os.remove(lib_path)
