"""The CPU suite again, against host-sanitized builds (no GPU needed).

The oracle (oracle/gdp_oracle.c) and the library's host side (every entry
point's validation of shapes, dtypes, strides, workspace and aliasing, among
them the rule that no output may overlap an input, which covers final_state
aliasing initial_state: FlashInfer docs, "flashinfer.gdp_prefill.
chunk_gated_delta_product", output_state) are rebuilt with clang's
AddressSanitizer and UndefinedBehaviorSanitizer, and every `-m "not gpu"` test
runs in a child process that loads those builds (GDP_LIBRARY,
GDP_ORACLE_LIBRARY) with the ASan runtime preloaded.  Any sanitizer report
aborts the child, which fails this test.  The builds are redone only when a
source is newer than them."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from gated_deltaproduct_recurrence_amd import build as lib_build  # noqa: E402
from oracle import build as oracle_build  # noqa: E402


def _stale(out, sources):
    return not os.path.exists(out) or os.path.getmtime(out) < max(os.path.getmtime(s) for s in sources)


@pytest.mark.skipif(os.environ.get("GDP_SANITIZED") == "1", reason="already inside the sanitized run")
def test_cpu_suite_under_address_and_ub_sanitizers():
    rt = lib_build.asan_runtime()
    if rt is None or not os.path.exists(lib_build.HIPCC):
        pytest.skip("clang ASan runtime or hipcc not installed")
    os.makedirs(os.path.dirname(lib_build.SANITIZED_LIB), exist_ok=True)
    headers = glob.glob(os.path.join(lib_build.CSRC, "*.h")) + glob.glob(os.path.join(lib_build.INCLUDE, "*.h"))
    if _stale(lib_build.SANITIZED_LIB, lib_build.SOURCES + headers + [lib_build.__file__]):
        lib_build.build_library(out=lib_build.SANITIZED_LIB, sanitize=True)
    if _stale(oracle_build.SANITIZED_LIB, [oracle_build.SRC, oracle_build.__file__]):
        oracle_build.compile_oracle(out=oracle_build.SANITIZED_LIB, sanitize=True)
    env = dict(os.environ, GDP_SANITIZED="1", GDP_LIBRARY=lib_build.SANITIZED_LIB,
               GDP_ORACLE_LIBRARY=oracle_build.SANITIZED_LIB, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-x", "-q", "-m", "not gpu",
                          "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (res.stdout + res.stderr)[-4000:]
    assert res.returncode == 0, tail
    assert "AddressSanitizer" not in tail and "runtime error" not in tail, tail
