"""Host checks of the library build description (no compile, no GPU)."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from gated_deltaproduct_recurrence_amd import build as lib_build  # noqa: E402


def test_sources_exist():
    for src in lib_build.SOURCES:
        assert os.path.isfile(src), src


def test_source_flags_name_real_sources():
    # a misspelt key would drop its flags without any error
    names = {os.path.basename(s) for s in lib_build.SOURCES}
    assert set(lib_build.SOURCE_FLAGS) <= names


def test_device_flags_disable_packed_fp32():
    f = lib_build.DEVICE_FLAGS
    assert "--offload-arch=gfx950" in f
    i = f.index("-packed-fp32-ops")
    assert f[i - 1] == "-Xclang" and f[i - 2] == "-target-feature"


def test_object_names_are_distinct():
    objs = [os.path.basename(s) + ".o" for s in lib_build.SOURCES]
    assert len(set(objs)) == len(objs)
