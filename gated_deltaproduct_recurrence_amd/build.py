"""Build step: compiles the gfx950 HIP library libgdp.so in-tree with hipcc."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libgdp.so")
SOURCES = [os.path.join(CSRC, "gdp_kernels.hip"), os.path.join(CSRC, "gdp_decode.hip"),
           os.path.join(CSRC, "gdp_segments.hip"), os.path.join(CSRC, "gdp_frontend.hip"),
           os.path.join(CSRC, "gdp_backward.hip"), os.path.join(CSRC, "gdp_validate.hip"),
           os.path.join(CSRC, "gdp_api.cpp")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed-fp32 VALU forms are disabled for every gfx950 compile.
DEVICE_FLAGS = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build_library(out=LIB, verbose=False):
    """Compile and link libgdp.so; raises CalledProcessError on failure."""
    tmp = out + ".tmp"
    cmd = [HIPCC, *DEVICE_FLAGS, "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
           f"-I{INCLUDE}", f"-I{CSRC}", *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd))
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        res.check_returncode()
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_library(verbose=True))
