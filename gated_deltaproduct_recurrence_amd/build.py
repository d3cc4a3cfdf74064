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
           os.path.join(CSRC, "gdp_backward.hip"), os.path.join(CSRC, "gdp_bwd_chunk.hip"),
           os.path.join(CSRC, "gdp_validate.hip"),
           os.path.join(CSRC, "gdp_noalloc.hip"),
           os.path.join(CSRC, "gdp_api.cpp")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed-fp32 VALU forms are disabled for every gfx950 compile.
DEVICE_FLAGS = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]

# Per-source flags.  The prefill kernels are scheduled for instruction-level
# parallelism: the fused kernel then takes about 1% less time on the
# long-context prefill and no kernel of that file spills but the 12-wave
# summary instantiation (76 bytes per lane, no measurable cost).  The backward
# kernels, at 256 VGPRs, keep the default scheduler.
SOURCE_FLAGS = {"gdp_kernels.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]}
OBJ_DIR = os.path.join(ROOT, "_build", "obj")


# Host-side AddressSanitizer and UndefinedBehaviorSanitizer for the check build
# (each -fsanitize applies to the host compile only; the device code is built
# as usual).  Such a library needs the clang ASan runtime loaded first
# (LD_PRELOAD) and is meant for the CPU test suite: it exercises the host-side
# validation and never runs a kernel.
HOST_SANITIZE_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-shared-libsan",
                       "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                       "-Xarch_host", "-fno-sanitize-recover=all"]
SANITIZED_LIB = os.path.join(ROOT, "_build", "sanitize", "libgdp_hostcheck.so")


def asan_runtime():
    """Path of the clang AddressSanitizer runtime that the sanitized builds link against."""
    import glob
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd))
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        res.check_returncode()


def build_library(out=LIB, verbose=False, sanitize=False):
    """Compile and link libgdp.so; raises CalledProcessError on failure.
    sanitize=True builds the host-sanitized check library instead (to `out`),
    in one hipcc call without the per-source flags (it never runs a kernel)."""
    tmp = out + ".tmp"
    if sanitize:
        _run([HIPCC, *DEVICE_FLAGS, *HOST_SANITIZE_FLAGS, "-std=c++17", "-fPIC", "-shared", "-Wall",
              f"-I{INCLUDE}", f"-I{CSRC}", *SOURCES, "-o", tmp], verbose)
        os.replace(tmp, out)
        return out
    from concurrent.futures import ThreadPoolExecutor
    os.makedirs(OBJ_DIR, exist_ok=True)
    objs = [os.path.join(OBJ_DIR, os.path.basename(src) + ".o") for src in SOURCES]
    cmds = [[HIPCC, *DEVICE_FLAGS, "-O3", "-std=c++17", "-fPIC", "-Wall", f"-I{INCLUDE}", f"-I{CSRC}",
             *SOURCE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
            for src, obj in zip(SOURCES, objs)]
    with ThreadPoolExecutor(max_workers=max(1, min(len(cmds), os.cpu_count() or 1, 8))) as pool:
        for f in [pool.submit(_run, c, verbose) for c in cmds]:
            f.result()
    _run([HIPCC, *DEVICE_FLAGS, "-fPIC", "-shared", *objs, "-o", tmp], verbose)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_library(verbose=True))
