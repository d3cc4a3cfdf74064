"""Build step for the CPU oracle: compiles gdp_oracle.c into a shared library.

Test infrastructure only (see the header of gdp_oracle.c).  The library is
built with portable x86-64-v3 code generation so that a build made on one
host also runs on another host of the same architecture level.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gdp_oracle.c")
LIB = os.path.join(HERE, "libgdp_oracle.so")


SANITIZED_LIB = os.path.join(os.path.dirname(HERE), "_build", "sanitize", "libgdp_oracle_sanitized.so")


def compile_oracle(src=SRC, out=LIB, extra_flags=(), sanitize=False):
    """Compile ``src`` to the shared library ``out``; raises on failure.
    sanitize=True builds it with clang's AddressSanitizer and
    UndefinedBehaviorSanitizer (the same runtime as the library's check build)."""
    if sanitize:
        cmd = ["/opt/rocm/llvm/bin/clang", "-O1", "-g", "-fno-omit-frame-pointer", "-march=x86-64-v3", "-fPIC",
               "-shared", "-shared-libsan", "-pthread", "-std=c11", "-Wall", "-Wextra", "-Wno-unused-parameter",
               "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
               *extra_flags, src, "-o", out + ".tmp", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(out + ".tmp", out)
        return out
    cmd = ["gcc", "-O3", "-march=x86-64-v3", "-fPIC", "-shared", "-pthread",
           "-std=c11", "-Wall", "-Wextra", "-Wno-unused-parameter",
           *extra_flags, src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(compile_oracle(*sys.argv[1:2]))
