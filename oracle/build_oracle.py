"""Build the CPU oracle's shared library (plain C, gcc, OpenMP).

Test infrastructure only: the oracle checks the HIP path and is never part of it.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "pagedkv_ref.c")
LIB = os.path.join(HERE, "libpagedkv_ref.so")


def build(verbose: bool = False, src: str = SRC, lib: str = LIB) -> str:
    """Compile the oracle's C source (by default oracle/pagedkv_ref.c into
    oracle/libpagedkv_ref.so) and return the library's path."""
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
