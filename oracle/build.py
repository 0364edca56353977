"""Build the fp64 CPU oracle (test infrastructure only) with gcc.

Usage: python oracle/build.py  -> writes oracle/liboracle.so
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "attn_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def compile_to(src: str, lib: str, verbose: bool = False) -> str:
    """Compile one C source into a shared library at `lib`."""
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False) -> str:
    """Compile attn_oracle.c into liboracle.so (always recompiles)."""
    return compile_to(SRC, LIB, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
