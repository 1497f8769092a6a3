"""Build the CPU oracle (test infrastructure only) with gcc.

The oracle is a separate shared library, liboxref.so, compiled from plain C
with gcc (never hipcc): -O2 -fopenmp -ffp-contract=off, so no multiply-add is
contracted and every sum keeps the order the source states.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboxref.so")


def build(verbose: bool = False) -> str:
    """Compile oxref.c into liboxref.so next to this file; return its path."""
    src = os.path.join(HERE, "oxref.c")
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
