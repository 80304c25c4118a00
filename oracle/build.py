"""Build the CPU oracle (test infrastructure only) with gcc.

The oracle is plain C, compiled with the host compiler, never with hipcc,
and it shares nothing with the GPU library.  -ffp-contract=off keeps every
multiply and add separately rounded; -ffast-math is never used.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "oracle.c")
LIBRARY = os.path.join(HERE, "liboracle.so")

FLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
         "-fno-fast-math", "-Wall", "-Wextra"]


def build(verbose=False):
    """Compile oracle.c into liboracle.so next to it; returns the path."""
    tmp = LIBRARY + ".tmp%d" % os.getpid()
    cmd = ["gcc"] + FLAGS + [SOURCE, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
