"""Build the fp64 CPU oracle (test infrastructure) into oracle/liboracle.so.

The oracle is a plain C file compiled with gcc; it is built next to its source
so that it travels with the tree.  No -march=native: the library built here must
also run on other x86-64 hosts.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False, src: str = SRC, out: str = LIB) -> str:
    """Compile ``src`` (default: oracle.c) into the shared library ``out``."""
    cmd = [
        "gcc", "-std=c99", "-O2", "-fopenmp", "-fPIC", "-shared",
        "-Wall", "-Wextra", "-o", out + ".tmp", src, "-lm",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv[1:]))
