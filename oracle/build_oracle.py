"""Build the CPU oracle (plain C, fp64, OpenMP) into ``oracle/libconv_oracle.so``.

Test infrastructure only: the HIP library never links or loads this.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "conv_oracle.c")
LIB = os.path.join(HERE, "libconv_oracle.so")


def build(verbose: bool = False) -> str:
    """Compile the oracle with gcc; always recompiles.  Returns the library path."""
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
