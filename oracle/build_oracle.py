"""Build the CPU oracle (plain C, fp64, OpenMP) into ``oracle/libconv_oracle.so``.

Test infrastructure only: the HIP library never links or loads this.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "conv_oracle.c")
LIB = os.path.join(HERE, "libconv_oracle.so")
SRC_ND = os.path.join(HERE, "convnd_oracle.c")
LIB_ND = os.path.join(HERE, "libconvnd_oracle.so")
CFLAGS = ["-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    """Compile both oracle libraries (2-D, and the generalised N-D one) with gcc; always
    recompiles.  Returns the 2-D library's path."""
    for src, lib in ((SRC, LIB), (SRC_ND, LIB_ND)):
        tmp = lib + ".tmp"
        cmd = ["gcc"] + CFLAGS + [src, "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
