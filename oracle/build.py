"""Build the CPU oracle's shared library (test infrastructure only).

The oracle is plain C compiled by gcc: -O2, POSIX threads over output rows,
no fast-math and -ffp-contract=off, so every multiply and add in it is a
separately rounded IEEE fp64 operation.  It links no OpenMP runtime (the
process that loads it may already hold PyTorch's own).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "sgmv_oracle.c")
LIBRARY = os.path.join(HERE, "libsgmv_oracle.so")

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    """Compile sgmv_oracle.c into libsgmv_oracle.so next to it; return the path."""
    tmp = LIBRARY + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, SOURCE, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
