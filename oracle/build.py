"""Compile the fp64 CPU oracle into oracle/libgdr_ref.so (test infrastructure)."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libgdr_ref.so")


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(HERE, f) for f in ("gdr_ref.c", "gdr_ref_bwd.c")]
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall", "-Wextra",
           "-o", LIB + ".tmp", *srcs, "-lm"]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.check_call(cmd)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
