"""Compile the fp64 CPU oracle into oracle/libgdr_ref.so (test infrastructure)."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libgdr_ref.so")


SOURCES = ("gdr_ref.c", "gdr_ref_bwd.c")


def build(verbose: bool = False, out: str = LIB, sanitize: bool = False) -> str:
    """Compile the oracle; sanitize=True adds AddressSanitizer and UndefinedBehaviorSanitizer
    (host code only, for the CPU test that runs the pins under them)."""
    srcs = [os.path.join(HERE, f) for f in SOURCES]
    flags = ["-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall", "-Wextra"]
    if sanitize:
        flags = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                 "-fno-sanitize-recover=undefined", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                 "-Wall", "-Wextra"]
    cmd = ["gcc", *flags, "-o", out + ".tmp", *srcs, "-lm"]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.check_call(cmd)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
