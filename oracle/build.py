"""Build the fp64 CPU oracle (test infrastructure) with gcc into oracle/liblla_oracle.so."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "lla_oracle.c")
LIB = os.path.join(HERE, "liblla_oracle.so")


def build(verbose: bool = False) -> str:
    # -ffp-contract=off keeps every product and sum a separately rounded fp64 operation, so the
    # oracle's arithmetic is exactly what the source says.
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-std=c99",
           "-Wall", "-Wextra", "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
