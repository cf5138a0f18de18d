"""Compile the CPU oracle (test infrastructure only) into oracle/libring_oracle.so."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ring_oracle.c")
LIB = os.path.join(HERE, "libring_oracle.so")


def build(verbose: bool = False) -> str:
    # No fast-math and no contraction: every add is one IEEE binary32 add.
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c99", "-Wall",
           "-fPIC", "-shared", SRC, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
