"""Builds the CPU oracle (liboracle.so) in place: plain C99, -O2, no fast-math,
no FMA contraction. Test infrastructure only."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def build(verbose: bool = False) -> None:
    cmd = ["gcc", "-O2", "-std=c99", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-Wno-unused-parameter",
           os.path.join(HERE, "oracle.c"), "-o", os.path.join(HERE, "liboracle.so"), "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


if __name__ == "__main__":
    build(verbose=True)
