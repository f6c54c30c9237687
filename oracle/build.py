"""Builds the CPU oracle in place, twice from the same source: liboracle.so
(plain C99, -O2, no fast-math, no FMA contraction, one thread; calls
between the library's own functions may be inlined) and
liboracle_omp.so (the same flags plus OpenMP: the loops over independent
matrix rows run on all host cores; the arithmetic of every row is
unchanged). Test infrastructure only."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
COMMON = ["gcc", "-O2", "-fno-semantic-interposition", "-std=c99", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared",
          "-Wall", "-Wextra", "-Wno-unused-parameter"]


def build(verbose: bool = False) -> None:
    src = os.path.join(HERE, "oracle.c")
    for extra, out in ((["-Wno-unknown-pragmas"], "liboracle.so"), (["-fopenmp"], "liboracle_omp.so")):
        cmd = COMMON + extra + [src, "-o", os.path.join(HERE, out), "-lm"]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)


if __name__ == "__main__":
    build(verbose=True)
