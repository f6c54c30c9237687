"""Builds the input generator libraries in place: libsynth.so (host C, OpenMP)
and libsynth_dev.so (its HIP twin for gfx950)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose: bool = False) -> None:
    host = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
            os.path.join(HERE, "synth.c"), "-o", os.path.join(HERE, "libsynth.so"), "-lm"]
    dev = ["hipcc", *HIP_FLAGS, os.path.join(HERE, "synth_dev.hip"),
           "-o", os.path.join(HERE, "libsynth_dev.so")]
    for cmd in (host, dev):
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True, stderr=None if verbose else subprocess.DEVNULL)


if __name__ == "__main__":
    build(verbose=True)
