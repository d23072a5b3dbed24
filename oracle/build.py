"""Build the CPU reference (test infrastructure) into liboracle.so with gcc."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SO = os.path.join(HERE, "liboracle.so")


def build(verbose=False):
    # Plain -O2: no -ffast-math, so every float operation is IEEE-rounded in
    # source order.
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
           os.path.join(HERE, "oracle.c"), "-o", SO, "-lm"]
    subprocess.run(cmd, check=True, capture_output=not verbose)
    return SO


if __name__ == "__main__":
    build(verbose=True)
