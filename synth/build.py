"""Build the seeded-input libraries: libsynth_host.so (gcc, OpenMP) and
libsynth_gpu.so (hipcc, gfx950)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
HOST_SO = os.path.join(HERE, "libsynth_host.so")
GPU_SO = os.path.join(HERE, "libsynth_gpu.so")
HIP_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build_host(verbose=False):
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           os.path.join(HERE, "synth_host.c"), "-o", HOST_SO]
    subprocess.run(cmd, check=True, capture_output=not verbose)
    return HOST_SO


def build_gpu(verbose=False):
    cmd = ["hipcc", "--offload-arch=gfx950", "-O3", "-fPIC", "-shared", *HIP_FLAGS,
           os.path.join(HERE, "synth_gpu.hip"), "-o", GPU_SO]
    subprocess.run(cmd, check=True, capture_output=not verbose)
    return GPU_SO


def build(verbose=False):
    build_host(verbose)
    build_gpu(verbose)


if __name__ == "__main__":
    build(verbose=True)
