"""Build libmkd.so (the decode megakernel C-ABI library) in-tree with hipcc for gfx950."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
SO = os.path.join(HERE, "libmkd.so")

HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 instructions stay off (only scalar fp32 VALU ops are emitted)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
SOURCES = ["mkd_kernels.hip", "mkd_plan.cpp", "mkd_engine.cpp", "mkd_static.hip", "mkd_serve.hip", "mkd_litmus.hip"]


def build(verbose=False, extra=(), out=SO):
    """Compile every source and link `out`; `extra` holds additional hipcc flags (e.g.
    -DMKD_RING=8 to change a tuning constant)."""
    objs = []
    tag = str(abs(hash((tuple(extra), out))))
    for src in SOURCES:
        obj = os.path.join(CSRC, src.rsplit(".", 1)[0] + "." + tag + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = ["hipcc", *HIP_FLAGS, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stderr)
            raise RuntimeError(f"hipcc failed on {src}")
        objs.append(obj)
    cmd = ["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stderr)
        raise RuntimeError("link of libmkd.so failed")
    for o in objs:
        os.remove(o)
    return out


if __name__ == "__main__":
    build(verbose=True)
