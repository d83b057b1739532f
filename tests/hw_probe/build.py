"""Build tests/hw_probe/libhwprobe.so (test support: the hardware exp2 / reciprocal error
probe used by tests/test_gpu_hw_bounds.py) for gfx950, in-tree.

    python tests/hw_probe/build.py
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "hwprobe.hip")
LIB = os.path.join(HERE, "libhwprobe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared", "-ffp-contract=off",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall",
           "-Wno-unused-command-line-argument", SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
