"""Build libkvq.so (the HIP library behind include/kvq.h) for gfx950, in-tree.

    python -m quantized_paged_kv_compress_amd._build [--save-temps DIR]

Flags: -O3, C++17, --offload-arch=gfx950; -ffp-contract=off so that the RoPE products
and sums are rounded one at a time (fused multiply-adds are written out explicitly where
they are wanted); packed-fp32 instructions disabled.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "kvq_capi.hip")
LIB = os.path.join(HERE, "libkvq.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"


def command(out=LIB, extra=()):
    return [
        HIPCC, "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
        "-ffp-contract=off",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-command-line-argument",
        "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
        SRC, "-o", out, *extra,
    ]


def build(verbose: bool = False, extra=()) -> str:
    tmp = LIB + ".tmp"
    cmd = command(tmp, extra)
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    extra = []
    if "--save-temps" in sys.argv:
        d = sys.argv[sys.argv.index("--save-temps") + 1]
        os.makedirs(d, exist_ok=True)
        extra = [f"-save-temps={'obj'}"]
        os.chdir(d)
    build(verbose=True, extra=extra)
