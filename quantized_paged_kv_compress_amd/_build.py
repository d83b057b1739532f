"""Build libkvq.so (the HIP library behind include/kvq.h) for gfx950, in-tree.

    python -m quantized_paged_kv_compress_amd._build [--save-temps DIR]

Flags: -O3, C++17, --offload-arch=gfx950; -ffp-contract=off so that the RoPE products
and sums are rounded one at a time (fused multiply-adds are written out explicitly where
they are wanted); packed-fp32 instructions disabled.  The SHA-256 of the sources (and of
this file, which holds the flags) is compiled in as kvq_build_id(), so a loader can tell
a stale library from a current one.
"""
import hashlib
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "kvq_capi.hip")
LIB = os.path.join(HERE, "libkvq.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
SOURCES = [os.path.join(HERE, "csrc", f) for f in
           ("kvq_capi.hip", "kvq_kernels.hpp", "kvq_device.hpp", "kvq_layout.hpp")] + \
          [os.path.join(ROOT, "include", "kvq.h"), os.path.abspath(__file__)]


def source_hash() -> str:
    """SHA-256 (hex) of the library's sources and build flags."""
    h = hashlib.sha256()
    for f in SOURCES:
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode() + b"\0" + fh.read())
    return h.hexdigest()


def command(out=LIB, extra=()):
    return [
        HIPCC, "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
        "-ffp-contract=off",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-command-line-argument",
        "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
        f'-DKVQ_BUILD_ID="{source_hash()}"',
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
