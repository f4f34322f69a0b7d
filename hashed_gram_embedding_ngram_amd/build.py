"""Build libngram.so in-tree with hipcc for gfx950.

Flags: -O3; -ffp-contract=off so that every fp32 add and multiply stays the
single IEEE operation written in the source (the gate's fused multiply-add is
an explicit fmaf); packed fp32 instructions disabled (the kernels need none).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "ngram.hip")
LIB = os.path.join(HERE, "libngram.so")
ARCH = os.environ.get("NGRAM_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    "-O3", f"--offload-arch={ARCH}", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose: bool = False, extra=()) -> str:
    cmd = ["hipcc", *HIPCC_FLAGS, *extra, "-o", LIB + ".tmp", SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed to build libngram.so")
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
