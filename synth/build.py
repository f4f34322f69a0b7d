"""Build synth/libsynth.so (GPU fill kernels for the synthetic inputs) and
synth/libprobe.so (a bare-gather measurement probe for the benchmark)."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "fill.hip")
LIB = os.path.join(HERE, "libsynth.so")


PROBE_SRC = os.path.join(HERE, "probe.hip")
PROBE_LIB = os.path.join(HERE, "libprobe.so")


def _hipcc(src, lib, verbose):
    cmd = ["hipcc", "-O3", "--offload-arch=gfx950", "-std=c++17", "-fPIC", "-shared",
           "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-o", lib + ".tmp", src]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed to build {os.path.basename(lib)}")
    os.replace(lib + ".tmp", lib)


def build(verbose: bool = False) -> str:
    _hipcc(SRC, LIB, verbose)
    _hipcc(PROBE_SRC, PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
