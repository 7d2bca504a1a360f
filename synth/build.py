"""Build the seeded input generator libraries.

libsynth_host.so   gcc, OpenMP; used by the oracle side and by tests.
libsynth_device.so hipcc for gfx950; fills device buffers with the same bits.

Both are compiled with floating-point contraction off so the double-precision
Box-Muller arithmetic in synth_core.h rounds identically on host and device.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(HERE, "libsynth_host.so")
DEVICE_LIB = os.path.join(HERE, "libsynth_device.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _run(cmd):
    print("+", " ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build_host():
    _run(["gcc", "-O2", "-std=gnu11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
          "-fPIC", "-shared", "-Wall", "-o", HOST_LIB, os.path.join(HERE, "synth_host.c"), "-lm"])


def build_device():
    _run([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-ffp-contract=off",
          "-fno-fast-math", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fPIC", "-shared", "-o", DEVICE_LIB, os.path.join(HERE, "synth_device.hip")])


def build():
    build_host()
    build_device()


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "host":
        build_host()
    else:
        build()
