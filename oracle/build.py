"""Build the CPU oracle (plain C, double precision, OpenMP) into liboracle.so.

Test infrastructure only; built with gcc, never linked with the GPU library.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


def build():
    cmd = ["gcc", "-O2", "-std=gnu11", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
           "-fPIC", "-shared", "-Wall", "-o", LIB, os.path.join(HERE, "hsa_oracle.c"), "-lm"]
    print("+", " ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


if __name__ == "__main__":
    build()
