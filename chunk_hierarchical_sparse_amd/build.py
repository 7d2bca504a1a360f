"""Build libhsa_attn.so (gfx950 only) in-tree with hipcc.

Every translation unit is compiled separately (in parallel) and linked into
one shared library that exports the C ABI of include/hsa_attn.h.
"""
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libhsa_attn.so")
BUILD_DIR = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["api.cpp", "landmarks.hip", "prefill.hip", "decode.hip", "dhsa.hip", "dhsa_decode.hip",
           "swa.hip", "prefill_bwd.hip", "decode_noalloc.hip",
           "upper.hip"]

FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Wno-unused-function", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
         # packed fp32 instructions stay off (see the design notes)
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src):
    obj = os.path.join(BUILD_DIR, src + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC] + FLAGS + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{out}")
    if out.strip():
        print(out, flush=True)
    return obj


def build(verbose=True):
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", LIB] + objs
    subprocess.run(cmd, check=True)
    if verbose:
        print("built", LIB, flush=True)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
