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
# the same sources with device checks compiled in (HSA_ATTN_DEBUG=1 loads it)
LIB_DEBUG = os.path.join(HERE, "libhsa_attn_debug.so")
BUILD_DIR = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["api.cpp", "landmarks.hip", "prefill.hip", "decode.hip", "dhsa.hip", "dhsa_decode.hip",
           "swa.hip", "prefill_bwd.hip", "decode_noalloc.hip",
           "upper.hip", "prefill_qmajor.hip"]

FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Wno-unused-function", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
         # packed fp32 instructions stay off (see the design notes)
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src, debug):
    out_dir = os.path.join(BUILD_DIR, "debug") if debug else BUILD_DIR
    obj = os.path.join(out_dir, src + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    defs = ["-DHSA_DEVICE_CHECKS=1"] if debug else []
    cmd = [HIPCC] + FLAGS + defs + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{out}")
    if out.strip() and not debug:
        print(out, flush=True)
    return obj


def build(verbose=True, debug=True):
    """Compile every source for gfx950 and link libhsa_attn.so; with `debug`
    also the device-checked libhsa_attn_debug.so from the same sources."""
    variants = [False, True] if debug else [False]
    for v in variants:
        os.makedirs(os.path.join(BUILD_DIR, "debug") if v else BUILD_DIR, exist_ok=True)
    jobs = [(src, v) for v in variants for src in SOURCES]
    workers = min(len(jobs), max(1, os.cpu_count() or 1))
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    for v in variants:
        lib = LIB_DEBUG if v else LIB
        mine = [o for o, (_, jv) in zip(objs, jobs) if jv == v]
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", lib] + mine
        subprocess.run(cmd, check=True)
        if verbose:
            print("built", lib, flush=True)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
