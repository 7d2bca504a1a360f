"""Host-side AddressSanitizer + UndefinedBehaviorSanitizer builds of the CPU
code: the oracle, the seeded generator's host library, and the C-ABI layer
of the GPU library (argument validation, workspace carving, launch
sequencing: api.cpp, compiled with g++ and linked with the library's
unsanitized gfx950 objects).  GPU code is never instrumented.  Outputs go to
_build/asan/; the regular libraries are left untouched.

The builds use gcc's sanitizer runtimes (libasan, libubsan), so a process
that loads them must preload both (see run_sanitized.py).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
OUT = os.path.join(ROOT, "_build", "asan")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]

ORACLE = os.path.join(OUT, "liboracle.so")
SYNTH = os.path.join(OUT, "libsynth_host.so")
HSA = os.path.join(OUT, "libhsa_attn.so")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")


def build():
    sys.path.insert(0, ROOT)
    from chunk_hierarchical_sparse_amd import build as lib_build

    os.makedirs(OUT, exist_ok=True)
    _run(["gcc", "-std=gnu11", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC",
          "-shared", "-Wall"] + SAN + ["-o", ORACLE, os.path.join(ROOT, "oracle", "hsa_oracle.c"),
                                       "-lm"])
    _run(["gcc", "-std=gnu11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
          "-shared", "-Wall"] + SAN + ["-o", SYNTH, os.path.join(ROOT, "synth", "synth_host.c"),
                                       "-lm"])
    # the gfx950 objects of the regular build, api.cpp replaced by a sanitized one
    hip_objs = []
    for src in lib_build.SOURCES:
        if src == "api.cpp":
            continue
        obj = os.path.join(lib_build.BUILD_DIR, src + ".o")
        if not os.path.exists(obj):
            lib_build.build(verbose=False)
        hip_objs.append(obj)
    api_obj = os.path.join(OUT, "api.o")
    _run(["g++", "-std=c++17", "-fPIC", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
          "-I" + os.path.join(ROOT, "include"), "-I" + lib_build.CSRC] + SAN +
         ["-c", os.path.join(lib_build.CSRC, "api.cpp"), "-o", api_obj])
    _run(["g++", "-shared"] + SAN + ["-o", HSA, api_obj] + hip_objs +
         ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"])
    return ORACLE, SYNTH, HSA


if __name__ == "__main__":
    print("\n".join(build()))
