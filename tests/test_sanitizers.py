"""The CPU code under AddressSanitizer and UndefinedBehaviorSanitizer: the
oracle, the seeded generator's host library and the C-ABI layer (argument
validation) are rebuilt with -fsanitize=address,undefined (host code only;
no GPU code is instrumented) and the CPU test files that exercise them run
against those builds in a child process with the sanitizer runtimes
preloaded.  Any sanitizer report aborts the child (halt on error, no
recovery), so the test fails."""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _runtime(name):
    r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.slow
def test_cpu_code_under_asan_and_ubsan():
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not found")
    sys.path.insert(0, os.path.join(HERE, "sanitize"))
    import build_asan
    build_asan.build()
    env = dict(os.environ)
    env["LD_PRELOAD"] = f"{asan}:{ubsan}"
    # python and torch are not instrumented: leaks and allocator pairing in
    # them are not ours to report
    env["ASAN_OPTIONS"] = "detect_leaks=0:alloc_dealloc_mismatch=0:detect_odr_violation=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    files = [os.path.join(HERE, f) for f in ("test_oracle_pins.py", "test_oracle_golden.py",
                                             "test_synth.py", "test_abi.py")]
    r = subprocess.run([sys.executable, os.path.join(HERE, "sanitize", "run_sanitized.py"), "-x",
                        "-q", "-m", "not gpu", "-p", "no:cacheprovider"] + files,
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
