"""Run CPU tests against the sanitized builds of build_asan.py, in this
process: the loaders are pointed at _build/asan/ before anything is loaded.
Start it with libasan and libubsan preloaded (LD_PRELOAD), e.g. through
tests/test_sanitizers.py.  Arguments are passed to pytest."""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.dirname(HERE))

sys.path.insert(0, HERE)
import build_asan  # noqa: E402
import oracle.build  # noqa: E402
import synth.build  # noqa: E402
import chunk_hierarchical_sparse_amd.build as lib_build  # noqa: E402

oracle.build.LIB = build_asan.ORACLE
synth.build.HOST_LIB = build_asan.SYNTH
lib_build.LIB = build_asan.HSA

import pytest  # noqa: E402

sys.exit(pytest.main(sys.argv[1:]))
