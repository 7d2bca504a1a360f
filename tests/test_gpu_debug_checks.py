"""The device-checked debug library (HSA_ATTN_DEBUG=1): every compute entry
point runs with its gather-index checks and reports none failed, its results
agree with the release library's, and the self-test shows that a failed
check is reported (with its source line) and then cleared."""
import os
import subprocess
import sys

import numpy as np
import pytest

import chunk_hierarchical_sparse_amd as hsa
from gpu_util import TOL_BF16, TOL_F32_REL, say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CHILD = os.path.join(ROOT, "tests", "debug_checks_child.py")


def run_child(debug, path):
    env = dict(os.environ, HSA_ATTN_DEBUG="1" if debug else "0",
               PYTHONPATH=os.pathsep.join([ROOT, os.path.join(ROOT, "tests")]))
    say(f"child HSA_ATTN_DEBUG={int(debug)}")
    r = subprocess.run([sys.executable, "-u", CHILD, path], env=env, capture_output=True,
                       text=True, timeout=400)
    say(r.stdout[-2000:])
    assert r.returncode == 0, r.stderr[-4000:]
    return np.load(path)


def test_debug_library_checks_pass_and_match_release(tmp_path):
    assert os.path.exists(hsa._build.LIB_DEBUG), "the debug library is not built"
    dbg = run_child(True, str(tmp_path / "debug.npz"))
    rel = run_child(False, str(tmp_path / "release.npz"))
    st = dbg["selftest"]
    assert st.tolist() == [hsa.HSA_OK, hsa.HSA_ERR_HIP, hsa.HSA_OK], st
    msg = str(dbg["selftest_msg"])
    assert "device check failed at" in msg and "landmarks.hip:" in msg and "(1 failures)" in msg, msg
    assert str(dbg["selftest_msg2"]) == msg  # cleared after the report: counted once again
    assert "selftest" not in rel.files
    for key in rel.files:
        a, b = dbg[key], rel[key]
        assert a.shape == b.shape, key
        if a.dtype.kind in "iu":
            assert (a == b).all(), f"{key}: integer outputs differ"
        else:
            scale = float(np.abs(b).max()) or 1.0
            err = float(np.abs(a.astype(np.float64) - b).max())
            tol = TOL_F32_REL * scale if ("f32" in key or key in ("lmk",) or "khat" in key) \
                else TOL_BF16
            assert err <= tol, f"{key}: debug vs release differ by {err}"
            say(f"  {key}: max |debug - release| = {err:.3g}")
