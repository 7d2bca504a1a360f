"""The C-ABI library loads, exports every entry point its header declares,
and rejects invalid arguments on the host before touching the GPU (these
calls return before any HIP call, so they run without a GPU)."""
import ctypes
import os
import re

import pytest
import torch  # noqa: F401  (the library binds to torch's HIP runtime)

import chunk_hierarchical_sparse_amd as hsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hsa_attn.h")

INV, UNS, WS = hsa.HSA_ERR_INVALID_ARGUMENT, hsa.HSA_ERR_UNSUPPORTED, hsa.HSA_ERR_WORKSPACE_TOO_SMALL
F32, BF16 = hsa.DTYPE_F32, hsa.DTYPE_BF16


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\**\s+\**(\w+)\(", text, re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ["hsa_build_landmarks", "hsa_prefill", "hsa_decode", "dhsa_prefill",
              "hsa_prefill_workspace_size", "hsa_decode_workspace_size",
              "dhsa_prefill_workspace_size", "hsa_status_string", "hsa_last_error_message",
              "hsa_prefill_interval", "dhsa_build_chunk_keys", "dhsa_decode", "swa_prefill",
              "swa_decode", "hsa_prefill_backward", "hsa_prefill_backward_workspace_size"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(hsa.lib_path())
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_status_strings():
    assert hsa.hsa_status_string(0).startswith("HSA_OK")
    for code in range(1, 5):
        assert hsa.hsa_status_string(code).startswith("HSA_ERR")
    assert "unknown" in hsa.hsa_status_string(99)


def lib():
    return hsa.load_library()


def msg():
    return lib().hsa_last_error_message().decode()


def prefill(**kw):
    a = dict(Q=1, K=1, V=1, lmk=None, O=1, sel=None, w=None, B=1, L=256, Hq=4, Hkv=2, d=128,
             S=64, topk=8, dt=BF16, ws=None, wsb=0)
    a.update(kw)
    return lib().hsa_prefill(a["Q"], a["K"], a["V"], a["lmk"], a["O"], a["sel"], a["w"], a["B"],
                             a["L"], a["Hq"], a["Hkv"], a["d"], a["S"], a["topk"], a["dt"],
                             a["ws"], a["wsb"], None)


def test_prefill_validation():
    assert prefill(Hq=3, Hkv=2) == INV
    assert prefill(Hkv=0) == INV
    assert prefill(d=96) == UNS
    assert prefill(S=0) == INV
    assert prefill(S=2048) == INV
    assert prefill(topk=0) == INV
    assert prefill(topk=33) == INV
    assert prefill(dt=7) == UNS
    assert prefill(Hq=128, Hkv=2) == UNS
    assert prefill(B=-1) == INV
    assert prefill(Q=None) == INV and "NULL" in msg()
    assert prefill(L=1 << 30, topk=32) == UNS
    # valid arguments, but no workspace
    assert prefill() == WS and "workspace needs" in msg()
    need = lib().hsa_prefill_workspace_size(1, 256, 4, 2, 128, 64, 8, BF16)
    assert need > 0
    assert prefill(ws=1 << 20, wsb=need - 1) == WS
    # nothing to do is success without any launch
    assert prefill(L=0) == hsa.HSA_OK and prefill(B=0) == hsa.HSA_OK


def test_workspace_sizes_grow_with_the_problem():
    a = lib().hsa_prefill_workspace_size(1, 4096, 16, 4, 128, 64, 8, BF16)
    b = lib().hsa_prefill_workspace_size(1, 8192, 16, 4, 128, 64, 8, BF16)
    c = lib().hsa_prefill_workspace_size(1, 4096, 16, 4, 128, 64, 8, F32)
    assert 0 < a < b and c > a
    assert lib().hsa_prefill_workspace_size(1, 4096, 16, 3, 128, 64, 8, BF16) == 0
    assert lib().hsa_decode_workspace_size(32, 32, 8, 128, 64, 8, 131072) > 0
    assert lib().dhsa_prefill_workspace_size(1, 16384, 8, 128, 228, BF16) > 0
    assert lib().dhsa_prefill_workspace_size(1, 16384, 8, 128, 0, BF16) == 0


def test_landmark_validation():
    L = lib()
    assert L.hsa_build_landmarks(1, 1, 1, 2, 256, 128, 64, 0, 5, BF16, None) == INV  # > L/S
    assert L.hsa_build_landmarks(1, 1, 1, 2, 256, 128, 64, 3, 2, BF16, None) == INV
    assert L.hsa_build_landmarks(1, 1, 1, 2, 256, 100, 64, 0, 4, BF16, None) == UNS
    assert L.hsa_build_landmarks(None, 1, 1, 2, 256, 128, 64, 0, 4, BF16, None) == INV
    assert L.hsa_build_landmarks(1, 1, 1, 2, 256, 128, 64, 2, 2, BF16, None) == hsa.HSA_OK


def decode(**kw):
    a = dict(q=1, K=1, V=1, lmk=1, n_ctx=4096, n_max=4096, o=1, sel=None, w=None, B=2, Hq=8,
             Hkv=2, d=128, S=64, topk=8, dt=BF16, ws=None, wsb=0)
    a.update(kw)
    return lib().hsa_decode(a["q"], a["K"], a["V"], a["lmk"], a["n_ctx"], a["n_max"], a["o"],
                            a["sel"], a["w"], a["B"], a["Hq"], a["Hkv"], a["d"], a["S"],
                            a["topk"], a["dt"], a["ws"], a["wsb"], None)


def test_decode_validation():
    assert decode(n_ctx=5000) == INV  # beyond the cache
    assert decode(n_ctx=-1) == INV
    assert decode(Hq=6, Hkv=4) == INV
    assert decode(K=None) == INV
    assert decode(lmk=None) == INV
    assert decode() == WS
    assert decode(B=0) == hsa.HSA_OK


def dhsa(offsets, **kw):
    import numpy as np
    offs = np.ascontiguousarray(offsets, dtype=np.int32)
    a = dict(Q=1, K=1, V=1, nc=len(offs) - 1, budget=64, O=1, mask=None, order=None, B=1,
             L=int(offs[-1]), H=2, d=128, dt=BF16, ws=None, wsb=0)
    a.update(kw)
    return lib().dhsa_prefill(a["Q"], a["K"], a["V"], offs.ctypes.data, a["nc"], a["budget"],
                              a["O"], a["mask"], a["order"], a["B"], a["L"], a["H"], a["d"],
                              a["dt"], a["ws"], a["wsb"], None)


def test_dhsa_validation():
    assert dhsa([0, 10, 10, 30]) == INV  # empty chunk
    assert dhsa([0, 20, 10, 30]) == INV  # decreasing
    assert dhsa([1, 10, 30]) == INV      # does not start at 0
    assert dhsa([0, 10, 30], L=31) == INV  # does not end at L
    assert dhsa([0, 10, 30], budget=0) == INV
    assert dhsa([0, 10, 30], dt=F32) == WS  # fp32 accepted: only the workspace is missing
    assert dhsa([0, 10, 30], dt=7) == UNS
    assert dhsa([0, 10, 30], d=80) == UNS
    assert dhsa([0, 10, 30], Q=None) == INV
    assert dhsa([0, 10, 30]) == WS
    assert dhsa([0, 10, 30], B=0) == hsa.HSA_OK


def test_python_layer_rejects_host_tensors():
    q = torch.zeros(1, 2, 64, 64)
    with pytest.raises(ValueError):
        hsa.hsa_prefill(q, q, q, 16, 2)


def _offs(vals):
    import numpy as np
    a = np.asarray(vals, dtype=np.int32)
    return a, a.ctypes.data


def dhsa_decode_call(**kw):
    offs, optr = _offs(kw.pop("offsets", [0, 4, 9, 20]))
    a = dict(q=1, m=3, K=1, V=1, n_max=64, khat=1, n_cap=8, n=len(offs) - 1, budget=16, o=1,
             B=1, H=2, d=128, dt=BF16, ws=None, wsb=0, optr=optr)
    a.update(kw)
    return lib().dhsa_decode(a["q"], a["m"], a["K"], a["V"], a["n_max"], a["khat"], a["n_cap"],
                             a["optr"], a["n"], a["budget"], a["o"], None, a["B"], a["H"], a["d"],
                             a["dt"], a["ws"], a["wsb"], None)


def test_dhsa_decode_validation():
    assert dhsa_decode_call(m=0) == INV
    assert dhsa_decode_call(d=96) == UNS
    assert dhsa_decode_call(dt=7) == UNS
    assert dhsa_decode_call(budget=0) == INV
    assert dhsa_decode_call(n_cap=2) == INV
    assert dhsa_decode_call(offsets=[1, 4, 9, 20]) == INV and "start at 0" in msg()
    assert dhsa_decode_call(offsets=[0, 4, 4, 20]) == INV and "increasing" in msg()
    assert dhsa_decode_call(m=50) == INV and "past the cache" in msg()
    assert dhsa_decode_call(q=None) == INV and "NULL" in msg()
    assert dhsa_decode_call(offsets=list(range(0, 5000)), n_cap=5000, n_max=1 << 20) == UNS
    assert dhsa_decode_call(B=1 << 20, H=64, budget=1 << 20, n_max=1 << 21) == UNS
    assert dhsa_decode_call() == WS and "workspace needs" in msg()
    need = lib().dhsa_decode_workspace_size(1, 2, 128, 3, 16, 64)
    assert need > 0
    assert dhsa_decode_call(ws=1 << 20, wsb=need - 1) == WS


def test_dhsa_build_chunk_keys_validation():
    offs, optr = _offs([0, 4, 9, 20])

    def call(**kw):
        a = dict(K=1, khat=1, n=3, cb=0, ce=3, B=1, H=2, n_max=64, d=128, n_cap=3, dt=BF16,
                 ws=None, wsb=0, optr=optr)
        a.update(kw)
        return lib().dhsa_build_chunk_keys(a["K"], a["khat"], a["optr"], a["n"], a["cb"],
                                           a["ce"], a["B"], a["H"], a["n_max"], a["d"],
                                           a["n_cap"], a["dt"], a["ws"], a["wsb"], None)

    assert call(ce=4) == INV
    assert call(cb=2, ce=1) == INV
    assert call(n_cap=2) == INV
    assert call(n_max=10) == INV and "past the cache" in msg()
    assert call(d=64 + 1) == UNS
    assert call(K=None) == INV
    assert call() == WS
    assert call(cb=1, ce=1) == 0  # empty range: nothing to do


def test_prefill_interval_validation():
    def call(**kw):
        a = dict(R=8, B=1, L=256, ws=None, wsb=0)
        a.update(kw)
        return lib().hsa_prefill_interval(1, 1, 1, None, 1, None, None, a["B"], a["L"], 4, 2,
                                          128, 64, 8, a["R"], BF16, a["ws"], a["wsb"], None)
    assert call(R=0) == INV and "interval" in msg()
    assert call() == WS
    n8 = lib().hsa_prefill_interval_workspace_size(1, 256, 4, 2, 128, 64, 8, 8, BF16)
    n1 = lib().hsa_prefill_interval_workspace_size(1, 256, 4, 2, 128, 64, 8, 1, BF16)
    assert n1 == lib().hsa_prefill_workspace_size(1, 256, 4, 2, 128, 64, 8, BF16)
    assert 0 < n8 < n1  # one selection row per block
    assert lib().hsa_prefill_interval_workspace_size(1, 256, 4, 2, 128, 64, 8, 0, BF16) == 0


def swa_call(which, **kw):
    a = dict(Q=1, K=1, V=1, O=1, B=1, L=256, Hq=4, Hkv=2, d=128, W=512, dt=BF16, pos=10,
             n_max=256)
    a.update(kw)
    if which == "prefill":
        return lib().swa_prefill(a["Q"], a["K"], a["V"], a["O"], a["B"], a["L"], a["Hq"],
                                 a["Hkv"], a["d"], a["W"], a["dt"], None)
    return lib().swa_decode(a["Q"], a["K"], a["V"], a["pos"], a["n_max"], a["W"], a["O"],
                            a["B"], a["Hq"], a["Hkv"], a["d"], a["dt"], None)


@pytest.mark.parametrize("which", ["prefill", "decode"])
def test_swa_validation(which):
    assert swa_call(which, Hq=3, Hkv=2) == INV
    assert swa_call(which, Hkv=0) == INV
    assert swa_call(which, d=96) == UNS
    assert swa_call(which, W=0) == INV
    assert swa_call(which, dt=7) == UNS
    assert swa_call(which, B=-1) == INV
    assert swa_call(which, Q=None) == INV and "NULL" in msg()
    assert swa_call(which, B=0) == hsa.HSA_OK  # nothing to do, nothing launched
    if which == "prefill":
        assert swa_call(which, L=-1) == INV
        assert swa_call(which, L=0) == hsa.HSA_OK
        assert swa_call(which, B=64, Hq=64, Hkv=8, L=1 << 20) == UNS
    else:
        assert swa_call(which, pos=-1) == INV
        assert swa_call(which, pos=256) == INV and "pos" in msg()


def backward_call(**kw):
    a = dict(Q=1, K=1, V=1, dO=1, lmk=None, dQ=1, dK=1, dV=1, B=1, L=256, Hq=4, Hkv=2, d=128,
             S=64, topk=8, dt=BF16, ws=None, wsb=0)
    a.update(kw)
    return lib().hsa_prefill_backward(a["Q"], a["K"], a["V"], a["dO"], a["lmk"], a["dQ"], a["dK"],
                                      a["dV"], a["B"], a["L"], a["Hq"], a["Hkv"], a["d"], a["S"],
                                      a["topk"], a["dt"], a["ws"], a["wsb"], None)


def test_backward_validation():
    assert backward_call(dt=F32) == UNS and "bf16" in msg()
    assert backward_call(S=128) == UNS and "S <= 64" in msg()
    assert backward_call(Hq=3) == INV
    assert backward_call(dO=None) == INV and "NULL" in msg()
    assert backward_call() == WS
    need = lib().hsa_prefill_backward_workspace_size(1, 256, 4, 2, 128, 64, 8, BF16)
    assert need > lib().hsa_prefill_workspace_size(1, 256, 4, 2, 128, 64, 8, BF16)
    assert backward_call(ws=1 << 20, wsb=need - 1) == WS
    assert lib().hsa_prefill_backward_workspace_size(1, 256, 4, 2, 128, 64, 8, F32) == 0
    assert lib().hsa_prefill_backward_workspace_size(1, 256, 4, 2, 128, 128, 8, BF16) == 0
    assert backward_call(B=0) == hsa.HSA_OK


def test_hsa_swa_decode_validation():
    def call(**kw):
        a = dict(n_ctx=1000, n_max=2000, W=512, B=1, Hq=4, Hkv=2, d=128, S=64, K=8, dt=BF16,
                 ws=None, wsb=0, o=1)
        a.update(kw)
        return lib().hsa_swa_decode(1, 1, 1, 1, a["n_ctx"], a["n_max"], a["W"], a["o"], a["o"],
                                    None, None, a["B"], a["Hq"], a["Hkv"], a["d"], a["S"], a["K"],
                                    a["dt"], a["ws"], a["wsb"], None)
    assert call(S=128) == UNS
    assert call(W=5000, n_ctx=8000, n_max=9000) == UNS
    assert call(W=0) == INV
    assert call(n_ctx=2000) == INV
    assert call(Hq=3) == INV
    assert call(o=None) == INV
    assert call() == WS and "workspace needs" in msg()
    assert lib().hsa_swa_decode_workspace_size(1, 4, 2, 128, 64, 8, 1000, 512) > \
        lib().hsa_decode_workspace_size(1, 4, 2, 128, 64, 8, 1000)


LOG_SCRIPT = r"""
import chunk_hierarchical_sparse_amd as hsa
lib = hsa.load_library()
st = lib.hsa_prefill(1, 1, 1, None, 1, None, None, 1, 256, 4, 2, 128, 0, 8, hsa.DTYPE_BF16,
                     None, 0, None)
assert st == hsa.HSA_ERR_INVALID_ARGUMENT, st
"""


@pytest.mark.parametrize("value,shown", [("1", True), ("0", False), ("", False)])
def test_log_lines_name_the_call_and_its_status(value, shown):
    # HSA_ATTN_LOG is read once per process, so each setting runs in a child
    import subprocess
    import sys
    env = dict(os.environ, HSA_ATTN_LOG=value, PYTHONPATH=ROOT)
    r = subprocess.run([sys.executable, "-c", LOG_SCRIPT], env=env, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    lines = [l for l in r.stderr.splitlines() if l.startswith("hsa_attn:")]
    if not shown:
        assert lines == []
        return
    assert lines[0] == "hsa_attn: hsa_prefill B=1 L=256 Hq=4 Hkv=2 d=128 S=0 topk=8 dtype=1"
    assert lines[1].startswith("hsa_attn:   status 1: ") and "chunk size" in lines[1]


def test_release_library_has_no_device_checks():
    assert lib().hsa_device_checks_enabled() == 0
    assert lib().hsa_device_checks_selftest(1, None) == UNS and "debug library" in msg()


DEBUG_SCRIPT = r"""
import re
import chunk_hierarchical_sparse_amd as hsa
path = hsa.lib_path()
assert path.endswith("libhsa_attn_debug.so"), path
lib = hsa.load_library()
assert lib.hsa_device_checks_enabled() == 1
import ctypes
raw = ctypes.CDLL(path)
text = open(HEADER).read()
names = set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\**\s+\**(\w+)\(", text, re.M))
missing = [n for n in names if not hasattr(raw, n)]
assert not missing, missing
st = lib.hsa_prefill(1, 1, 1, None, 1, None, None, 1, 256, 4, 2, 128, 0, 8, hsa.DTYPE_BF16,
                     None, 0, None)
assert st == hsa.HSA_ERR_INVALID_ARGUMENT, st
print("ok")
"""


def test_debug_library_loads_with_device_checks():
    # HSA_ATTN_DEBUG=1 selects the device-checked build of the same sources
    import subprocess
    import sys
    env = dict(os.environ, HSA_ATTN_DEBUG="1", PYTHONPATH=ROOT)
    r = subprocess.run([sys.executable, "-c", f"HEADER = {HEADER!r}\n" + DEBUG_SCRIPT], env=env,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "ok" in r.stdout, r.stderr[-3000:]
