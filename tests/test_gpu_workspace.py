"""Workspace contents on entry do not matter: every entry point that takes a
workspace gives the same bits with a workspace filled with 0xFF bytes, one
filled with zeros, and one just used by a call of another shape (the library
clears whatever it accumulates into, in its own launches).  This also shows
run-to-run bitwise reproducibility, the backward's dK and dV included: their
sums over each chunk's list run in token order."""
import numpy as np
import pytest
import torch

import chunk_hierarchical_sparse_amd as hsa
import synth
from gpu_util import dev, gen, qkv, say

pytestmark = pytest.mark.gpu


def filled(nbytes, value):
    return torch.full((max(nbytes, 1),), value, dtype=torch.uint8, device="cuda")


def as_tuple(r):
    return tuple(r) if isinstance(r, (tuple, list)) else (r,)


def assert_same(a, b, what):
    a, b = as_tuple(a), as_tuple(b)
    assert len(a) == len(b), what
    for i, (x, y) in enumerate(zip(a, b)):
        assert x.dtype == y.dtype and x.shape == y.shape, f"{what}: result {i}"
        xv = x.contiguous().view(torch.uint8) if x.element_size() == 1 else \
            x.contiguous().view(torch.int16 if x.element_size() == 2 else torch.int32)
        yv = y.contiguous().view(xv.dtype)
        assert torch.equal(xv, yv), f"{what}: result {i} differs"


def three_ways(call, size, other_call, other_size, what):
    """call(ws) on a 0xFF workspace, on a zeroed one, and on one that
    other_call(ws) (another shape) has just used; all must agree bitwise."""
    r_ff = call(filled(size, 0xFF))
    r_zero = call(filled(size, 0))
    shared = filled(max(size, other_size), 0xFF)
    other_call(shared)
    r_reused = call(shared)
    torch.cuda.synchronize()
    assert_same(r_ff, r_zero, f"{what}: 0xFF vs zero workspace")
    assert_same(r_ff, r_reused, f"{what}: reused workspace")
    say(f"  {what}: identical")


def test_prefill_workspace_contents():
    Q, K, V = (dev(x) for x in qkv(1, 8, 2, 1500, 128, "bf16", 31))
    Q2, K2, V2 = (dev(x) for x in qkv(2, 4, 4, 2100, 128, "bf16", 32))
    n1 = hsa.hsa_prefill_workspace_size(1, 1500, 8, 2, 128, 64, 8, torch.bfloat16)
    n2 = hsa.hsa_prefill_workspace_size(2, 2100, 4, 4, 128, 32, 4, torch.bfloat16)
    three_ways(lambda ws: hsa.hsa_prefill(Q, K, V, 64, 8, return_selection=True, workspace=ws),
               n1, lambda ws: hsa.hsa_prefill(Q2, K2, V2, 32, 4, workspace=ws), n2, "prefill")


def test_prefill_interval_workspace_contents():
    Q, K, V = (dev(x) for x in qkv(1, 8, 2, 1300, 128, "bf16", 33))
    n1 = hsa.hsa_prefill_interval_workspace_size(1, 1300, 8, 2, 128, 64, 8, 8, torch.bfloat16)
    n2 = hsa.hsa_prefill_workspace_size(1, 1300, 8, 2, 128, 64, 8, torch.bfloat16)
    three_ways(lambda ws: hsa.hsa_prefill_interval(Q, K, V, 64, 8, 8, return_selection=True,
                                                   workspace=ws),
               n1, lambda ws: hsa.hsa_prefill(Q, K, V, 64, 8, workspace=ws), n2,
               "prefill, interval 8")


def test_decode_workspace_contents():
    B, Hq, Hkv, d, S, n_max = 4, 16, 4, 128, 64, 6000
    q = dev(gen((B, Hq, d), "bf16", 34, synth.TID_QDEC))
    Kc = dev(gen((B, Hkv, n_max, d), "bf16", 34, synth.TID_K))
    Vc = dev(gen((B, Hkv, n_max, d), "bf16", 34, synth.TID_V))
    lmk = hsa.hsa_build_landmarks(Kc, S)
    n1 = hsa.hsa_decode_workspace_size(B, Hq, Hkv, d, S, 8, 5900)
    n2 = hsa.hsa_decode_workspace_size(B, Hq, Hkv, d, S, 16, 3000)
    three_ways(lambda ws: hsa.hsa_decode(q, Kc, Vc, lmk, 5900, S, 8, return_selection=True,
                                         workspace=ws),
               n1, lambda ws: hsa.hsa_decode(q, Kc, Vc, lmk, 3000, S, 16, workspace=ws), n2,
               "decode")


def test_dhsa_prefill_workspace_contents():
    L, H, d = 1200, 2, 128
    Q, K, V = (dev(x) for x in qkv(1, H, H, L, d, "bf16", 35))
    offs = synth.chunk_offsets(L, 16, 128, seed=35)
    offs2 = synth.chunk_offsets(L, 5, 40, seed=36)
    n1 = hsa.dhsa_prefill_workspace_size(1, L, H, d, len(offs) - 1, torch.bfloat16)
    n2 = hsa.dhsa_prefill_workspace_size(1, L, H, d, len(offs2) - 1, torch.bfloat16)
    three_ways(lambda ws: hsa.dhsa_prefill(Q, K, V, offs, 300, return_order=True, workspace=ws),
               n1, lambda ws: hsa.dhsa_prefill(Q, K, V, offs2, 100, workspace=ws), n2,
               "dhsa prefill")


def test_dhsa_decode_workspace_contents():
    B, H, d, n_max = 2, 2, 128, 3000
    offs_all = synth.chunk_offsets(2800, 16, 128, seed=37)
    offs = offs_all[:-1]
    n = len(offs) - 1
    m = int(offs_all[-1] - offs_all[-2])
    Kc = dev(gen((B, H, n_max, d), "bf16", 37, synth.TID_K))
    Vc = dev(gen((B, H, n_max, d), "bf16", 37, synth.TID_V))
    qcur = dev(gen((B, H, m, d), "bf16", 37, synth.TID_QDEC))
    khat = hsa.dhsa_build_chunk_keys(Kc, offs, n_cap=n + 2)
    offs_b = offs[: n // 2 + 1]
    n1 = hsa.dhsa_decode_workspace_size(B, H, d, n, 700, n_max)
    n2 = hsa.dhsa_decode_workspace_size(B, H, d, len(offs_b) - 1, 2000, n_max)
    three_ways(lambda ws: hsa.dhsa_decode(qcur, Kc, Vc, khat, offs, 700, return_order=True,
                                          workspace=ws),
               n1, lambda ws: hsa.dhsa_decode(qcur, Kc, Vc, khat, offs_b, 2000, workspace=ws),
               n2, "dhsa decode")


def test_backward_workspace_contents():
    B, Hq, Hkv, L, d = 1, 8, 2, 1100, 128
    Q, K, V = (dev(x) for x in qkv(B, Hq, Hkv, L, d, "bf16", 38, 0.5))
    dO = dev(gen((B, Hq, L, d), "bf16", 38, synth.TID_DO))
    Q2, K2, V2 = (dev(x) for x in qkv(1, 4, 4, 1700, d, "bf16", 39, 0.5))
    dO2 = dev(gen((1, 4, 1700, d), "bf16", 39, synth.TID_DO))
    n1 = hsa.hsa_prefill_backward_workspace_size(B, L, Hq, Hkv, d, 64, 8, torch.bfloat16)
    n2 = hsa.hsa_prefill_backward_workspace_size(1, 1700, 4, 4, d, 32, 4, torch.bfloat16)
    three_ways(lambda ws: hsa.hsa_prefill_backward(Q, K, V, dO, 64, 8, workspace=ws), n1,
               lambda ws: hsa.hsa_prefill_backward(Q2, K2, V2, dO2, 32, 4, workspace=ws), n2,
               "backward")
