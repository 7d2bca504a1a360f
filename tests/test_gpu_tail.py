"""Key/value tensors whose allocation continues past their last row with
bf16 NaN: the kernels that stage blocks of up to 128 keys (DHSA attention,
sliding-window prefill) and the 64-key chunk stagers (HSA prefill, decode)
must never read past a tensor's last row, so every output stays finite and
matches the oracle.  Every read here stays inside the allocation: the NaN
tail is part of the same buffer, past the [B,H,L,d] view the kernels get."""
import numpy as np
import pytest
import torch

import chunk_hierarchical_sparse_amd as hsa
import oracle
import synth
from gpu_util import MARGIN, check_out, compare_selection, host, qkv, say

pytestmark = pytest.mark.gpu

TAIL = 256 * 128  # elements of NaN after the view: 256 rows of d = 128


def nan_tailed(arr):
    """A contiguous device view of arr (bf16 bits) whose allocation holds
    TAIL bf16 NaN elements after it."""
    n = arr.size
    buf = torch.full((n + TAIL,), float("nan"), dtype=torch.bfloat16, device="cuda")
    src = torch.from_numpy(np.ascontiguousarray(arr).reshape(-1).view(np.int16))
    buf[:n].copy_(src.view(torch.bfloat16).cuda())
    return buf[:n].view(arr.shape)


def plain(arr):
    return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()


@pytest.mark.parametrize("L,lo,hi", [(700, 16, 128), (1000, 100, 300), (517, 5, 40)])
def test_dhsa_last_chunk_short_with_nan_tail(L, lo, hi):
    # the last chunk of the last head is shorter than a 128-key block
    B, H, d, budget = 1, 2, 128, 160
    offs = synth.chunk_offsets(L, lo, hi, seed=300 + L)
    say(f"dhsa nan tail L={L} chunks={len(offs) - 1} last={offs[-1] - offs[-2]}")
    Q, K, V = qkv(B, H, H, L, d, "bf16", 300 + L)
    out = hsa.dhsa_prefill(plain(Q), nan_tailed(K), nan_tailed(V), offs, budget)
    torch.cuda.synchronize()
    out = host(out)
    assert np.isfinite(out).all(), "non-finite DHSA output"
    ref = oracle.dhsa_prefill(Q, K, V, offs, budget)
    keep = ref["margin"] > MARGIN
    check_out(out[keep], ref["out"][keep], "bf16", "dhsa output")


@pytest.mark.parametrize("L,W", [(700, 100), (1000, 512), (129, 600)])
def test_swa_prefill_with_nan_tail(L, W):
    B, Hq, Hkv, d = 1, 8, 2, 128
    say(f"swa nan tail L={L} W={W}")
    Q, K, V = qkv(B, Hq, Hkv, L, d, "bf16", 310 + L)
    out = hsa.swa_prefill(plain(Q), nan_tailed(K), nan_tailed(V), W)
    torch.cuda.synchronize()
    out = host(out)
    assert np.isfinite(out).all(), "non-finite SWA output"
    check_out(out, oracle.swa_prefill(Q, K, V, W), "bf16", "swa output")


def test_hsa_prefill_and_decode_with_nan_tail():
    B, Hq, Hkv, L, d, S, K = 1, 8, 2, 1000, 128, 64, 4
    say(f"hsa nan tail L={L} S={S} K={K}")
    Q, Kx, V = qkv(B, Hq, Hkv, L, d, "bf16", 320, 0.5)
    out, sel, _ = hsa.hsa_prefill(plain(Q), nan_tailed(Kx), nan_tailed(V), S, K,
                                  return_selection=True)
    torch.cuda.synchronize()
    out, sel = host(out), host(sel)
    assert np.isfinite(out).all(), "non-finite prefill output"
    ref = oracle.hsa_prefill(Q, Kx, V, S, K)
    same, _ = compare_selection(sel, ref["sel"], ref["margin"], "prefill selection")
    rows = np.repeat(same, Hq // Hkv, axis=1)
    check_out(out[rows], ref["out"][rows], "bf16", "prefill output")
    q = Q[:, :, L - 1].copy()
    lmk = oracle.landmarks(Kx, S).astype(np.float32)
    o = hsa.hsa_decode(plain(q), nan_tailed(Kx), nan_tailed(V), torch.from_numpy(lmk).cuda(), L,
                       S, K)
    torch.cuda.synchronize()
    o = host(o)
    assert np.isfinite(o).all(), "non-finite decode output"
    r = oracle.hsa_decode(q, Kx, V, lmk, S, L, K)
    if (r["margin"] > MARGIN).all():
        check_out(o, r["out"], "bf16", "decode output")
