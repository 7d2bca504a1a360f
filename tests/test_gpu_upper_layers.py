"""The upper layers' two attentions of one new query in one pass
(hsa_swa_decode): the HSA output against the oracle's HSA decode and bit for
bit against hsa_decode (the same kernels), the sliding-window output against
the oracle's sliding-window decode, across window sizes (one key, not a
multiple of the 64-key pieces, past the context), chunk sizes, top-K, group
sizes, head dims and both dtypes."""
import numpy as np
import pytest
import torch

import chunk_hierarchical_sparse_amd as hsa
import oracle
import synth
from gpu_util import MARGIN, check_exempt, check_out, dev, gen, host, say

pytestmark = pytest.mark.gpu


def run_case(B, Hq, Hkv, n_max, n_ctx, d, S, K, W, dt, seed):
    say(f"hsa+swa decode B={B} Hq={Hq} Hkv={Hkv} n_ctx={n_ctx} d={d} S={S} K={K} W={W} {dt}")
    q = gen((B, Hq, d), dt, seed, synth.TID_QDEC)
    Kc = gen((B, Hkv, n_max, d), dt, seed, synth.TID_K)
    Vc = gen((B, Hkv, n_max, d), dt, seed, synth.TID_V)
    n = n_ctx // S
    lmk = np.zeros((B, Hkv, n_max // S, d), np.float32)
    if n:
        lmk[:, :, :n] = oracle.landmarks(Kc[:, :, : n * S], S).astype(np.float32)
    qd, kd, vd, ld = dev(q), dev(Kc), dev(Vc), dev(lmk)
    oh, osw, sel, w = hsa.hsa_swa_decode(qd, kd, vd, ld, n_ctx, S, K, W, return_selection=True)
    ref_h, ref_sel, ref_w = hsa.hsa_decode(qd, kd, vd, ld, n_ctx, S, K, return_selection=True)
    torch.cuda.synchronize()
    # the HSA part runs hsa_decode's kernels: the same bits
    view = (lambda t: t.view(torch.int16)) if dt == "bf16" else (lambda t: t)
    assert torch.equal(view(oh), view(ref_h)) and torch.equal(sel, ref_sel)
    assert torch.equal(w, ref_w)
    r = oracle.hsa_decode(q, Kc, Vc, lmk, S, n_ctx, K)
    ok = r["margin"] > MARGIN
    check_exempt(ok, "hsa+swa decode rows")
    okh = np.repeat(ok, Hq // Hkv, axis=1)
    err_h = check_out(host(oh)[okh], r["out"][okh], dt, "hsa output")
    err_s = check_out(host(osw), oracle.swa_decode(q, Kc, Vc, n_ctx, W), dt, "swa output")
    say(f"  ok: hsa err {err_h:.3g}, swa err {err_s:.3g}")


CASES = [
    # B, Hq, Hkv, n_max, n_ctx, d, S, K, W, dtype
    (4, 32, 8, 9000, 8999 - 37, 128, 64, 8, 512, "bf16"),   # the upper-layer shapes
    (2, 16, 4, 5000, 4321, 128, 64, 16, 100, "bf16"),        # window not a multiple of 64
    (3, 8, 8, 3000, 2999, 64, 16, 4, 1, "bf16"),             # a window of one key
    (2, 8, 2, 700, 650, 128, 32, 8, 4096, "bf16"),           # window past the context
    (2, 4, 1, 300, 40, 128, 64, 4, 512, "bf16"),             # no complete chunk yet
    (2, 12, 4, 2000, 1900, 128, 64, 8, 700, "f32"),
    (1, 6, 2, 1500, 1234, 64, 16, 32, 333, "f32"),
]


@pytest.mark.parametrize("case", CASES, ids=[str(i) for i in range(len(CASES))])
def test_hsa_swa_decode(case):
    run_case(*case, seed=600 + CASES.index(case))


def test_hsa_swa_decode_rejects_what_it_cannot_run():
    q = torch.zeros((1, 4, 128), dtype=torch.bfloat16, device="cuda")
    Kc = torch.zeros((1, 2, 9000, 128), dtype=torch.bfloat16, device="cuda")
    lmk = torch.zeros((1, 2, 9000 // 128, 128), device="cuda")
    with pytest.raises(hsa.HsaError):  # chunks longer than 64 keys
        hsa.hsa_swa_decode(q, Kc, Kc, lmk, 8000, 128, 8, 512)
    lmk64 = torch.zeros((1, 2, 9000 // 64, 128), device="cuda")
    with pytest.raises(hsa.HsaError):  # a window above 4096 keys
        hsa.hsa_swa_decode(q, Kc, Kc, lmk64, 8000, 64, 8, 5000)
    with pytest.raises(hsa.HsaError):  # the new token must be in the cache
        hsa.hsa_swa_decode(q, Kc, Kc, lmk64, 9000, 64, 8, 512)


def run_prefill_case(B, Hq, Hkv, L, d, S, K, W, dt, seed, scale=1.0):
    say(f"hsa+swa prefill B={B} Hq={Hq} Hkv={Hkv} L={L} d={d} S={S} K={K} W={W} {dt}")
    Q, Kx, V = (gen((B, H, L, d), dt, seed, t, scale)
                for H, t in ((Hq, synth.TID_Q), (Hkv, synth.TID_K), (Hkv, synth.TID_V)))
    qd, kd, vd = dev(Q), dev(Kx), dev(V)
    oh, osw, sel, w = hsa.hsa_swa_prefill(qd, kd, vd, S, K, W, return_selection=True)
    ref_h, ref_sel, ref_w = hsa.hsa_prefill(qd, kd, vd, S, K, return_selection=True)
    ref_s = hsa.swa_prefill(qd, kd, vd, W)
    torch.cuda.synchronize()
    # the same kernels as the separate calls: the same bits
    view = (lambda t: t.view(torch.int16)) if dt == "bf16" else (lambda t: t)
    assert torch.equal(view(oh), view(ref_h)), "HSA output differs from hsa_prefill"
    assert torch.equal(view(osw), view(ref_s)), "window output differs from swa_prefill"
    assert torch.equal(sel, ref_sel) and torch.equal(w, ref_w)
    r = oracle.hsa_prefill(Q, Kx, V, S, K)
    ok = r["margin"] > MARGIN
    check_exempt(ok, "hsa+swa prefill rows")
    same = (np.sort(host(sel), -1) == np.sort(r["sel"], -1)).all(-1) | ~ok
    assert same.all(), "selection differs above the margin"
    okh = np.repeat(ok, Hq // Hkv, axis=1)
    err_h = check_out(host(oh)[okh], r["out"][okh], dt, "hsa output")
    err_s = check_out(host(osw), oracle.swa_prefill(Q, Kx, V, W), dt, "swa output")
    say(f"  ok: hsa err {err_h:.3g}, swa err {err_s:.3g}")


PREFILL_CASES = [
    # B, Hq, Hkv, L, d, S, K, W, dtype
    (1, 16, 4, 2000, 128, 64, 8, 512, "bf16"),  # the upper-layer shapes (one launch)
    (2, 8, 8, 777, 64, 32, 4, 100, "bf16"),     # 32-key chunks, no grouping
    (1, 6, 2, 513, 128, 16, 8, 33, "bf16"),     # groups of 3 heads: one head per window block
    (1, 4, 1, 300, 128, 64, 4, 1, "bf16"),      # a window of one key
    (1, 4, 2, 50, 128, 64, 4, 512, "bf16"),     # shorter than a chunk: window blocks only
    (1, 4, 2, 600, 128, 100, 4, 200, "bf16"),   # 100-key chunks: two launches
    (2, 4, 2, 400, 64, 64, 4, 64, "f32"),       # fp32: two launches
]


@pytest.mark.parametrize("case", PREFILL_CASES, ids=[str(i) for i in range(len(PREFILL_CASES))])
def test_hsa_swa_prefill(case):
    run_prefill_case(*case, seed=640 + PREFILL_CASES.index(case))


def test_hsa_swa_prefill_32k_workload_equals_separate_calls():
    # the 32K GQA bf16 sequence, 512-token window: bit for bit the separate calls
    B, Hq, Hkv, L, d, S, K, W = 1, 16, 4, 32768, 128, 64, 8, 512
    say("hsa+swa prefill 32K")
    Q, Kx, V = (gen((B, H, L, d), "bf16", 2, t, 0.5)
                for H, t in ((Hq, synth.TID_Q), (Hkv, synth.TID_K), (Hkv, synth.TID_V)))
    qd, kd, vd = dev(Q), dev(Kx), dev(V)
    oh, osw = hsa.hsa_swa_prefill(qd, kd, vd, S, K, W)
    ref_h = hsa.hsa_prefill(qd, kd, vd, S, K)
    ref_s = hsa.swa_prefill(qd, kd, vd, W)
    torch.cuda.synchronize()
    assert torch.equal(oh.view(torch.int16), ref_h.view(torch.int16))
    assert torch.equal(osw.view(torch.int16), ref_s.view(torch.int16))
