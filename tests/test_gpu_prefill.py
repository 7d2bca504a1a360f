"""HSA prefill on the GPU against the CPU oracle: the tiny fp32 workload,
the 32K-token GQA bf16 workload, a shape sweep with ragged tails, edge cases,
landmarks and run-to-run determinism."""
import numpy as np
import pytest
import torch

import chunk_hierarchical_sparse_amd as hsa
import oracle
import synth
from gpu_util import (by_chunk, compare_selection, check_out, dev, gen, host, qkv, say)

pytestmark = pytest.mark.gpu


def run_case(B, Hq, Hkv, L, d, S, topk, dt, seed, scale=1.0, rows=None):
    say(f"prefill case B={B} Hq={Hq} Hkv={Hkv} L={L} d={d} S={S} K={topk} {dt} seed={seed}")
    Q, K, V = qkv(B, Hq, Hkv, L, d, dt, seed, scale)
    out, sel, w = hsa.hsa_prefill(dev(Q), dev(K), dev(V), S, topk, return_selection=True)
    torch.cuda.synchronize()
    out, sel, w = host(out), host(sel), host(w)
    ref = oracle.hsa_prefill(Q, K, V, S, topk, rows=rows)
    r = slice(None) if rows is None else np.asarray(rows)
    sel_g = sel[:, :, r]
    same, exempt = compare_selection(sel_g, ref["sel"], ref["margin"], "prefill selection",
                                     ref["sel_score"])
    G = Hq // Hkv
    same_h = np.repeat(same, G, axis=1)  # [B,Hq,R]
    err = check_out(out[:, :, r][same_h], ref["out"][same_h], dt, "prefill output")
    wg, wr = by_chunk(sel_g, w[:, :, r], G), by_chunk(ref["sel"], ref["w"], G)
    werr = float(np.abs(wg[same_h] - wr[same_h]).max()) if same_h.any() else 0.0
    assert werr <= 1e-5, f"fusion weights differ by {werr}"
    # padding convention: -1 indices, zero weights
    n = L // S
    for t in (0, min(L - 1, S), L - 1):
        m = min(topk, min(t // S, n))
        assert (sel[:, :, t, m:] == -1).all() and (sel[:, :, t, :m] >= 0).all()
        assert (w[:, :, t, m:] == 0).all()
    say(f"  ok: max err {err:.3g}, weight err {werr:.2g}, exempt {exempt:.4f}")
    return out, sel


def test_tiny_fp32_workload():
    # B=1, H=1, L=1024, d=64, S=64 (16 chunks), K=4, fp32, N(0,1), seed 1
    run_case(1, 1, 1, 1024, 64, 64, 4, "f32", seed=1)


def test_gqa_32k_bf16_workload():
    # B=1, L=32768, 16 query heads over 4 KV heads, d=128, S=64, K=8,
    # 0.5*N(0,1), seed 2.  Selection, fusion weights and outputs on every row.
    B, Hq, Hkv, L, d, S, topk = 1, 16, 4, 32768, 128, 64, 8
    say("prefill 32K workload")
    Q, K, V = qkv(B, Hq, Hkv, L, d, "bf16", 2, 0.5)
    out, sel, w = hsa.hsa_prefill(dev(Q), dev(K), dev(V), S, topk, return_selection=True)
    torch.cuda.synchronize()
    out, sel, w = host(out), host(sel), host(w)
    ref = oracle.hsa_prefill(Q, K, V, S, topk)
    same, exempt = compare_selection(sel, ref["sel"], ref["margin"], "32K selection",
                                     ref["sel_score"], max_exempt=0.01)
    say(f"  selection ok on all rows, exempt fraction {exempt:.4f}")
    same_h = np.repeat(same, Hq // Hkv, axis=1)
    err = check_out(out[same_h], ref["out"][same_h], "bf16", "32K output")
    werr = float(np.abs(by_chunk(sel, w, Hq // Hkv) - by_chunk(ref["sel"], ref["w"], Hq // Hkv))
                 [same_h].max())
    assert werr <= 1e-5, f"32K fusion weights: max error {werr}"
    say(f"  output ok on all {int(same_h.sum())} (row, head) pairs with equal sets, "
        f"max err {err:.3g}, weight err {werr:.2g}")


SWEEP = [
    # B, Hq, Hkv, L, d, S, topk, dtype
    (2, 4, 2, 700, 128, 64, 8, "bf16"),
    (1, 8, 2, 1000, 64, 16, 4, "bf16"),
    (1, 2, 2, 333, 64, 1, 16, "bf16"),
    (1, 4, 1, 900, 128, 100, 3, "bf16"),
    (2, 2, 1, 515, 64, 64, 1, "f32"),
    (1, 4, 4, 640, 128, 16, 32, "f32"),
    (1, 6, 3, 1300, 128, 128, 5, "bf16"),
    (1, 32, 1, 256, 64, 32, 2, "bf16"),
    (1, 2, 1, 9000, 64, 1, 4, "bf16"),  # 9000 chunks: past the LDS histograms of the invert
]


@pytest.mark.parametrize("case", SWEEP, ids=[str(i) for i in range(len(SWEEP))])
def test_shape_sweep(case):
    B, Hq, Hkv, L, d, S, topk, dt = case
    run_case(B, Hq, Hkv, L, d, S, topk, dt, seed=10 + SWEEP.index(case))


def test_short_sequences_output_zero():
    # L < S: no chunk at all; L = S: every query sees nothing (chunk 0 holds t)
    for L in (5, 64):
        Q, K, V = qkv(1, 2, 1, L, 64, "bf16", 30)
        out, sel, w = hsa.hsa_prefill(dev(Q), dev(K), dev(V), 64, 4, return_selection=True)
        torch.cuda.synchronize()
        assert not host(out).any() and (host(sel) == -1).all() and not host(w).any()


def test_landmarks_match_oracle():
    for dt, d, S, L in (("bf16", 128, 64, 4096 + 17), ("f32", 64, 64, 1024), ("bf16", 64, 7, 300)):
        say(f"landmarks {dt} d={d} S={S} L={L}")
        K = gen((2, 3, L, d), dt, 40, synth.TID_K)
        lm = host(hsa.hsa_build_landmarks(dev(K), S))
        ref = oracle.landmarks(K, S)
        np.testing.assert_allclose(lm, ref, rtol=2e-6, atol=2e-6)
    # chunk-range update leaves other chunks alone
    K = gen((1, 2, 640, 128), "bf16", 41, synth.TID_K)
    lm = torch.full((1, 2, 10, 128), 7.0, device="cuda")
    hsa.hsa_build_landmarks(dev(K), 64, chunk_begin=3, chunk_end=6, lmk=lm)
    lm = host(lm)
    ref = oracle.landmarks(K, 64)
    np.testing.assert_allclose(lm[:, :, 3:6], ref[:, :, 3:6], rtol=2e-6, atol=2e-6)
    assert (lm[:, :, :3] == 7).all() and (lm[:, :, 6:] == 7).all()


def test_precomputed_landmarks_give_the_same_result():
    Q, K, V = qkv(1, 4, 2, 1024, 128, "bf16", 50, 0.5)
    q, k, v = dev(Q), dev(K), dev(V)
    a = hsa.hsa_prefill(q, k, v, 64, 8)
    lm = hsa.hsa_build_landmarks(k, 64)
    b = hsa.hsa_prefill(q, k, v, 64, 8, lmk=lm)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_bitwise_determinism():
    Q, K, V = qkv(1, 16, 4, 8192, 128, "bf16", 60, 0.5)
    q, k, v = dev(Q), dev(K), dev(V)
    r1 = hsa.hsa_prefill(q, k, v, 64, 8, return_selection=True)
    r2 = hsa.hsa_prefill(q, k, v, 64, 8, return_selection=True)
    torch.cuda.synchronize()
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)
