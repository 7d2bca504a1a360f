"""HSA decode at full size against the CPU oracle.

 - batch 32, 131072-token caches, 32 query heads over 8 KV heads, top-8;
 - batch 1, 16,777,216-token caches (32 GiB of bf16 K/V), 16 over 4 heads,
   top-16, with a planted needle chunk that must rank first in every group.

The caches are filled on the GPU by the seeded generator; the host
regenerates the same values slab by slab (checked bit-exact on samples) to
compute the oracle's landmarks (double, rounded to fp32), and only the
selected chunks for the oracle's attention.  The GPU decode receives the
oracle's landmarks, so selection and attention are compared on identical
inputs; the GPU landmark kernel is compared with the oracle on the same
slabs.
"""
import numpy as np
import pytest
import torch

import chunk_hierarchical_sparse_amd as hsa
import oracle
import synth
from gpu_util import by_chunk, check_out, compare_selection, dev, host, say

pytestmark = pytest.mark.gpu

SLAB = 1 << 20  # tokens regenerated on the host at a time


def oracle_landmarks_from_generator(B, Hkv, N, d, S, seed, needle=None):
    """fp32 landmarks [B,Hkv,N/S,d] of the generator's K, slab by slab.
    needle = (chunk, {group: key row bf16 bits}) replaces that chunk's keys."""
    n = N // S
    lmk = np.empty((B, Hkv, n, d), np.float32)
    for b in range(B):
        for g in range(Hkv):
            if N >= SLAB or g == 0:
                say(f"    landmarks b={b} g={g}")
            for t0 in range(0, N, SLAB):
                t1 = min(N, t0 + SLAB)
                first = ((b * Hkv + g) * N + t0) * d
                K = synth.normal(((t1 - t0), d), synth.BF16, seed, synth.TID_K, first=first)
                if needle is not None:
                    c, rows = needle
                    lo, hi = max(t0, c * S), min(t1, (c + 1) * S)
                    if lo < hi:
                        K[lo - t0:hi - t0] = rows[g]
                lmk[b, g, t0 // S:t1 // S] = oracle.landmarks(K[None, None], S)[0, 0].astype(
                    np.float32)
    return lmk


def selected_chunks(sel, B, Hkv, N, d, S, seed, tid, needle=None):
    """[B,Hkv,K,S,d] bf16 bits of the selected chunks, regenerated."""
    topk = sel.shape[2]
    out = np.zeros((B, Hkv, topk, S, d), np.uint16)
    for b in range(B):
        for g in range(Hkv):
            for k in range(topk):
                c = int(sel[b, g, k])
                if c < 0:
                    continue
                first = ((b * Hkv + g) * N + c * S) * d
                out[b, g, k] = synth.normal((S, d), synth.BF16, seed, tid, first=first)
                if needle is not None and tid == synth.TID_K and c == needle[0]:
                    out[b, g, k] = needle[1][g]
    return out


def run_large(B, Hq, Hkv, N, d, S, topk, seed, plant_needle):
    say(f"large decode B={B} Hq={Hq} Hkv={Hkv} N={N} K={topk}")
    Kc = torch.empty((B, Hkv, N, d), dtype=torch.bfloat16, device="cuda")
    Vc = torch.empty_like(Kc)
    synth.normal_device(Kc, seed, synth.TID_K)
    synth.normal_device(Vc, seed, synth.TID_V)
    torch.cuda.synchronize()
    # device generator == host generator (samples at the start, the middle and the end)
    for first in (0, Kc.numel() // 2 + 12345, Kc.numel() - 4096):
        ref = synth.normal((4096,), synth.BF16, seed, synth.TID_K, first=first)
        got = Kc.view(-1)[first:first + 4096].view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, ref), "device and host generators differ"
    q = synth.normal((B, Hq, d), synth.BF16, seed, synth.TID_QDEC)
    needle = None
    if plant_needle:
        cstar = synth.pick_index(N // S, seed)
        G = Hq // Hkv
        rows = {g: synth.needle_key(q[0, g * G:(g + 1) * G], True) for g in range(Hkv)}
        for g in range(Hkv):
            Kc[0, g, cstar * S:(cstar + 1) * S] = dev(np.broadcast_to(rows[g], (S, d)).copy())
        needle = (cstar, {g: np.broadcast_to(rows[g], (S, d)).copy() for g in range(Hkv)})
    say("  oracle landmarks (host)")
    lmk = oracle_landmarks_from_generator(B, Hkv, N, d, S, seed, needle)
    lmk_dev = dev(lmk)
    # the GPU landmark kernel against the oracle's
    say("  GPU landmarks")
    glmk = hsa.hsa_build_landmarks(Kc, S)
    torch.cuda.synchronize()
    g_h = host(glmk)
    np.testing.assert_allclose(g_h, lmk, rtol=2e-6, atol=2e-6)
    del glmk, g_h
    say("  GPU decode")
    o, sel, w = hsa.hsa_decode(dev(q), Kc, Vc, lmk_dev, N, S, topk, return_selection=True)
    torch.cuda.synchronize()
    o, sel, w = host(o), host(sel), host(w)
    sel_ref, margin, score_ref = oracle.hsa_decode_select(q, lmk, S, N, topk, Hkv)
    same, exempt = compare_selection(sel, sel_ref, margin, "large decode selection", score_ref)
    if plant_needle:
        assert (sel[0, :, 0] == needle[0]).all(), "needle not ranked first"
    say("  oracle attention on the selected chunks")
    Ks = selected_chunks(sel_ref, B, Hkv, N, d, S, seed, synth.TID_K, needle)
    Vs = selected_chunks(sel_ref, B, Hkv, N, d, S, seed, synth.TID_V)
    lsel = np.zeros((B, Hkv, topk, d), np.float32)
    for b in range(B):
        for g in range(Hkv):
            for k in range(topk):
                if sel_ref[b, g, k] >= 0:
                    lsel[b, g, k] = lmk[b, g, sel_ref[b, g, k]]
    out_ref, w_ref = oracle.hsa_decode_attend(q, Ks, Vs, lsel, sel_ref, S)
    G = Hq // Hkv
    same_h = np.repeat(same, G, axis=1)
    err = check_out(o[same_h], out_ref[same_h], "bf16", "large decode output")
    wg, wr = by_chunk(sel, w, G), by_chunk(sel_ref, w_ref, G)
    werr = float(np.abs(wg[same_h] - wr[same_h]).max()) if same_h.any() else 0.0
    assert werr <= 1e-5
    say(f"  ok: max err {err:.3g}, weight err {werr:.2g}, exempt {exempt:.3f}")
    del Kc, Vc, lmk_dev
    torch.cuda.empty_cache()


def test_decode_batch32_131k():
    run_large(32, 32, 8, 131072, 128, 64, 8, seed=3, plant_needle=False)


def test_decode_16m_tokens_with_needle():
    run_large(1, 16, 4, 16777216, 128, 64, 16, seed=4, plant_needle=True)
