"""HSA decode on the GPU against the CPU oracle (small and mid-size caches).
The 131072-token batch-32 and 16M-token workloads live in
test_gpu_decode_large.py."""
import numpy as np
import pytest
import torch

import chunk_hierarchical_sparse_amd as hsa
import oracle
import synth
from gpu_util import by_chunk, compare_selection, check_out, dev, gen, host, say

pytestmark = pytest.mark.gpu


def run_case(B, Hq, Hkv, n_max, n_ctx, d, S, topk, dt, seed):
    say(f"decode case B={B} Hq={Hq} Hkv={Hkv} n_max={n_max} n_ctx={n_ctx} d={d} S={S} "
        f"K={topk} {dt}")
    q = gen((B, Hq, d), dt, seed, synth.TID_QDEC)
    Kc = gen((B, Hkv, n_max, d), dt, seed, synth.TID_K)
    Vc = gen((B, Hkv, n_max, d), dt, seed, synth.TID_V)
    lmk = oracle.landmarks(Kc, S).astype(np.float32)
    o, sel, w = hsa.hsa_decode(dev(q), dev(Kc), dev(Vc), dev(lmk), n_ctx, S, topk,
                               return_selection=True)
    torch.cuda.synchronize()
    o, sel, w = host(o), host(sel), host(w)
    ref = oracle.hsa_decode(q, Kc, Vc, lmk, S, n_ctx, topk)
    same, exempt = compare_selection(sel, ref["sel"], ref["margin"], "decode selection",
                                     ref["sel_score"])
    G = Hq // Hkv
    same_h = np.repeat(same, G, axis=1)
    err = check_out(o[same_h], ref["out"][same_h], dt, "decode output")
    wg, wr = by_chunk(sel, w, G), by_chunk(ref["sel"], ref["w"], G)
    werr = float(np.abs(wg[same_h] - wr[same_h]).max()) if same_h.any() else 0.0
    assert werr <= 1e-5
    say(f"  ok: max err {err:.3g}, exempt {exempt:.3f}")


CASES = [
    (2, 8, 2, 4096, 4000, 128, 64, 8, "bf16"),
    (3, 4, 4, 2048, 2048, 64, 64, 4, "f32"),
    (1, 16, 4, 65536, 65536, 128, 64, 16, "bf16"),
    (2, 4, 1, 1000, 999, 128, 16, 32, "bf16"),
    (1, 2, 2, 300, 300, 64, 1, 8, "f32"),
    (1, 8, 1, 5000, 4500, 128, 200, 3, "bf16"),
    # chunks of <= 64 keys take one wave per chunk; these cover fp32 rows of
    # 128, groups of 16 heads handled in rounds of 8 and of 4, R = 2 blocks
    # per group, and groups of 3 heads with d = 64 in bf16
    (2, 16, 1, 3000, 2900, 128, 64, 8, "f32"),
    (1, 32, 2, 2048, 2047, 128, 32, 16, "bf16"),
    (2, 6, 2, 1500, 1400, 64, 64, 8, "bf16"),
    # batches of 16 to 20 (b, group) pairs, fp32, d = 64, S = 16 and S = 128
    (3, 12, 6, 2048, 2000, 64, 64, 8, "bf16"),
    (4, 8, 4, 3000, 2950, 128, 64, 8, "f32"),
    (5, 16, 4, 1024, 1000, 128, 16, 4, "bf16"),
    (4, 4, 4, 4096, 4000, 128, 128, 4, "bf16"),
]


@pytest.mark.parametrize("case", CASES, ids=[str(i) for i in range(len(CASES))])
def test_decode_cases(case):
    run_case(*case, seed=70 + CASES.index(case))


def test_decode_without_chunks_outputs_zero():
    q = gen((2, 4, 128), "bf16", 80, synth.TID_QDEC)
    Kc = gen((2, 2, 64, 128), "bf16", 80, synth.TID_K)
    lmk = torch.zeros((2, 2, 1, 128), device="cuda")
    o, sel, w = hsa.hsa_decode(dev(q), dev(Kc), dev(Kc), lmk, 63, 64, 4, return_selection=True)
    torch.cuda.synchronize()
    assert not host(o).any() and (host(sel) == -1).all() and not host(w).any()


def test_decode_equals_prefill_last_row():
    # a decode query at position L equals prefill row L of the same tokens
    B, Hq, Hkv, L, d, S, topk = 1, 8, 2, 2048, 128, 64, 8
    Q = gen((B, Hq, L + 1, d), "bf16", 81, synth.TID_Q)
    K = gen((B, Hkv, L + 1, d), "bf16", 81, synth.TID_K)
    V = gen((B, Hkv, L + 1, d), "bf16", 81, synth.TID_V)
    pre = hsa.hsa_prefill(dev(Q), dev(K), dev(V), S, topk)
    kc, vc = dev(K[:, :, :L]), dev(V[:, :, :L])
    lm = hsa.hsa_build_landmarks(kc, S)
    dec = hsa.hsa_decode(dev(np.ascontiguousarray(Q[:, :, L])), kc, vc, lm, L, S, topk)
    torch.cuda.synchronize()
    diff = (host(pre)[:, :, L] - host(dec))
    assert np.abs(diff).max() <= 1e-2


def test_decode_merge_with_many_candidates_above_the_bound():
    # One KV head, S = 1, top-32 over 32768 chunks: 128 slices of 256 chunks
    # feed the merge.  Landmarks are given directly so that the scores are
    # set per chunk: each slice's first 32 chunks take distinct values
    # 10 + u/64 (u a permutation of 0..4095), the rest lie below 1.  The
    # slices' top-32 lists then interleave, more than 64 candidates reach
    # the merge's lower bound and the radix-select path runs.
    B, Hq, Hkv, N, d, S, topk = 1, 1, 1, 32768, 64, 1, 32
    rng = np.random.default_rng(91)
    q = np.zeros((B, Hq, d), np.uint16)
    q[0, 0, 0] = synth.f32_to_bf16(np.float32(1.0))
    score = rng.uniform(0.0, 1.0, N)
    perm = rng.permutation(128 * 32)
    for j in range(128):
        for r in range(32):
            score[j * 256 + r] = 10.0 + perm[j * 32 + r] / 64.0
    lmk = np.zeros((B, Hkv, N, d), np.float32)
    lmk[0, 0, :, 0] = (score * np.sqrt(d)).astype(np.float32)
    Kc = gen((B, Hkv, N, d), "bf16", 91, synth.TID_K)
    Vc = gen((B, Hkv, N, d), "bf16", 91, synth.TID_V)
    o, sel, w = hsa.hsa_decode(dev(q), dev(Kc), dev(Vc), dev(lmk), N, S, topk,
                               return_selection=True)
    torch.cuda.synchronize()
    o, sel, w = host(o), host(sel), host(w)
    ref = oracle.hsa_decode(q, Kc, Vc, lmk, S, N, topk)
    assert ref["margin"].min() > 1e-4
    assert np.array_equal(sel, ref["sel"])
    check_out(o, ref["out"], "bf16", "decode output (many candidates)")
    assert np.abs(w - ref["w"]).max() <= 1e-5
