"""The tie rule on the GPU: equal selection scores rank the lower chunk
index first (and, for DHSA, the boundary chunk keeps its lowest tokens).

Inputs are small integers, chunk sizes are 16 or 64 (sqrt of a power of
two) and the current DHSA decode chunk holds 1, 4 or 16 tokens, so every
landmark, pooled vector and selection score is exact in fp32 on the GPU and
in double in the oracle: equal scores are exactly equal on both sides and
distinct ones keep their order.  Duplicate chunks are planted (a copied
chunk has the same landmark or pooled key as its original), many of them
near the K-th place, so exact ties fall across the cut on many rows.  With
exact scores no row is exempt: selections (in rank order), DHSA kept sets
and chunk rankings must equal the oracle's on every row, and each case
checks that it really contains rows whose K-th/(K+1)-th margin is zero."""
import numpy as np
import pytest
import torch

import chunk_hierarchical_sparse_amd as hsa
import oracle
import synth
from gpu_util import by_chunk, check_out, dev, host, say, unpack_mask

pytestmark = pytest.mark.gpu


def bf16(x):
    return synth.f32_to_bf16(np.asarray(x, np.float32))


def hsa_inputs(B, Hq, Hkv, L, d, S, topk, seed):
    """Integer Q (leaning on dim 0), K, V; per KV head a 'hot' chunk pattern
    copied into topk + 4 chunks, and n/4 chunks overwritten by copies of
    other chunks."""
    rng = np.random.default_rng(seed)
    Q = rng.integers(-1, 2, (B, Hq, L, d)).astype(np.float32)
    Q[..., 0] += 2
    K = rng.integers(-2, 3, (B, Hkv, L, d)).astype(np.float32)
    V = rng.integers(-1, 2, (B, Hkv, L, d)).astype(np.float32)
    n = L // S
    for b in range(B):
        for g in range(Hkv):
            hot = rng.integers(-2, 3, (S, d)).astype(np.float32)
            hot[:, 0] = 2
            for c in rng.choice(n, min(n, topk + 4), replace=False):
                K[b, g, c * S:(c + 1) * S] = hot
            for _ in range(n // 4):
                c, c2 = rng.choice(n, 2, replace=False)
                K[b, g, c2 * S:(c2 + 1) * S] = K[b, g, c * S:(c + 1) * S]
    return bf16(Q), bf16(K), bf16(V)


PREFILL = [
    # B, Hq, Hkv, L, d, S, topk
    (1, 8, 2, 2048, 64, 16, 8),
    (1, 16, 4, 4096, 128, 64, 8),   # the 32K workload's heads, chunk size and K
    (2, 4, 4, 1500, 64, 64, 4),     # no grouping, ragged tail
    (1, 4, 1, 2000, 128, 16, 16),
]


@pytest.mark.parametrize("case", PREFILL, ids=[str(i) for i in range(len(PREFILL))])
def test_prefill_ties_exact_on_every_row(case):
    B, Hq, Hkv, L, d, S, topk = case
    seed = 500 + PREFILL.index(case)
    say(f"prefill ties B={B} Hq={Hq} Hkv={Hkv} L={L} d={d} S={S} K={topk}")
    Q, K, V = hsa_inputs(B, Hq, Hkv, L, d, S, topk, seed)
    out, sel, w = hsa.hsa_prefill(dev(Q), dev(K), dev(V), S, topk, return_selection=True)
    torch.cuda.synchronize()
    out, sel, w = host(out), host(sel), host(w)
    ref = oracle.hsa_prefill(Q, K, V, S, topk)
    ties = int((ref["margin"] == 0).sum())
    assert ties >= 50, f"only {ties} rows with a tie across the K-th place"
    bad = (sel != ref["sel"]).any(-1)
    assert not bad.any(), f"{int(bad.sum())} rows differ, first {np.argwhere(bad)[0].tolist()}: " \
                          f"gpu {sel[tuple(np.argwhere(bad)[0])]} " \
                          f"oracle {ref['sel'][tuple(np.argwhere(bad)[0])]}"
    err = check_out(out, ref["out"], "bf16", "prefill output")
    G = Hq // Hkv
    werr = float(np.abs(by_chunk(sel, w, G) - by_chunk(ref["sel"], ref["w"], G)).max())
    assert werr <= 1e-5, f"fusion weights differ by {werr}"
    say(f"  ok: every row exact, {ties} rows tied at the K-th place, max err {err:.3g}")

    if case == PREFILL[0]:
        # retrieval every 8 tokens on the same inputs: every block's selection
        R = 8
        o2, sel2, _ = hsa.hsa_prefill_interval(dev(Q), dev(K), dev(V), S, topk, R,
                                               return_selection=True)
        torch.cuda.synchronize()
        starts = np.arange(0, L, R)
        ref2 = oracle.hsa_prefill(Q, K, V, S, topk, rows=starts)
        assert int((ref2["margin"] == 0).sum()) >= 10
        assert np.array_equal(host(sel2), ref2["sel"]), "interval block selections differ"
        ref3 = oracle.hsa_prefill(Q, K, V, S, topk, retrieval_interval=R)
        err = check_out(host(o2), ref3["out"], "bf16", "interval output")
        say(f"  interval R={R}: every block exact, max err {err:.3g}")


def test_decode_ties_exact():
    # caches with planted duplicate chunks; the query leans on the hot pattern
    B, Hq, Hkv, N, d, S, topk = 8, 16, 4, 8192, 128, 64, 8
    Q, K, V = hsa_inputs(B, Hq, Hkv, N, d, S, topk, 520)
    lmk = oracle.landmarks(K, S).astype(np.float32)
    kd, vd, ld = dev(K), dev(V), dev(lmk)
    ties = 0
    for n_ctx in (N, N - 37, 70 * S):
        q = np.ascontiguousarray(Q[:, :, n_ctx - 1])
        o, sel, w = hsa.hsa_decode(dev(q), kd, vd, ld, n_ctx, S, topk, return_selection=True)
        torch.cuda.synchronize()
        ref = oracle.hsa_decode(q, K, V, lmk, S, n_ctx, topk)
        ties += int((ref["margin"] == 0).sum())
        assert np.array_equal(host(sel), ref["sel"]), f"decode selection differs at {n_ctx}"
        check_out(host(o), ref["out"], "bf16", "decode output")
        assert np.abs(host(w) - ref["w"]).max() <= 1e-5
    assert ties >= 8, f"only {ties} (b, group) rows tied at the K-th place"
    say(f"  decode ok, {ties} rows tied at the K-th place")


@pytest.mark.parametrize("n_top", [40, 300])
def test_decode_merge_ties_across_slices(n_top):
    # unit chunks, top-32 over 32768 candidates: n_top chunks spread over
    # the slices share the highest score exactly, so the slices' lists and
    # the merge (sorted path at 40, candidate cut and radix select at 300)
    # must keep the lowest indices
    B, Hq, Hkv, N, d, S, topk = 1, 2, 1, 32768, 64, 1, 32
    rng = np.random.default_rng(530 + n_top)
    q = np.zeros((B, Hq, d), np.float32)
    q[0, :, 0] = 1.0
    lmk = np.zeros((B, Hkv, N, d), np.float32)
    lmk[0, 0, :, 0] = rng.integers(0, 64, N).astype(np.float32) / 8.0
    top = np.sort(rng.choice(N, n_top, replace=False))
    lmk[0, 0, top, 0] = 9.0
    Kc = bf16(rng.integers(-2, 3, (B, Hkv, N, d)))
    Vc = bf16(rng.integers(-1, 2, (B, Hkv, N, d)))
    o, sel, w = hsa.hsa_decode(dev(bf16(q)), dev(Kc), dev(Vc), dev(lmk), N, S, topk,
                               return_selection=True)
    torch.cuda.synchronize()
    ref = oracle.hsa_decode(bf16(q), Kc, Vc, lmk, S, N, topk)
    assert np.array_equal(ref["sel"][0, 0], top[:topk])  # the oracle keeps the lowest
    assert np.array_equal(host(sel), ref["sel"]), "merge broke a tie the wrong way"
    check_out(host(o), ref["out"], "bf16", "decode output (tied candidates)")


def dhsa_inputs(B, H, n_chunks, d, seed):
    """Integer Q, K, V; chunk lengths 16 or 64; a third of the chunks get
    the keys of an earlier chunk of the same length."""
    rng = np.random.default_rng(seed)
    lens = rng.choice([16, 64], n_chunks)
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    L = int(offs[-1])
    Q = rng.integers(-1, 2, (B, H, L, d)).astype(np.float32)
    K = rng.integers(-1, 2, (B, H, L, d)).astype(np.float32)
    V = rng.integers(-1, 2, (B, H, L, d)).astype(np.float32)
    for b in range(B):
        for h in range(H):
            for _ in range(n_chunks // 3):
                c2 = int(rng.integers(1, n_chunks))
                same = np.flatnonzero(lens[:c2] == lens[c2])
                if same.size:
                    c = int(rng.choice(same))
                    K[b, h, offs[c2]:offs[c2 + 1]] = K[b, h, offs[c]:offs[c + 1]]
    return bf16(Q), bf16(K), bf16(V), offs


@pytest.mark.parametrize("d,budget", [(64, 256), (128, 700)])
def test_dhsa_prefill_ties_exact_on_every_row(d, budget):
    B, H = 1, 3
    Q, K, V, offs = dhsa_inputs(B, H, 60, d, 540 + d)
    L = int(offs[-1])
    say(f"dhsa ties L={L} chunks={len(offs) - 1} d={d} budget={budget}")
    out, mask, order = hsa.dhsa_prefill(dev(Q), dev(K), dev(V), offs, budget, return_mask=True,
                                        return_order=True)
    torch.cuda.synchronize()
    out, mask, order = host(out), host(mask), host(order)
    ref = oracle.dhsa_prefill(Q, K, V, offs, budget, want_kept=True, want_sc=True)
    ties = int((ref["margin"] == 0).sum())
    assert ties >= 100, f"only {ties} rows with a tie at the cut"
    bits = unpack_mask(mask, L)
    bad = (bits != ref["kept"]).any(-1)
    assert not bad.any(), f"{int(bad.sum())} kept sets differ, first {np.argwhere(bad)[0].tolist()}"
    nc = len(offs) - 1
    for h in range(H):
        for l in range(nc):
            row = ref["sc"][0, h, l, : l + 1]
            assert np.array_equal(order[0, h, l, : l + 1],
                                  np.lexsort((np.arange(l + 1), -row))), (h, l)
    err = check_out(out, ref["out"], "bf16", "dhsa output")
    say(f"  ok: every row exact, {ties} rows tied at the cut, max err {err:.3g}")


@pytest.mark.parametrize("m", [1, 4, 16])
def test_dhsa_decode_ties_exact(m):
    B, H, d, budget = 4, 2, 128, 400
    Q, K, V, offs_all = dhsa_inputs(B, H, 50, d, 550 + m)
    n = len(offs_all) - 2
    offs = offs_all[: n + 1]
    pos = int(offs[-1]) + m - 1
    if m == 16:
        # the current chunk repeats an earlier 16-token chunk's keys: it ties
        # with that chunk and ranks after it
        lens = np.diff(offs)
        c = int(np.flatnonzero(lens == 16)[0])
        K[:, :, offs[-1]:pos + 1] = K[:, :, offs[c]:offs[c + 1]]
    qcur = np.ascontiguousarray(Q[:, :, offs[-1]:pos + 1])
    kd, vd = dev(K), dev(V)
    khat = hsa.dhsa_build_chunk_keys(kd, offs)
    o, order = hsa.dhsa_decode(dev(qcur), kd, vd, khat, offs, budget, return_order=True)
    torch.cuda.synchronize()
    ref = oracle.dhsa_decode(qcur, K, V, offs, budget, want_kept=True)
    sc = ref["sc"]
    for b in range(B):
        for h in range(H):
            assert np.array_equal(host(order)[b, h],
                                  np.lexsort((np.arange(n + 1), -sc[b, h]))), (b, h)
    check_out(host(o), ref["out"], "bf16", "dhsa decode output")
    say(f"  dhsa decode m={m} ok, {int((ref['margin'] == 0).sum())} of {B * H} rows tied at "
        f"the cut")
