"""HSA prefill with retrieval every R tokens on the GPU against the CPU
oracle: one selection per block of R tokens (made at the block's first
token), per-token attention and fusion."""
import numpy as np
import pytest
import torch

import chunk_hierarchical_sparse_amd as hsa
import oracle
import synth
from gpu_util import by_chunk, check_out, compare_selection, dev, host, qkv, say

pytestmark = pytest.mark.gpu


def run_case(B, Hq, Hkv, L, d, S, topk, R, dt, seed, scale=1.0, rows=None):
    say(f"interval case B={B} Hq={Hq} Hkv={Hkv} L={L} d={d} S={S} K={topk} R={R} {dt}")
    Q, K, V = qkv(B, Hq, Hkv, L, d, dt, seed, scale)
    out, sel, w = hsa.hsa_prefill_interval(dev(Q), dev(K), dev(V), S, topk, R,
                                           return_selection=True)
    torch.cuda.synchronize()
    out, sel, w = host(out), host(sel), host(w)
    G = Hq // Hkv
    # every block's selection against the oracle at the block starts
    starts = np.arange(0, L, R)
    ref_s = oracle.hsa_prefill(Q, K, V, S, topk, rows=starts, want_out=False)
    same_b, exempt = compare_selection(sel, ref_s["sel"], ref_s["margin"], "block selection",
                                       ref_s["sel_score"])
    # outputs and weights on rows whose block selection matched
    rows = np.arange(L) if rows is None else np.asarray(rows)
    ref = oracle.hsa_prefill(Q, K, V, S, topk, rows=rows, retrieval_interval=R)
    ok = same_b[:, :, rows // R]                       # [B, Hkv, rows]
    ok_h = np.repeat(ok, G, axis=1)
    err = check_out(out[:, :, rows][ok_h], ref["out"][ok_h], dt, "interval output")
    sel_rows = sel[:, :, rows // R]
    wg, wr = by_chunk(sel_rows, w[:, :, rows], G), by_chunk(ref["sel"], ref["w"], G)
    werr = float(np.abs(wg[ok_h] - wr[ok_h]).max()) if ok_h.any() else 0.0
    assert werr <= 1e-5, werr
    say(f"  ok: max err {err:.3g}, weight err {werr:.2g}, exempt {exempt:.3f}")


SWEEP = [
    (1, 8, 2, 1500, 128, 64, 8, 8, "bf16"),
    (2, 4, 4, 777, 64, 16, 4, 3, "f32"),
    (1, 4, 1, 600, 128, 32, 32, 64, "bf16"),
    (1, 2, 2, 300, 64, 1, 8, 5, "f32"),      # S = 1: token-level chunks
    (1, 12, 4, 1000, 128, 100, 3, 7, "bf16"),  # S > 64, G = 3
    (1, 4, 2, 520, 128, 64, 8, 600, "bf16"),  # one block spans the sequence
    # R * G = 32 in bf16 with K <= 8 and S <= 64 runs query-major (one wave
    # per block of R tokens, fused in registers): G = 2, 8 and 1, d = 64,
    # S = 32 (one key sub-tile), 16 and 48 (a partial second sub-tile), a
    # partial last block (1000 and 900 tokens), K = 4 and 6; K = 12 with
    # R * G = 32 takes the chunk-major path
    (2, 8, 4, 1000, 64, 32, 4, 16, "bf16"),
    (1, 32, 4, 900, 128, 16, 8, 4, "bf16"),
    (1, 16, 16, 700, 128, 64, 6, 32, "bf16"),
    (1, 8, 2, 1500, 128, 48, 8, 8, "bf16"),
    (1, 8, 2, 800, 128, 32, 12, 8, "bf16"),
    (1, 8, 2, 600, 128, 1, 8, 8, "bf16"),     # query-major with S = 1 (token chunks)
]


@pytest.mark.parametrize("case", SWEEP, ids=[str(i) for i in range(len(SWEEP))])
def test_interval_sweep(case):
    run_case(*case, seed=100 + SWEEP.index(case))


def test_interval_32k_workload():
    # the 32K GQA bf16 prefill with retrieval every 8 tokens (the query-major
    # path): every block's selection, every row's output and weights
    run_case(1, 16, 4, 32768, 128, 64, 8, 8, "bf16", seed=2, scale=0.5)


def test_interval_one_is_per_token_prefill():
    Q, K, V = qkv(1, 8, 2, 2000, 128, "bf16", 109, 0.5)
    q, k, v = dev(Q), dev(K), dev(V)
    a = hsa.hsa_prefill(q, k, v, 64, 8)
    b = hsa.hsa_prefill_interval(q, k, v, 64, 8, 1)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
