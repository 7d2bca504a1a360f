"""HSA prefill backward on the GPU against the CPU oracle.

The top-K selection is held fixed by the backward, so a row whose oracle
selection margin is below 1e-4 (a near tie the GPU's fp32 scores may break
the other way) is taken out of the comparison by zeroing its output
gradient: both sides then see the gradient of the same sum without that
row's terms.  At the full 32K size the output gradient is kept on 2,048
sampled rows, so the oracle computes exactly those rows' terms and every
element of dQ, dK and dV is compared.

Bar: max |gpu - oracle| <= 2e-2 * max |oracle| and a relative Frobenius error
<= 1e-2 (bf16 operands and outputs, fp32 accumulation)."""
import numpy as np
import pytest
import torch

import chunk_hierarchical_sparse_amd as hsa
import oracle
import synth
from gpu_util import MARGIN, check_exempt, dev, gen, host, qkv, say

pytestmark = pytest.mark.gpu

TOL_MAX = 2e-2
TOL_FRO = 1e-2


def compare(got, ref, what):
    scale = max(float(np.abs(ref).max()), 1e-6)
    err = float(np.abs(got.astype(np.float64) - ref).max())
    fro = float(np.linalg.norm(got.astype(np.float64) - ref) / max(np.linalg.norm(ref), 1e-12))
    assert err <= TOL_MAX * scale, f"{what}: max error {err} > {TOL_MAX} * {scale}"
    assert fro <= TOL_FRO, f"{what}: relative Frobenius error {fro}"
    return err / scale, fro


def run_case(B, Hq, Hkv, L, d, S, topk, seed, scale=1.0, rows=None):
    say(f"backward B={B} Hq={Hq} Hkv={Hkv} L={L} d={d} S={S} K={topk}"
        + ("" if rows is None else f" rows={len(rows)}"))
    Q, K, V = qkv(B, Hq, Hkv, L, d, "bf16", seed, scale)
    dO = gen((B, Hq, L, d), "bf16", seed, synth.TID_DO)
    keep = np.arange(L) if rows is None else np.asarray(rows)
    sel = oracle.hsa_prefill(Q, K, V, S, topk, rows=keep, want_out=False)
    G = Hq // Hkv
    live = np.zeros((B, Hq, L), bool)
    live[:, :, keep] = np.repeat(sel["margin"] > MARGIN, G, axis=1)
    check_exempt(sel["margin"] > MARGIN, "backward rows")
    dO[~live] = 0
    say(f"  rows kept {live.mean():.4f} of all (near ties dropped: "
        f"{1 - (sel['margin'] > MARGIN).mean():.4f})")
    dq, dk, dv = hsa.hsa_prefill_backward(dev(Q), dev(K), dev(V), dev(dO), S, topk)
    torch.cuda.synchronize()
    ref = oracle.hsa_prefill_backward(Q, K, V, dO, S, topk, rows=keep)
    res = [compare(host(x), ref[k], k) for x, k in ((dq, "dQ"), (dk, "dK"), (dv, "dV"))]
    say("  ok: " + ", ".join(f"{k} max {m:.3g} fro {f:.3g}" for k, (m, f) in zip("QKV", res)))
    return dq, dk, dv


SWEEP = [
    # B, Hq, Hkv, L, d, S, topk
    (1, 8, 2, 1000, 128, 64, 8),
    (2, 4, 4, 777, 64, 32, 4),     # no grouping, S = 32, ragged tail
    (1, 12, 4, 600, 128, 16, 8),   # groups of 3 heads, small chunks
    (1, 4, 1, 400, 128, 64, 32),   # top-K past the available chunks
    (1, 4, 2, 200, 64, 1, 8),      # unit chunks
    (1, 2, 2, 300, 128, 48, 3),    # a chunk size that is not a power of two
    (1, 2, 1, 4096, 64, 1, 4),     # 4096 unit chunks: the largest count with token-ordered lists
    (1, 2, 1, 4400, 64, 1, 4),     # 4400 chunks: lists in atomic order
]


@pytest.mark.parametrize("case", SWEEP, ids=[str(i) for i in range(len(SWEEP))])
def test_backward_sweep(case):
    run_case(*case, seed=300 + SWEEP.index(case))


def test_backward_32k_workload_sampled_rows():
    # the 32K GQA bf16 prefill: output gradient kept on 2,048+ sampled rows
    # (early, late, chunk edges), every element of dQ, dK, dV compared
    rng = np.random.default_rng(13)
    rows = np.unique(np.concatenate([rng.choice(np.arange(64, 32768), 2048, replace=False),
                                     [64, 127, 128, 4095, 32767]]))
    run_case(1, 16, 4, 32768, 128, 64, 8, seed=2, scale=0.5, rows=rows)


def test_backward_short_sequence_has_zero_gradients():
    # fewer than S tokens: no chunk is ever available, the output is zero
    Q, K, V = qkv(1, 4, 2, 50, 128, "bf16", 310)
    dO = gen((1, 4, 50, 128), "bf16", 310, synth.TID_DO)
    dq, dk, dv = hsa.hsa_prefill_backward(dev(Q), dev(K), dev(V), dev(dO), 64, 8)
    torch.cuda.synchronize()
    for x in (dq, dk, dv):
        assert float(x.float().abs().max()) == 0.0
