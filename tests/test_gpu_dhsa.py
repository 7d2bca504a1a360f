"""DHSA prefill on the GPU against the CPU oracle: the 16K-token workload
(sampled rows, plus the budget property on every row), shape sweeps and the
reductions (budget covering everything, unit chunks)."""
import numpy as np
import pytest
import torch

import chunk_hierarchical_sparse_amd as hsa
import oracle
import synth
from gpu_util import MARGIN, check_out, dev, host, qkv, say, unpack_mask

pytestmark = pytest.mark.gpu


def run_case(B, H, L, d, offs, budget, seed, rows=None, check_order=True):
    say(f"dhsa case B={B} H={H} L={L} d={d} chunks={len(offs) - 1} budget={budget} seed={seed}")
    Q, K, V = qkv(B, H, H, L, d, "bf16", seed)
    out, mask, order = hsa.dhsa_prefill(dev(Q), dev(K), dev(V), offs, budget, return_mask=True,
                                        return_order=True)
    torch.cuda.synchronize()
    out, mask, order = host(out), host(mask), host(order)
    ref = oracle.dhsa_prefill(Q, K, V, offs, budget, rows=rows, want_kept=True,
                              want_sc=check_order)
    r = np.arange(L) if rows is None else np.asarray(rows)
    bits = unpack_mask(mask[:, :, r], L)
    # every row keeps exactly min(N_b, i+1) keys, all causal
    counts = unpack_mask(mask, L).sum(-1)
    assert (counts == np.minimum(budget, np.arange(L) + 1)).all(), "kept count != min(N_b, i+1)"
    strict = ref["margin"] > MARGIN
    bad = (bits != ref["kept"]).any(-1) & strict
    assert not bad.any(), f"kept sets differ above the margin at {np.argwhere(bad)[0].tolist()}"
    same = (bits == ref["kept"]).all(-1)
    err = check_out(out[:, :, r][same], ref["out"][same], "bf16", "dhsa output")
    if check_order:
        nc = len(offs) - 1
        sc = ref["sc"]
        for b in range(B):
            for h in range(H):
                for l in range(nc):
                    row = sc[b, h, l, : l + 1]
                    exp = np.lexsort((np.arange(l + 1), -row))
                    gaps = np.abs(np.diff(row[exp]))
                    if gaps.size == 0 or gaps.min() > MARGIN:
                        assert (order[b, h, l, : l + 1] == exp).all()
                    assert (order[b, h, l, l + 1:] == -1).all()
    say(f"  ok: max err {err:.3g}, exempt {float((~strict).mean()):.4f}")


def test_dhsa_16k_workload():
    # B=1, L=16384, H=8, d=128, chunk lengths U{16..128} (seed 5), N_b=2048
    L = 16384
    offs = synth.chunk_offsets(L, 16, 128, seed=5)
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 1, 15, 16, 2046, 2047, 2048, 2049, L - 1],
                                     offs[:-1][:40], offs[1:-1][:40] - 1,
                                     rng.integers(0, L, 300)]))
    run_case(1, 8, L, 128, offs, 2048, seed=5, rows=rows, check_order=False)


SWEEP = [
    # B, H, L, d, lo, hi, budget
    (1, 2, 700, 128, 16, 128, 128),
    (2, 3, 1000, 64, 5, 40, 200),
    (1, 1, 513, 128, 1, 1, 37),       # unit chunks: top-N_b token attention
    (1, 2, 400, 128, 16, 64, 4096),   # budget covers everything: dense causal
    (1, 2, 600, 64, 100, 300, 150),   # chunks longer than a 128-row tile
    (1, 1, 64, 128, 64, 64, 8),       # a single chunk
]


@pytest.mark.parametrize("case", SWEEP, ids=[str(i) for i in range(len(SWEEP))])
def test_dhsa_sweep(case):
    B, H, L, d, lo, hi, budget = case
    offs = synth.chunk_offsets(L, lo, hi, seed=90 + SWEEP.index(case))
    run_case(B, H, L, d, offs, budget, seed=90 + SWEEP.index(case))
