"""DHSA prefill on the GPU against the CPU oracle: the 16K-token workload
(every row, plus the budget property on every row), shape sweeps and the
reductions (budget covering everything, unit chunks), in bf16 and fp32."""
import numpy as np
import pytest
import torch

import chunk_hierarchical_sparse_amd as hsa
import oracle
import synth
from gpu_util import MARGIN, check_exempt, check_out, dev, host, qkv, say, unpack_mask

pytestmark = pytest.mark.gpu


def run_case(B, H, L, d, offs, budget, seed, rows=None, check_order=True, block=2048, dt="bf16"):
    say(f"dhsa case B={B} H={H} L={L} d={d} chunks={len(offs) - 1} budget={budget} seed={seed} "
        f"{dt}")
    Q, K, V = qkv(B, H, H, L, d, dt, seed)
    out, mask, order = hsa.dhsa_prefill(dev(Q), dev(K), dev(V), offs, budget, return_mask=True,
                                        return_order=True)
    torch.cuda.synchronize()
    out, mask, order = host(out), host(mask), host(order)
    # every row keeps exactly min(N_b, i+1) keys, all causal
    counts = np.bitwise_count(np.ascontiguousarray(mask).view(np.uint32)).sum(-1)
    assert (counts == np.minimum(budget, np.arange(L) + 1)).all(), "kept count != min(N_b, i+1)"
    r_all = np.arange(L) if rows is None else np.asarray(rows)
    err, n_strict, n_rows = 0.0, 0, 0
    sc = None
    # the oracle runs on blocks of rows so its kept-set arrays stay small
    for k0 in range(0, len(r_all), block):
        r = r_all[k0:k0 + block]
        ref = oracle.dhsa_prefill(Q, K, V, offs, budget, rows=r, want_kept=True,
                                  want_sc=check_order and sc is None)
        if ref["sc"] is not None:
            sc = ref["sc"]
        bits = unpack_mask(mask[:, :, r], L)
        strict = ref["margin"] > MARGIN
        bad = (bits != ref["kept"]).any(-1) & strict
        assert not bad.any(), \
            f"kept sets differ above the margin at {np.argwhere(bad)[0].tolist()} (block {k0})"
        same = (bits == ref["kept"]).all(-1)
        err = max(err, check_out(out[:, :, r][same], ref["out"][same], dt, "dhsa output"))
        n_strict += int(strict.sum())
        n_rows += strict.size
    exempt = check_exempt(np.arange(n_rows) < n_strict, "dhsa kept sets")
    if check_order:
        nc = len(offs) - 1
        for b in range(B):
            for h in range(H):
                for l in range(nc):
                    row = sc[b, h, l, : l + 1]
                    exp = np.lexsort((np.arange(l + 1), -row))
                    gaps = np.abs(np.diff(row[exp]))
                    if gaps.size == 0 or gaps.min() > MARGIN:
                        assert (order[b, h, l, : l + 1] == exp).all()
                    assert (order[b, h, l, l + 1:] == -1).all()
    say(f"  ok: {len(r_all)} rows, max err {err:.3g}, exempt {exempt:.4f}")


def test_dhsa_16k_workload():
    # B=1, L=16384, H=8, d=128, chunk lengths U{16..128} (seed 5), N_b=2048:
    # every row's kept set and output, and the chunk ranking of every chunk
    L = 16384
    offs = synth.chunk_offsets(L, 16, 128, seed=5)
    run_case(1, 8, L, 128, offs, 2048, seed=5)


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


F32_SWEEP = [
    # B, H, L, d, lo, hi, budget
    (1, 2, 700, 128, 16, 128, 128),
    (2, 2, 1000, 64, 5, 40, 200),
    (1, 1, 300, 128, 1, 1, 37),       # unit chunks
    (1, 2, 400, 64, 16, 64, 4096),    # dense causal
    (1, 1, 600, 128, 100, 300, 150),  # chunks longer than a 128-row tile
    (1, 2, 2048, 128, 16, 128, 512),
]


@pytest.mark.parametrize("case", F32_SWEEP, ids=[str(i) for i in range(len(F32_SWEEP))])
def test_dhsa_f32_sweep(case):
    # fp32 inputs run the fp32 attention (relative error <= 1e-5 of max |O|)
    B, H, L, d, lo, hi, budget = case
    offs = synth.chunk_offsets(L, lo, hi, seed=120 + F32_SWEEP.index(case))
    run_case(B, H, L, d, offs, budget, seed=120 + F32_SWEEP.index(case), dt="f32")
